"""MI355X (gfx950) Kimi Delta Attention chunked operator with a recompute backward.

The operator runs as hand-written HIP kernels behind the C ABI of
``include/kda.h`` (``_build/libkda.so``); this package is its Python binding.
"""
from .ops import (Checkpoints, KDAFunction, KdaError, Problem, kda, kda_backward, kda_forward,
                  kda_forward_noalloc, kda_prologue, gdn2_backward, gdn2_forward)

__all__ = ["Checkpoints", "KDAFunction", "KdaError", "Problem", "kda", "kda_backward", "kda_forward",
           "kda_forward_noalloc", "kda_prologue", "gdn2_backward", "gdn2_forward"]
