// kda_fwd_noalloc: the forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). Its workspace is a file-scope device array the library
// holds on each GPU it runs on until the process ends; the caller passes
// only inputs and outputs.
//
// The forward's workspace (chunk table, two state carry slots, the chunk
// operands of one segment) shrinks with the segment length, so the call
// takes the longest segment whose workspace fits the array and runs the
// ordinary forward over it: the same kernels, the same per-chunk arithmetic,
// the state crossing segments in fp32 carry slots, so O is bit-identical to
// kda_fwd's. Nothing in the array has to start at zero (every kernel writes
// what a later one reads). Calls that overlap on one GPU share the array and
// race; calls must be ordered (one stream, or synchronised streams).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"

namespace {

__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (host code must not
// use the array's name as an address), looked up once per device.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int kda_fwd_noalloc(const kda_problem* p, const void* q, const void* k,
                               const void* v, const void* raw_g, const void* raw_beta,
                               const float* A_log, const float* dt_bias,
                               const int32_t* cu_seqlens, void* o, void* stream) {
  const int st = kda_check_problem(p);
  if (st != KDA_OK) return st;
  if (!q || !k || !v || !raw_g || !raw_beta || !A_log || !dt_bias || !cu_seqlens || !o)
    return KDA_ERR_INVALID;
  // the longest segment (in chunks) whose forward workspace fits the array;
  // the workspace grows with the segment until the segment holds every chunk
  kda_problem pp = *p;
  pp.seg_chunks = 1;
  if (kda_fwd_workspace_bytes(&pp) > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
  int nc = 0;
  for (int n = 0; n < p->n_seqs; ++n)
    nc += (p->cu_seqlens_host[n + 1] - p->cu_seqlens_host[n] + p->chunk - 1) / p->chunk;
  int lo = 1, hi = nc > 1 ? nc : 1;  // lo fits
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    pp.seg_chunks = mid;
    if (kda_fwd_workspace_bytes(&pp) <= KDA_NOALLOC_SCRATCH_BYTES) lo = mid; else hi = mid - 1;
  }
  pp.seg_chunks = lo;
  void* ws = scratch_ptr();
  if (!ws) return KDA_ERR_HIP;
  return kda_fwd_ex(&pp, q, k, v, raw_g, raw_beta, A_log, dt_bias, cu_seqlens, o, nullptr, ws,
                    KDA_NOALLOC_SCRATCH_BYTES, stream);
}
