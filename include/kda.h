/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention chunked operator:
 * a forward pass and a backward pass that recomputes its intermediates
 * instead of saving them.
 *
 * Operator ("KDA Memory with Recompute: FLA vs cuDNN Frontend FROST",
 * section "Sources and measurement configuration"; per-chunk operations in
 * "KDA at the production shape..." section 2.1 and section 1.1):
 *   per packed sequence and head, with the state S (K x V) starting at zero,
 *     qh = scale * q / sqrt(|q|^2 + eps),  kh = k / sqrt(|k|^2 + eps)
 *     beta = sigmoid(raw_beta)
 *     g = L * sigmoid(exp(A_log[h]) * (raw_g + dt_bias[h,:]))   (L = gate_lower_bound;
 *         the default gate map, see gate_mode below)
 *     S_t = (I - beta_t kh_t kh_t^T) Diag(exp(g_t)) S_{t-1} + beta_t kh_t v_t^T
 *     o_t = S_t^T qh_t
 *   the state restarts at every sequence boundary of cu_seqlens, from zero
 *   (the measured setting of the FROST page: no initial state, no final
 *   state). The backward returns the gradients of all seven inputs (q, k, v,
 *   raw_g, raw_beta, A_log, dt_bias) of sum(o * dO). kda_fwd_ex / kda_bwd_ex
 *   add an optional initial state per sequence, its final state and their
 *   gradients, and optional forward-saved checkpoints (FROST's
 *   checkpoint_every_n_tokens, same page, "Both sides really use
 *   recomputation").
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, row-major with
 *     the innermost dimension contiguous: q, k, raw_g [T, H, K]; v, o, dO
 *     [T, H, V]; raw_beta [T, H]; A_log [H] (fp32); dt_bias [H, K] (fp32)
 *     (raw_g [T, H] and dt_bias [H] under KDA_GATE_PER_HEAD);
 *     cu_seqlens [n_seqs + 1] (int32, device copy). Pointers must be 16-byte
 *     aligned.
 *   - dtype selects the element type of q, k, v, raw_g, raw_beta, dO, o and
 *     of dq, dk, dv, draw_g, draw_beta (fp32 or bf16). dA_log and ddt_bias
 *     are always fp32.
 *   - `stream` is a hipStream_t (passed as void*; NULL is the null stream).
 *     All work is enqueued on it asynchronously; no call synchronises the
 *     host with the device. Outputs are overwritten, never accumulated.
 *   - The library allocates no device memory and keeps no state between
 *     calls: scratch comes from the caller's `workspace` (size from the
 *     *_workspace_bytes query for the same problem). Calls are reentrant and
 *     thread-safe; calls sharing a workspace must be stream-ordered.
 *   - All argument validation happens on the host before any HIP call.
 *     Return value: KDA_OK or one of the error codes below. NaN/Inf inputs
 *     propagate; they are not checked.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KDA_OK = 0,
  KDA_ERR_INVALID = 1,     /* null pointer, non-positive size, bad cu_seqlens_host */
  KDA_ERR_UNSUPPORTED = 2, /* K/V/chunk/dtype/gate combination not built */
  KDA_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace_bytes query */
  KDA_ERR_HIP = 4          /* a HIP launch failed; kda_status_string names it */
};

enum { KDA_F32 = 0, KDA_BF16 = 1 };

/* Gate maps (the pages fix the bound L and the FP32 A_log / dt_bias drive,
   not the formula), with z = raw_g + dt_bias[h,:]:
     KDA_GATE_SIGMOID_BOUND   g = L * sigmoid(exp(A_log[h]) * z)
     KDA_GATE_SOFTPLUS_CLAMP  g = max(L, -exp(A_log[h]) * softplus(z));
                              no gradient flows where the bound holds.
   Either may be OR-ed with KDA_GATE_PER_HEAD: one scalar gate per head and
   token, the Gated DeltaNet form of FLA's chunk_gdn ("KDA at the production
   shape...", sections 1.1 and 1.2; KDA adds a decay per key channel). Then
   raw_g and draw_g are [T, H], dt_bias and ddt_bias are [H], z = raw_g[t,h]
   + dt_bias[h], and every channel of the state decays by the same exp(g).
   Other values: KDA_ERR_UNSUPPORTED. */
enum { KDA_GATE_SIGMOID_BOUND = 0, KDA_GATE_SOFTPLUS_CLAMP = 1, KDA_GATE_PER_HEAD = 16 };

typedef struct {
  int32_t n_seqs;          /* N >= 1 packed sequences (empty sequences allowed) */
  int64_t total_tokens;    /* T = cu_seqlens_host[N] >= 1 */
  int32_t H, K, V;         /* heads, key dim, value dim; built: K == V in {64, 128} */
  int32_t chunk;           /* chunk length C; tiling only, the result does not
                              depend on it beyond rounding. Built: fp32 K=64:
                              16, 32, 64; fp32 K=128: 16, 32; bf16 K=64 or
                              128: 32, 64 (others: KDA_ERR_UNSUPPORTED) */
  int32_t dtype;           /* KDA_F32 or KDA_BF16 */
  int32_t gate_mode;       /* KDA_GATE_SIGMOID_BOUND or KDA_GATE_SOFTPLUS_CLAMP,
                              optionally | KDA_GATE_PER_HEAD */
  float scale;             /* multiplies qh; 1.0 for the plain o_t = S_t^T qh_t */
  float gate_lower_bound;  /* L, -5.9 <= L < 0 (e.g. -5). The kernels split
                              every decay exp(G_r - G_s) of a chunk around
                              the first row of a 16-row block, so a factor
                              reaches exp(15 |L|), which must stay finite in
                              fp32 for either dtype: L < -5.9 returns
                              KDA_ERR_UNSUPPORTED, L >= 0 or not finite
                              KDA_ERR_INVALID */
  float l2_eps;            /* eps of the Q/K L2 normalisation, e.g. 1e-6 */
  int32_t seg_chunks;      /* most chunks one streaming segment holds (forward
                              and backward); 0 = automatic (the segments fit
                              the workspace budget). A segment is either a
                              run of the chunk order (sequences one after
                              another) or, for a packed batch with several
                              long sequences, a window of the same chunk
                              positions in every sequence; the library takes
                              the plan whose scans have the shorter chain */
  const int32_t *cu_seqlens_host; /* host copy of cu_seqlens [N+1]: non-decreasing
                                     from 0 to T; used for planning only */
} kda_problem;

/* Bytes of device workspace kda_fwd / kda_bwd need for this problem
   (0 when the problem is invalid or unsupported; call kda_check_problem for
   the reason). */
size_t kda_fwd_workspace_bytes(const kda_problem *p);
size_t kda_bwd_workspace_bytes(const kda_problem *p);

/* Host-side validation only: KDA_OK, KDA_ERR_INVALID or KDA_ERR_UNSUPPORTED. */
int kda_check_problem(const kda_problem *p);

/* Prologue only (the step that normalises Q/K, applies the beta sigmoid,
   the bounded gate and its chunk-local cumulative sum), exposed for testing.
   Outputs, all fp32 and caller-owned: qh, kh [T,H,K]; beta [T,H];
   gcum [T,H,K] = cumulative sum of g from the start of each chunk (chunks
   of length p->chunk counted from each sequence start). The workspace holds
   the chunk table (kda_prologue_workspace_bytes). */
size_t kda_prologue_workspace_bytes(const kda_problem *p);
int kda_prologue(const kda_problem *p, const void *q, const void *k,
                 const void *raw_g, const void *raw_beta, const float *A_log,
                 const float *dt_bias, const int32_t *cu_seqlens, float *qh,
                 float *kh, float *beta, float *gcum, void *workspace,
                 size_t workspace_bytes, void *stream);

/* Forward ("KDA Memory with Recompute: FLA vs cuDNN Frontend FROST", section
   "Sources and measurement configuration": the inputs, the in-kernel
   normalisation, sigmoid and safe gate, packed sequences; "KDA at the
   production shape...", section 2.1, the per-chunk operations, and section
   1.1, the state loop): writes o [T,H,V] (dtype). Saves nothing for the
   backward. Errors: KDA_ERR_INVALID / KDA_ERR_UNSUPPORTED from the problem
   (as kda_check_problem) or a null pointer, KDA_ERR_WORKSPACE when
   workspace_bytes < kda_fwd_workspace_bytes, KDA_ERR_HIP on a failed
   launch; all but the last are found before any launch. */
int kda_fwd(const kda_problem *p, const void *q, const void *k, const void *v,
            const void *raw_g, const void *raw_beta, const float *A_log,
            const float *dt_bias, const int32_t *cu_seqlens, void *o,
            void *workspace, size_t workspace_bytes, void *stream);

/* Backward (the FROST page, sections "Both sides really use recomputation"
   and "Why the larger FROST state series still wins": recompute instead of
   saving, gradients written once in the input dtype; all seven inputs
   differentiated as in "Sources and measurement configuration"):
   recomputes every intermediate from the inputs, streaming over
   segments of chunks, and writes dq, dk, draw_g [T,H,K], dv [T,H,V],
   draw_beta [T,H] (dtype) and dA_log [H], ddt_bias [H,K] (fp32); draw_g
   [T,H] and ddt_bias [H] under KDA_GATE_PER_HEAD. The
   gate-parameter gradients are reduced in a fixed order (bitwise
   reproducible run to run). Errors as kda_fwd, with
   kda_bwd_workspace_bytes. */
int kda_bwd(const kda_problem *p, const void *q, const void *k, const void *v,
            const void *raw_g, const void *raw_beta, const float *A_log,
            const float *dt_bias, const int32_t *cu_seqlens, const void *dO,
            void *dq, void *dk, void *dv, void *draw_g, void *draw_beta,
            float *dA_log, float *ddt_bias, void *workspace,
            size_t workspace_bytes, void *stream);

/* State ends and forward-saved checkpoints (all fp32, device, caller-owned;
   every pointer may be NULL):
     h0    [N, H, K, V]  state each sequence starts from (NULL: zero). An
                         empty sequence passes it through to ht.
     ht    [N, H, K, V]  kda_fwd_ex: the state after each sequence's last
                         token (NULL: not written).
     dht   [N, H, K, V]  kda_bwd_ex: gradient of the loss with respect to ht
                         (NULL: zero), so the gradients are those of
                         sum(o * dO) + sum(ht * dht).
     dh0   [N, H, K, V]  kda_bwd_ex: gradient with respect to h0 (NULL: not
                         written).
     ckpt, ckpt_bytes    kda_fwd_ex writes, kda_bwd_ex reads, the states
                         that enter the backward's segments inside each
                         sequence (kda_checkpoint_bytes bytes, a layout
                         private to the library), so the backward skips the
                         pass that recomputes them. Pass the same problem to
                         both calls (set seg_chunks explicitly, or keep the
                         workspace budget unchanged between them).
                         ckpt_bytes smaller than kda_checkpoint_bytes:
                         KDA_ERR_WORKSPACE.
   The backward still recomputes w, u and h of every chunk. kda_fwd_ex reads
   h0 and writes ht and ckpt; kda_bwd_ex reads h0, dht and ckpt (which it
   leaves unchanged) and writes dh0. The same problem and h0 must be passed
   to both. */
typedef struct {
  const float *h0;
  float *ht;
  const float *dht;
  float *dh0;
  float *ckpt;
  size_t ckpt_bytes;
} kda_state_io;

/* Bytes of the checkpoint buffer of kda_state_io for this problem, and the
   backward's segment length: chunks per segment, or chunks of each sequence
   per segment for a plan by windows (0 when the problem is invalid). */
size_t kda_checkpoint_bytes(const kda_problem *p);
int32_t kda_bwd_segment_chunks(const kda_problem *p);

/* kda_fwd / kda_bwd with state ends and checkpoints (io may be NULL, which
   is kda_fwd / kda_bwd). Workspace sizes are those of kda_fwd_workspace_bytes
   / kda_bwd_workspace_bytes. */
int kda_fwd_ex(const kda_problem *p, const void *q, const void *k, const void *v,
               const void *raw_g, const void *raw_beta, const float *A_log,
               const float *dt_bias, const int32_t *cu_seqlens, void *o,
               const kda_state_io *io, void *workspace, size_t workspace_bytes,
               void *stream);
int kda_bwd_ex(const kda_problem *p, const void *q, const void *k, const void *v,
               const void *raw_g, const void *raw_beta, const float *A_log,
               const float *dt_bias, const int32_t *cu_seqlens, const void *dO,
               void *dq, void *dk, void *dv, void *draw_g, void *draw_beta,
               float *dA_log, float *ddt_bias, const kda_state_io *io,
               void *workspace, size_t workspace_bytes, void *stream);

/* GDN-2 ("KDA at the production shape...", section 1.6, and the per-chunk
   operation table of its section 2.1: akk = (b k Gamma)(k / Gamma)^T,
   w = M^-1 (b k Gamma), u = M^-1 (w v)): the gated delta rule with a
   channel-wise erase gate and a channel-wise write gate in place of beta,
     b = sigmoid(raw_b) [K],  w = sigmoid(raw_w) [V]
     S_t = (I - kh_t (b_t * kh_t)^T) Diag(exp(g_t)) S_{t-1} + kh_t (w_t * v_t)^T
     o_t = S_t^T qh_t
   with the prologue, gate maps, packing and layouts of kda_fwd / kda_bwd.
   KDA is the case b = w = beta in every channel. raw_b [T, H, K] and raw_w
   [T, H, V] are in the problem's dtype (device, caller-owned); the backward
   writes draw_b [T, H, K] and draw_w [T, H, V] in that dtype, with dq, dk,
   dv, draw_g, dA_log, ddt_bias as kda_bwd. Workspace sizes are those of
   kda_fwd_workspace_bytes / kda_bwd_workspace_bytes. Not built for GDN-2
   (KDA_ERR_UNSUPPORTED): a gate per head (KDA_GATE_PER_HEAD), and fp32 at
   K = 64 with 64-token chunks. Errors otherwise as kda_fwd / kda_bwd. */
int kda_gdn2_fwd(const kda_problem *p, const void *q, const void *k, const void *v,
                 const void *raw_g, const void *raw_b, const void *raw_w, const float *A_log,
                 const float *dt_bias, const int32_t *cu_seqlens, void *o, void *workspace,
                 size_t workspace_bytes, void *stream);
int kda_gdn2_bwd(const kda_problem *p, const void *q, const void *k, const void *v,
                 const void *raw_g, const void *raw_b, const void *raw_w, const float *A_log,
                 const float *dt_bias, const int32_t *cu_seqlens, const void *dO, void *dq,
                 void *dk, void *dv, void *draw_g, void *draw_b, void *draw_w, float *dA_log,
                 float *ddt_bias, void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc): kda_fwd
   with its workspace in a device array of KDA_NOALLOC_SCRATCH_BYTES that the
   library holds on each GPU it runs on until the process ends (the caller
   passes inputs and outputs only; layouts and result as kda_fwd, O
   bit-identical to it). The call runs the forward over the longest segment
   of chunks whose workspace fits the array; a problem whose one-chunk
   segment needs more (its state carry slots are 2 * H * K * V * 4 bytes)
   returns KDA_ERR_WORKSPACE. It allocates nothing. Calls on one GPU share
   the array: calls that overlap in time race and must be ordered by the
   caller. Returns KDA_ERR_HIP if the array's device address cannot be
   obtained. */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_fwd_noalloc(const kda_problem *p, const void *q, const void *k, const void *v,
                    const void *raw_g, const void *raw_beta, const float *A_log,
                    const float *dt_bias, const int32_t *cu_seqlens, void *o, void *stream);

/* Optional per-kernel timing, for measurement tools. Between
   kda_profile_begin() and kda_profile_end(), every kernel the calling thread
   launches through this library is bracketed by two HIP events recorded on
   its own stream. kda_profile_end() waits for those events and writes, per
   kernel kind (index = KDA_KERNEL_*), the number of launches, their summed
   duration in milliseconds and the summed number of (chunk, head) units the
   launches processed into `launches` / `total_ms` / `units` (arrays of `n`
   entries, caller-owned, each may be NULL; n >= KDA_KERNEL_COUNT
   recommended). Returns KDA_OK or KDA_ERR_HIP. Timing adds two event
   records per launch. */
enum {
  KDA_KERNEL_CHUNK_TABLE = 0,
  KDA_KERNEL_PROLOGUE = 1,
  KDA_KERNEL_CHUNK_LOCAL = 2,       /* forward operand layout (kda_fwd) */
  KDA_KERNEL_SCAN_FWD = 3,          /* the output scan (kda_fwd) */
  KDA_KERNEL_SCAN_BWD = 4,          /* reverse state-gradient scan */
  KDA_KERNEL_CHUNK_GRAD = 5,
  KDA_KERNEL_GATE_REDUCE = 6,
  KDA_KERNEL_CHUNK_LOCAL_BWD = 7,   /* backward operand layout */
  KDA_KERNEL_CHUNK_LOCAL_STATE = 8, /* state operands only (checkpoint pass) */
  KDA_KERNEL_SCAN_REC = 9,          /* forward-direction scan recording h, Vn */
  KDA_KERNEL_SCAN_STATE = 10,       /* forward-direction scan, states only */
  KDA_KERNEL_COUNT = 11
};
int kda_profile_begin(void);
int kda_profile_end(int32_t *launches, double *total_ms, int64_t *units, int n);
const char *kda_kernel_name(int kind);

/* Human-readable text for a status code, including the HIP error of the
   last failed launch on this thread for KDA_ERR_HIP. */
const char *kda_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
