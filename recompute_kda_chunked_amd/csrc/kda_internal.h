// Internal interface between the host orchestration (kda_host.cpp) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Problem-wide constants every kernel needs.
struct Dims {
  int N, H;
  float scale, lb, eps;
  int gate_mode;  // 0: L * sigmoid(e^A (x + b)); 1: max(L, -e^A softplus(x + b))
  int gate_head;  // 1: one gate per head and token (raw_g [T][H], dt_bias [H],
                  // draw_g [T][H], ddt_bias [H]); 0: one per channel
  int gdn2;       // 1: GDN-2, a per-channel erase gate b = sigmoid(raw_b) [T][H][K]
                  // and write gate w = sigmoid(raw_w) [T][H][V] replace beta
                  // (Inputs::bk, Inputs::wv; Inputs::beta unused)
};

// Raw operator inputs (device pointers, dtype per the problem).
struct Inputs {
  const void *q, *k, *v, *g, *beta;
  const float *A_log, *dt_bias;
  const int32_t *cu;    // cu_seqlens [N+1]
  const int32_t *coff;  // chunk offsets [N+1]: sequence n has coff[n+1] - coff[n] chunks
  const int2 *cloc;     // per chunk in the plan's chunk order: {first token, valid rows} [NC]
  const void *bk = nullptr, *wv = nullptr;  // GDN-2: raw_b [T][H][K], raw_w [T][H][V]
};

// One segment of a plan: the chunks at indices [c0, c1) of the plan's chunk
// order (the order of cloc, of the chunk operands and of the gate-parameter
// partials). A sequence's chunks in a segment are consecutive chunks of the
// sequence and contiguous in that order; sequences [n0, n1) may have some.
//   pst == nullptr (plan in sequence order: the chunk order lists the
//     sequences one after another): sequence n has chunks
//     [max(coff[n], c0), min(coff[n+1], c1)).
//   pst != nullptr (plan by windows: the segment holds chunks pos0 ..
//     pos0 + window - 1 of every sequence): sequence n has chunks
//     [pst[n], pst[n+1]), its first at position pos0 of the sequence.
struct Seg {
  int c0, c1, n0, n1;
  const int32_t* pst;
  int pos0;
};

// Slots of the states that cross segment boundaries, each [H][K][V] fp32:
//   ckt != nullptr (checkpoint layout): the state entering chunk p of
//     sequence n (p counted from the sequence start) is slot
//     ckt[n].y + (ckt[n].x + p) / every;
//   otherwise sequence n uses slot xr[n] of each carry buffer (slot 0 when
//     xr is null).
// Slots are clamped to [0, nslots), the slots the buffers hold.
struct CarryMap {
  const int2* ckt;
  int every;
  const int32_t* xr;
  int nslots;
};

// Per-(chunk, head) operands produced by the chunk-local kernel for one
// segment; element (lc, h) of each array is at index lc * H + h where lc is
// the chunk index relative to the segment start. Operand element type is
// bf16 for bf16 problems and fp32 for fp32 problems. Wn, U, qg, kgT, Aqk,
// Aqk_lo, AqkT, kg, qgT, WnT and TT are stored fragment-major (FragMajor in
// kda_device.h; qg and kg in its row-parity slot order); PT is row-major and
// Uf in 16x16 blocks (see Uf). The forward layout keeps U in fp32
// and Aqk as a bf16 pair (Aqk + Aqk_lo) because the output takes them
// directly: rounding either to bf16 would add a bf16 rounding's worth of
// error to O.
struct ChunkOps {
  void *Wn;    // [C][K]  -W  (W = T (beta * kh * e^G))
  void *U;     // [C][V]  U = T (beta * v)                (backward only)
  float *Uf;   // [C][V]  U in fp32, 16x16 blocks (forward only): element (r, c) at
               //   ((r/16) (V/16) + c/16) 256 + (r%16) 16 + c%16, so a wave's
               //   16 rows x 4 columns per lane are one contiguous 1 KB run
  void *qg;    // [C][K]  qh * e^G                       (forward only)
  void *kgT;   // [K][C]  (kh * e^{G_c - G})^T
  void *Aqk;   // [C][C]  gated q.k, lower incl. diagonal (forward only)
  void *Aqk_lo;  // [C][C] Aqk - Aqk rounded to bf16 (forward, bf16 only)
  float *gam;  // [K]     e^{G_c}
  // backward extras
  void *AqkT;  // [C][C]
  void *kg;    // [C][K]
  void *qgT;   // [K][C]
  void *WnT;   // [K][C]
  void *TT;    // [C][C]  T^T
  void *PT;    // [C][C]  P^T, P = gated k.k without beta (strictly lower)
};

// States recorded by the backward scans for one segment, element (lc, h) at
// lc * H + h: entering state h_n and leaving-state gradient dh'_n as [K][V],
// Vn as [C][V], dVn^T as [V][C] (operand element type, all fragment-major).
struct SegStates {
  void *h, *dh, *Vn, *dVnT;
};

// Per-sequence state ends of a scan, all fp32 [N][H][K][V] (sequence n's
// slice at n * H * K * V) or null:
//   forward scan: init = initial states (null: zero), fin = final states
//     out (null: not written), ck = states entering the chunks ck_map puts
//     in a checkpoint slot (position p > 0 of sequence n with
//     (ckt[n].x + p) % every == 0), each into its slot (null: none);
//   reverse scan: init = final-state gradients (null: zero), fin = initial-
//     state gradients out (null: not written); ck unused.
struct ScanStates {
  const float* init;
  float* fin;
  float* ck;
  CarryMap ck_map;
};

// Launchers (defined next to their kernels). Each returns hipSuccess or the
// launch error. `dtype` is 0 (fp32) or 1 (bf16); D = K = V; C = chunk.
// The chunk table: coff, cloc in the plan's chunk order, and per sequence
// ckt (checkpoint layout of the plan `ck_every`, `ck_win`: by windows when
// nonzero, else in sequence order) and, for a plan by windows of `win`
// chunks over NS segments, xr (carry slot: rank among the sequences longer
// than one window) and pst (segment sg's sequence starts, [NS][N+1]).
struct TableArgs {
  const int32_t* cu;
  int N, C, NC;
  int win, NS;
  int ck_every, ck_win;
  int32_t* coff;
  int2* cloc;
  int2* ckt;
  int32_t* xr;
  int32_t* pst;
};
hipError_t launch_chunk_table(const TableArgs& a, hipStream_t s);
hipError_t launch_prologue(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           int64_t n_chunks, float* qh, float* kh, float* beta, float* gcum,
                           hipStream_t s);
// mode: KL_FWD (forward operand layout, for the output scan), KL_BWD
// (backward layouts), KL_STATE (forward layout, state operands only).
enum { KL_FWD = 0, KL_BWD = 1, KL_STATE = 2 };
hipError_t launch_chunk_local(int dtype, int D, int C, int mode, const Dims& d,
                              const Inputs& in, int seg_begin, int seg_chunks,
                              const ChunkOps& ops, hipStream_t s);
// Forward-direction scan over one segment (`active` of its sequences have
// chunks in it). out_o != nullptr writes O; st != nullptr records h and Vn
// for the backward. carry_in/out: the states of the sequences that cross
// the segment's first / last boundary, in slots per `cm`.
hipError_t launch_scan_fwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           const Seg& sg, int active, const ChunkOps& ops, void* out_o,
                           const SegStates* st, const float* carry_in, float* carry_out,
                           const CarryMap& cm, const ScanStates& ss, hipStream_t s);
// Reverse (state-gradient) scan over one segment; records dh' and dVn^T.
// carry_in: gradients entering from the following segment; carry_out:
// those leaving to the preceding one.
hipError_t launch_scan_bwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           const void* dO, const Seg& sg, int active, const ChunkOps& ops,
                           const SegStates& st, const float* carry_in, float* carry_out,
                           const CarryMap& cm, const ScanStates& ss, hipStream_t s);
// dst[n] = src[n] (or zero when src is null) for every empty sequence n;
// KV = K * V floats per (sequence, head).
hipError_t launch_state_passthrough(const int32_t* cu, int N, int H, int KV, const float* src,
                                    float* dst, hipStream_t s);
// Token-parallel gradients for one segment; writes dq, dk, dv, draw_g,
// draw_beta (GDN-2: draw_b [T][H][K] into dbeta, draw_w [T][H][V] into dw)
// for its tokens and gate-parameter partials [chunk][H][K+1].
hipError_t launch_chunk_grad(int dtype, int D, int C, const Dims& d, const Inputs& in,
                             const void* dO, int seg_begin, int seg_chunks,
                             const ChunkOps& ops, const SegStates& st, void* dq, void* dk,
                             void* dv, void* dg, void* dbeta, void* dw, double* partials,
                             hipStream_t s);
// gate_head: ddt_bias[h] is the sum over all K partial columns of head h.
hipError_t launch_gate_reduce(int D, int H, int n_chunks, int gate_head,
                              const double* partials, float* dA_log, float* ddt_bias,
                              hipStream_t s);

}  // namespace kda
