// Prologue of the KDA operator for one chunk of one head, shared by the
// chunk-local, gradient and standalone prologue kernels.
//
// Follows the input description of "KDA Memory with Recompute: FLA vs cuDNN
// Frontend FROST" (section "Sources and measurement configuration"): Q/K L2
// normalisation inside the operator, beta = sigmoid(raw beta), a gate bounded
// below by L and driven by FP32 A_log / dt_bias. The pages do not print the
// gate formula; two maps are built (gate_mode):
//   0: g = L * sigmoid(exp(A_log[h]) * (raw_g + dt_bias[h,:]))
//      (a smooth map onto (L, 0), the default)
//   1: g = max(L, -exp(A_log[h]) * softplus(raw_g + dt_bias[h,:]))
//      (the softplus decay clamped at the bound)
// With gate_head set there is one gate per head and token (raw_g [T][H],
// dt_bias [H]): the scalar-gate Gated DeltaNet form ("KDA at the production
// shape...", sections 1.1 and 1.2), computed as K equal channels. The
// chunk-local cumulative sum of g is taken in fp32, as the FLA forward keeps
// its gate cumulative sum (FROST page, "Where FLA's memory goes").
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Type of the cumulative gate G. For fp32 problems it is fp64: within a
// 64-row chunk |G| reaches ~160 at the bound, where one fp32 ulp (1.5e-5)
// would already exceed the fp32 tolerance once it becomes the relative error
// of every exp(G_r - G_s). bf16 problems keep it in fp32.
template <typename OpT>
struct GateT {
  typedef float T;
};
template <>
struct GateT<float> {
  typedef double T;
};

// Units of the cumulative gate in the chunk-local and gradient kernels. bf16
// problems keep it in base-2 units (G log2 e, summed from g log2 e), so each
// exponential of a gate difference is a single v_exp_f32; fp32 problems keep
// natural units in fp64 (see GateT).
template <typename OpT>
struct GateUnits {
  static constexpr float scale = 1.4426950408889634f;
  static __device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x); }
};
template <>
struct GateUnits<float> {
  static constexpr double scale = 1.0;
  static __device__ __forceinline__ float ex(double x) { return static_cast<float>(exp(x)); }
};

template <typename T>
__device__ __forceinline__ T sigmoid_t(T x);
template <>
__device__ __forceinline__ float sigmoid_t<float>(float x) { return sigmoidf(x); }
template <>
__device__ __forceinline__ double sigmoid_t<double>(double x) { return 1.0 / (1.0 + exp(-x)); }

// softplus(x) = log(1 + e^x); past the cut-off e^-x is below half an ulp of x.
template <typename T>
__device__ __forceinline__ T softplus_t(T x);
template <>
__device__ __forceinline__ float softplus_t<float>(float x) { return x > 20.f ? x : log1pf(expf(x)); }
template <>
__device__ __forceinline__ double softplus_t<double>(double x) { return x > 40.0 ? x : log1p(exp(x)); }

// The gate map g(x + b) for gate_mode 0 or 1 (ea = exp(A_log[h]), xb = raw_g +
// dt_bias, lb = L), in the precision of T.
template <typename T>
__device__ __forceinline__ T gate_map(int mode, T ea, T xb, T lb) {
  if (mode == 0) return lb * sigmoid_t<T>(ea * xb);
  const T c = -ea * softplus_t<T>(xb);
  return c > lb ? c : lb;
}

// Location of chunk c (global index) of a packed batch, from the chunk
// table (one dependent load).
struct ChunkLoc {
  int64_t t0;  // first token
  int len;     // valid rows (1..C)
};

template <int C>
__device__ __forceinline__ ChunkLoc locate(const Inputs& in, [[maybe_unused]] int N, int c) {
  const int2 e = in.cloc[c];
  return ChunkLoc{static_cast<int64_t>(e.x), e.y};
}

// Row part of the prologue. Each row is read with 16-byte vector loads by
// LPR = D / (16 / sizeof(TI)) consecutive lanes, so one wave instruction
// covers 64 / LPR rows; wave w takes row groups w, w + NW, ... and issues the
// loads of all its rows before any arithmetic.
template <typename TI>
struct Vec16;
template <>
struct Vec16<bf16> {
  typedef bf16x8 T;
};
template <>
struct Vec16<float> {
  typedef f32x4 T;
};

// The prologue's row loads for one chunk, in the row layout above: lane
// (w, lane) of iteration it holds row (w + NW * it) * RPI + lane / LPR,
// channels (lane % LPR) * VE .. + VE.
template <typename TI, int D, int C, int NW>
struct ProRows {
  typedef typename Vec16<TI>::T VT;
  static constexpr int VE = 16 / sizeof(TI);  // elements per vector load
  static constexpr int LPR = D / VE;          // lanes per row
  static constexpr int RPI = 64 / LPR;        // rows per wave instruction
  static constexpr int NIT = (C + NW * RPI - 1) / (NW * RPI);
  static_assert(D % VE == 0 && 64 % LPR == 0, "prologue row layout");
  VT qv[NIT], kv[NIT], xv[NIT];
  uint32_t bv[NIT];
  uint32_t xs[NIT];  // raw gate bits of a per-head gate (xv unused then)
  float alog, db[VE];
};

// Issue the prologue's loads. Rows past the chunk's end load the last valid
// row instead (always in bounds, no branch) and are masked at use: a load
// under a branch, or one converted on arrival, would make the wave wait for
// it right away.
template <typename TI, int D, int C, int NW>
__device__ __forceinline__ void prologue_load(const Dims& d, const Inputs& in, int h,
                                              const ChunkLoc& L, ProRows<TI, D, C, NW>& p) {
  using P = ProRows<TI, D, C, NW>;
  typedef typename P::VT VT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rsub = lane / P::LPR, c0 = (lane % P::LPR) * P::VE;
  const size_t ts = static_cast<size_t>(d.H) * D;
  const size_t hoff = static_cast<size_t>(h) * D + c0;
  const TI* q = static_cast<const TI*>(in.q) + L.t0 * ts + hoff;
  const TI* k = static_cast<const TI*>(in.k) + L.t0 * ts + hoff;
  const TI* x = static_cast<const TI*>(in.g) + L.t0 * ts + hoff;
  const TI* rb = static_cast<const TI*>(in.beta) + L.t0 * d.H + h;
  // the per-head parameters first: the arithmetic needs them with the first row
  p.alog = in.A_log[h];
  if (d.gate_head) {
    const float b = in.dt_bias[h];
#pragma unroll
    for (int j = 0; j < P::VE; ++j) p.db[j] = b;
  } else {
#pragma unroll
    for (int j = 0; j < P::VE; j += 4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(in.dt_bias + static_cast<size_t>(h) * D + c0 + j);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) p.db[j + jj] = b4[jj];
    }
  }
  const TI* xh = static_cast<const TI*>(in.g) + L.t0 * d.H + h;  // per-head gate
#pragma unroll
  for (int it = 0; it < P::NIT; ++it) {
    const int r = (w + NW * it) * P::RPI + rsub;
    const int rc = r < L.len ? r : L.len - 1;
    p.qv[it] = *reinterpret_cast<const VT*>(q + rc * ts);
    p.kv[it] = *reinterpret_cast<const VT*>(k + rc * ts);
    if (d.gate_head)
      p.xs[it] = load_bits<TI>(xh + static_cast<size_t>(rc) * d.H);
    else
      p.xv[it] = *reinterpret_cast<const VT*>(x + rc * ts);
    p.bv[it] = d.gdn2 ? 0u : load_bits<TI>(rb + static_cast<size_t>(rc) * d.H);
  }
}

// 1/sqrt(x) on v_rsq_f32 (about 1 ulp) instead of a correctly rounded sqrt
// and divide (some 40 instructions); a subnormal x is scaled by 2^64 first,
// which the hardware instruction does not take.
__device__ __forceinline__ float rsqrt_scaled(float x) {
  const bool tiny = x < 1.17549435e-38f;
  return __builtin_amdgcn_rsqf(tiny ? x * 0x1p64f : x) * (tiny ? 0x1p32f : 1.f);
}

// The gate values of one row vector (VE channels) times gscale, in the
// precision of GV; rows past the chunk's end (valid false) get 0. MODE is the
// gate map (hoisted out of the row loop). For fp32 gates the smooth map is
// evaluated as lb * gscale / (1 + 2^(c x + c b)) with c = -e^A log2 e, one
// fused multiply-add, v_exp_f32 and v_rcp_f32 per channel.
template <int MODE, typename TI, int VE, typename GV>
__device__ __forceinline__ void gate_vec(const Dims& d, GV ea, const float* db,
                                         const typename Vec16<TI>::T& xv, bool valid, GV gscale,
                                         GV* out) {
  if constexpr (MODE == 0 && sizeof(GV) == 4) {
    const float c = -static_cast<float>(ea) * 1.4426950408889634f;
    const float amp = d.lb * static_cast<float>(gscale);
#pragma unroll
    for (int j = 0; j < VE; ++j) {
      const float t = __builtin_amdgcn_exp2f(fmaf(c, to_f(xv[j]), c * db[j]));
      const float gv = amp * __builtin_amdgcn_rcpf(1.0f + t);
      out[j] = valid ? gv : 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < VE; ++j) {
      const GV xb = static_cast<GV>(to_f(xv[j])) + static_cast<GV>(db[j]);
      const GV gv = gate_map<GV>(MODE, ea, xb, static_cast<GV>(d.lb)) * gscale;
      out[j] = valid ? gv : GV(0);
    }
  }
}

// The gate value of a per-head gate (raw bits xs of one row, bias b), times
// gscale, repeated over the VE channels; 0 for rows past the chunk's end.
template <int MODE, typename TI, int VE, typename GV>
__device__ __forceinline__ void gate_head(const Dims& d, GV ea, float b, uint32_t xs, bool valid,
                                          GV gscale, GV* out) {
  const GV xb = static_cast<GV>(bits_to_f<TI>(xs)) + static_cast<GV>(b);
  const GV gv = valid ? gate_map<GV>(MODE, ea, xb, static_cast<GV>(d.lb)) * gscale : GV(0);
#pragma unroll
  for (int j = 0; j < VE; ++j) out[j] = gv;
}

// The prologue's arithmetic on loaded rows: for each row the per-row scalars
// and the gate value of each channel into G(r, k) (a functor returning a
// reference into LDS). Rows r >= len are padding: q = k = 0, beta = 0, g = 0,
// so they contribute nothing anywhere.
//   rq[r]  = 1/sqrt(|q|^2 + eps)  (so qbar = q * rq)
//   rqs[r] = scale * rq           (so qh = q * rqs)
//   rk[r]  = 1/sqrt(|k|^2 + eps)  (kh = k * rk)
//   be[r]  = sigmoid(raw_beta)
// gscale multiplies every gate value written to G (1 for natural units).
template <int MODE, bool PH, typename TI, int D, int C, int NW, class GRef>
__device__ __forceinline__ void prologue_compute_m(const Dims& d, const ChunkLoc& L,
                                                   const ProRows<TI, D, C, NW>& p, float* rq,
                                                   float* rqs, float* rk, float* be, GRef G,
                                                   typename GateT<TI>::T gscale) {
  using P = ProRows<TI, D, C, NW>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane % P::LPR, rsub = lane / P::LPR, c0 = sub * P::VE;
  typedef typename GateT<TI>::T GV;
  const GV ea = exp(static_cast<GV>(p.alog));
#pragma unroll
  for (int it = 0; it < P::NIT; ++it) {
    const int r = (w + NW * it) * P::RPI + rsub;
    const bool valid = r < L.len;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int j = 0; j < P::VE; ++j) {
      const float a = to_f(p.qv[it][j]), b = to_f(p.kv[it][j]);
      sq += a * a;
      sk += b * b;
    }
    sq = group_sum<P::LPR>(sq);
    sk = group_sum<P::LPR>(sk);
    if (r < C) {
      GV gv[P::VE];
      if constexpr (PH)
        gate_head<MODE, TI, P::VE, GV>(d, ea, p.db[0], p.xs[it], valid, gscale, gv);
      else
        gate_vec<MODE, TI, P::VE, GV>(d, ea, p.db, p.xv[it], valid, gscale, gv);
#pragma unroll
      for (int j = 0; j < P::VE; ++j) G(r, c0 + j) = gv[j];
      if (sub == 0) {
        const float a = valid ? rsqrt_scaled(sq + d.eps) : 0.f;
        const float b = valid ? rsqrt_scaled(sk + d.eps) : 0.f;
        rq[r] = a;
        rqs[r] = d.scale * a;
        rk[r] = b;
        // GDN-2 has no scalar beta: its gates act per channel (1 keeps the
        // beta-scaled terms of the kernels as they are)
        be[r] = valid ? (d.gdn2 ? 1.f : sigmoidf(bits_to_f<TI>(p.bv[it]))) : 0.f;
      }
    }
  }
}

template <typename TI, int D, int C, int NW, class GRef>
__device__ __forceinline__ void prologue_compute(const Dims& d, const ChunkLoc& L,
                                                 const ProRows<TI, D, C, NW>& p, float* rq,
                                                 float* rqs, float* rk, float* be, GRef G,
                                                 typename GateT<TI>::T gscale = 1) {
  if (d.gate_head) {
    if (d.gate_mode == 0)
      prologue_compute_m<0, true, TI, D, C, NW>(d, L, p, rq, rqs, rk, be, G, gscale);
    else
      prologue_compute_m<1, true, TI, D, C, NW>(d, L, p, rq, rqs, rk, be, G, gscale);
  } else {
    if (d.gate_mode == 0)
      prologue_compute_m<0, false, TI, D, C, NW>(d, L, p, rq, rqs, rk, be, G, gscale);
    else
      prologue_compute_m<1, false, TI, D, C, NW>(d, L, p, rq, rqs, rk, be, G, gscale);
  }
}

// Both parts: loads, then arithmetic.
template <typename TI, int D, int C, int NW, class GRef>
__device__ __forceinline__ void prologue_rows(const Dims& d, const Inputs& in, int h,
                                              const ChunkLoc& L, float* rq, float* rqs,
                                              float* rk, float* be, GRef G,
                                              typename GateT<TI>::T gscale = 1) {
  ProRows<TI, D, C, NW> p;
  prologue_load<TI, D, C, NW>(d, in, h, L, p);
  prologue_compute<TI, D, C, NW>(d, L, p, rq, rqs, rk, be, G, gscale);
}

// In-place inclusive cumulative sum over the C rows of every channel k of
// G(r, k), by all threads of the block (fixed order, deterministic).
// part_tot: LDS scratch of at least (blockDim / D) * D values of G's type.
struct NoMid {
  __device__ __forceinline__ void operator()() const {}
};
// mid() runs between the sum's two barriers (work that may wait for loads
// and must be ordered before the code after the sum).
template <int D, int C, int NT, class GRef, typename PT, class Mid = NoMid>
__device__ __forceinline__ void cumsum_rows(GRef G, PT* part_tot, Mid mid = Mid()) {
  constexpr int parts = NT / D;
  constexpr int rp = C / parts;
  static_assert(NT % D == 0 && C % parts == 0, "cumsum layout");
  const int tid = threadIdx.x;
  const int col = tid % D, part = tid / D;
  // all reads of the thread's run first (independent LDS loads in flight
  // together), then the running sum in registers
  PT v[rp];
#pragma unroll
  for (int i = 0; i < rp; ++i) v[i] = G(part * rp + i, col);
  PT run = 0;
#pragma unroll
  for (int i = 0; i < rp; ++i) {
    run += v[i];
    v[i] = run;
  }
  part_tot[part * D + col] = run;
  __syncthreads();
  mid();
  PT off = 0;
  for (int p = 0; p < part; ++p) off += part_tot[p * D + col];
#pragma unroll
  for (int i = 0; i < rp; ++i) G(part * rp + i, col) = v[i] + off;
  __syncthreads();
}

// Load KPL consecutive elements of TI as floats (KPL = 8 or 1).
template <typename TI, int KPL>
__device__ __forceinline__ void load_row_f(const TI* p, float* out) {
  if constexpr (KPL == 8 && sizeof(TI) == 2) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = static_cast<float>(v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < KPL; ++j) out[j] = to_f(p[j]);
  }
}

}  // namespace kda
