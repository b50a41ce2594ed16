// Inter-chunk state scans: one block per (sequence, head, value tile).
//
// Forward direction ("KDA at the production shape..." section 1.1: the state
// stays on chip for the whole chunk loop; per chunk v_new = u - w h, the
// output takes the inter part (q * e^G) h plus the intra part Aqk v_new, and
// the state is decayed channel-wise by the chunk's last cumulative gate and
// receives k^T v_new):
//   Vn = U - W h;   O = qg h + Aqk Vn;   h <- Diag(gamma) h + kg^T Vn
// Reverse direction (the state-gradient walk the backward needs):
//   dVn = Aqk^T dO + kg dh';   dh = Diag(gamma) dh' + qg^T dO - W^T dVn
// Value columns of the state evolve independently, so the value dimension is
// split into tiles of BV columns, one block each (the V-tiling of the FLA
// state kernel, section 1.1). The fp32 state lives in registers as 16x16
// MFMA accumulator tiles; an operand copy sits in LDS for the next chunk.
//
// Block-to-XCD mapping: blocks are dealt round-robin to the 8 XCDs, so the
// NVT value tiles of one (sequence, head) get block ids that are equal mod 8
// and share that XCD's L2 for the per-chunk operands they all read.
#include "kda_prologue.h"

namespace kda {

template <int NVT>
__device__ __forceinline__ bool scan_program(const Dims& d, int& n, int& h, int& vt) {
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  vt = slot % NVT;
  const int nh = (slot / NVT) * 8 + xcd;
  if (nh >= d.N * d.H) return false;
  n = nh / d.H;
  h = nh % d.H;
  return true;
}

template <typename TI, typename OpT, int D, int C, int BV, bool OUT_O, bool REC>
__global__ void __launch_bounds__(256) k_scan_fwd(Dims d, Inputs in, int seg_begin,
                                                  int seg_end, ChunkOps ops, TI* o,
                                                  SegStates st, const float* carry_in,
                                                  float* carry_out) {
  using M = Mma<OpT>;
  constexpr int K = D, V = D, NB = C / 16, NVT = V / BV, KPL = M::KPL, KS = M::KS;
  constexpr int BVT = BV / 16;
  constexpr int NHT = (K / 16) * BVT, HPW = NHT / 4;  // state tiles, per wave
  constexpr int NVN = NB * BVT;                         // Vn tiles
  constexpr int VPW = (NVN + 3) / 4;
  constexpr int LDH = K + 8, LDC = C + 8;
  static_assert(NHT % 4 == 0, "state tiles must split over 4 waves");
  __shared__ __attribute__((aligned(16))) OpT hT_s[BV * LDH];
  __shared__ __attribute__((aligned(16))) OpT VnT_s[BV * LDC];

  int n, h, vt;
  if (!scan_program<NVT>(d, n, h, vt)) return;
  const int cb = max(in.coff[n], seg_begin), ce = min(in.coff[n + 1], seg_end);
  if (cb >= ce) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int v0 = vt * BV;
  const size_t ts = static_cast<size_t>(d.H) * V;

  f32x4 hs[HPW];
  const bool fresh = (cb == in.coff[n]);
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kk = 16 * mk + 4 * g + rr, vv = v0 + 16 * nv + i;
      hs[j][rr] = fresh ? 0.f : carry_in[(static_cast<size_t>(h) * K + kk) * V + vv];
    }
  }
  auto put_state = [&]() {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
      OpT* dst = hT_s + (16 * nv + i) * LDH + 16 * mk + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f<OpT>(hs[j][rr]);
    }
  };
  put_state();
  __syncthreads();

  for (int c = cb; c < ce; ++c) {
    const size_t idx = static_cast<size_t>(c - seg_begin) * d.H + h;
    const OpT* Wn = static_cast<const OpT*>(ops.Wn) + idx * C * K;
    const OpT* kgT = static_cast<const OpT*>(ops.kgT) + idx * K * C;
    const float* gam = ops.gam + idx * K;
    if (REC) {
      // entering state h_n as [K][V]
      OpT* hd = static_cast<OpT*>(st.h) + idx * K * V;
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          hd[(16 * mk + 4 * g + rr) * V + v0 + 16 * nv + i] = from_f<OpT>(hs[j][rr]);
      }
    }
    // Vn = U - W h (and the inter part of O), tiles (row block m, value block nv)
    f32x4 accO[VPW];
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int t = w + 4 * j;
      if (t >= NVN) break;
      const int m = t / BVT, nv = t % BVT;
      f32x4 accV;
      if (REC) {
        const OpT* U = static_cast<const OpT*>(ops.U) + idx * C * V;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) accV[rr] = to_f(U[(16 * m + 4 * g + rr) * V + v0 + 16 * nv + i]);
      } else {
        const OpT* UT = static_cast<const OpT*>(ops.UT) + idx * V * C;
        const OpT* src = UT + (v0 + 16 * nv + i) * C + 16 * m + 4 * g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) accV[rr] = to_f(src[rr]);
      }
      accO[j] = zero4();
      const OpT* aw = Wn + (16 * m + i) * K + g * KPL;
      const OpT* bh = hT_s + (16 * nv + i) * LDH + g * KPL;
      if (OUT_O) {
        const OpT* aq = static_cast<const OpT*>(ops.qg) + idx * C * K + (16 * m + i) * K + g * KPL;
        for (int k0 = 0; k0 < K; k0 += KS) {
          const auto b = M::load(bh + k0);
          accV = M::mma(M::load(aw + k0), b, accV);
          accO[j] = M::mma(M::load(aq + k0), b, accO[j]);
        }
      } else {
        for (int k0 = 0; k0 < K; k0 += KS) accV = M::mma(M::load(aw + k0), M::load(bh + k0), accV);
      }
      OpT* dst = VnT_s + (16 * nv + i) * LDC + 16 * m + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f<OpT>(accV[rr]);
      if (REC) {
        OpT* vn = static_cast<OpT*>(st.Vn) + idx * C * V;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          vn[(16 * m + 4 * g + rr) * V + v0 + 16 * nv + i] = from_f<OpT>(accV[rr]);
      }
    }
    __syncthreads();
    if (OUT_O) {
      const int64_t t0 = static_cast<int64_t>(in.cu[n]) + static_cast<int64_t>(c - in.coff[n]) * C;
      const int len = static_cast<int>(min(static_cast<int64_t>(C), in.cu[n + 1] - t0));
      const OpT* Aqk = static_cast<const OpT*>(ops.Aqk) + idx * C * C;
#pragma unroll
      for (int j = 0; j < VPW; ++j) {
        const int t = w + 4 * j;
        if (t >= NVN) break;
        const int m = t / BVT, nv = t % BVT;
        accO[j] = tile_nt<OpT>(accO[j], Aqk + 16 * m * C, C, VnT_s + 16 * nv * LDC, LDC, 0,
                               kround<OpT>(16 * (m + 1)), lane);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * m + 4 * g + rr;
          if (r < len) o[(t0 + r) * ts + static_cast<size_t>(h) * V + v0 + 16 * nv + i] = from_f<TI>(accO[j][rr]);
        }
      }
    }
    // h <- Diag(gamma) h + kg^T Vn
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
      f32x4 acc;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[rr] = gam[16 * mk + 4 * g + rr] * hs[j][rr];
      hs[j] = tile_nt<OpT>(acc, kgT + 16 * mk * C, C, VnT_s + 16 * nv * LDC, LDC, 0, C, lane);
    }
    put_state();
    __syncthreads();
  }
  if (ce < in.coff[n + 1]) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        carry_out[(static_cast<size_t>(h) * K + 16 * mk + 4 * g + rr) * V + v0 + 16 * nv + i] = hs[j][rr];
    }
  }
}

template <typename TI, typename OpT, int D, int C, int BV>
__global__ void __launch_bounds__(256) k_scan_bwd(Dims d, Inputs in, const TI* dO,
                                                  int seg_begin, int seg_end, ChunkOps ops,
                                                  SegStates st, const float* carry_in,
                                                  float* carry_out) {
  using M = Mma<OpT>;
  constexpr int K = D, V = D, NB = C / 16, NVT = V / BV;
  constexpr int BVT = BV / 16;
  constexpr int NHT = (K / 16) * BVT, HPW = NHT / 4;
  constexpr int NVN = NB * BVT;
  constexpr int LDH = K + 8, LDC = C + 8;
  __shared__ __attribute__((aligned(16))) OpT dhT_s[BV * LDH];
  __shared__ __attribute__((aligned(16))) OpT dVnT_s[BV * LDC];
  __shared__ __attribute__((aligned(16))) OpT dOT_s[BV * LDC];

  int n, h, vt;
  if (!scan_program<NVT>(d, n, h, vt)) return;
  const int cb = max(in.coff[n], seg_begin), ce = min(in.coff[n + 1], seg_end);
  if (cb >= ce) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int v0 = vt * BV;
  const size_t ts = static_cast<size_t>(d.H) * V;

  f32x4 hs[HPW];  // dh' (gradient of the state leaving the current chunk)
  const bool fresh = (ce == in.coff[n + 1]);
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kk = 16 * mk + 4 * g + rr, vv = v0 + 16 * nv + i;
      hs[j][rr] = fresh ? 0.f : carry_in[(static_cast<size_t>(h) * K + kk) * V + vv];
    }
  }
  auto put_state = [&]() {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
      OpT* dst = dhT_s + (16 * nv + i) * LDH + 16 * mk + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f<OpT>(hs[j][rr]);
    }
  };
  put_state();

  for (int c = ce - 1; c >= cb; --c) {
    const size_t idx = static_cast<size_t>(c - seg_begin) * d.H + h;
    const int64_t t0 = static_cast<int64_t>(in.cu[n]) + static_cast<int64_t>(c - in.coff[n]) * C;
    const int len = static_cast<int>(min(static_cast<int64_t>(C), in.cu[n + 1] - t0));
    // dO tile, transposed into LDS ([BV][C]); padded rows are zero
    for (int e = tid; e < C * BV; e += 256) {
      const int r = e / BV, vv = e % BV;
      dOT_s[vv * LDC + r] = r < len ? from_f<OpT>(to_f(dO[(t0 + r) * ts + static_cast<size_t>(h) * V + v0 + vv]))
                                    : from_f<OpT>(0.f);
    }
    {
      OpT* hd = static_cast<OpT*>(st.dh) + idx * K * V;
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          hd[(16 * mk + 4 * g + rr) * V + v0 + 16 * nv + i] = from_f<OpT>(hs[j][rr]);
      }
    }
    __syncthreads();
    const OpT* AqkT = static_cast<const OpT*>(ops.AqkT) + idx * C * C;
    const OpT* kg = static_cast<const OpT*>(ops.kg) + idx * C * K;
    for (int t = w; t < NVN; t += 4) {
      const int m = t / BVT, nv = t % BVT;
      f32x4 acc = zero4();
      // Aqk^T[r][s] is zero for s < r: start the reduction at the block's row
      const int s_lo = (16 * m) / M::KS * M::KS;
      acc = tile_nt<OpT>(acc, AqkT + 16 * m * C, C, dOT_s + 16 * nv * LDC, LDC, s_lo, C, lane);
      acc = tile_nt<OpT>(acc, kg + 16 * m * K, K, dhT_s + 16 * nv * LDH, LDH, 0, K, lane);
      OpT* dst = dVnT_s + (16 * nv + i) * LDC + 16 * m + 4 * g;
      OpT* gd = static_cast<OpT*>(st.dVnT) + idx * V * C + (v0 + 16 * nv + i) * C + 16 * m + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        dst[rr] = from_f<OpT>(acc[rr]);
        gd[rr] = from_f<OpT>(acc[rr]);
      }
    }
    __syncthreads();
    const OpT* qgT = static_cast<const OpT*>(ops.qgT) + idx * K * C;
    const OpT* WnT = static_cast<const OpT*>(ops.WnT) + idx * K * C;
    const float* gam = ops.gam + idx * K;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
      f32x4 acc;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[rr] = gam[16 * mk + 4 * g + rr] * hs[j][rr];
      acc = tile_nt<OpT>(acc, qgT + 16 * mk * C, C, dOT_s + 16 * nv * LDC, LDC, 0, C, lane);
      hs[j] = tile_nt<OpT>(acc, WnT + 16 * mk * C, C, dVnT_s + 16 * nv * LDC, LDC, 0, C, lane);
    }
    __syncthreads();  // every wave is done reading dhT_s / dOT_s of this chunk
    put_state();
  }
  if (cb > in.coff[n]) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int t = w * HPW + j, mk = t / BVT, nv = t % BVT;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        carry_out[(static_cast<size_t>(h) * K + 16 * mk + 4 * g + rr) * V + v0 + 16 * nv + i] = hs[j][rr];
    }
  }
}

template <typename TI, int D, int C>
static constexpr int pick_bv() { return 32; }

template <typename TI, int D, int C>
static hipError_t launch_sf(const Dims& d, const Inputs& in, int seg_begin, int seg_end,
                            const ChunkOps& ops, void* o, const SegStates* st,
                            const float* carry_in, float* carry_out, hipStream_t s) {
  constexpr int BV = pick_bv<TI, D, C>(), NVT = D / BV;
  const int groups = (d.N * d.H + 7) / 8;
  const dim3 grid(groups * 8 * NVT), block(256);
  SegStates z{};
  if (o)
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, true, false>), grid, block, 0, s, d, in,
                       seg_begin, seg_end, ops, static_cast<TI*>(o), z, carry_in, carry_out);
  else if (st)
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, false, true>), grid, block, 0, s, d, in,
                       seg_begin, seg_end, ops, nullptr, *st, carry_in, carry_out);
  else
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, false, false>), grid, block, 0, s, d, in,
                       seg_begin, seg_end, ops, nullptr, z, carry_in, carry_out);
  return hipGetLastError();
}

template <typename TI, int D, int C>
static hipError_t launch_sb(const Dims& d, const Inputs& in, const void* dO, int seg_begin,
                            int seg_end, const ChunkOps& ops, const SegStates& st,
                            const float* carry_in, float* carry_out, hipStream_t s) {
  constexpr int BV = pick_bv<TI, D, C>(), NVT = D / BV;
  const int groups = (d.N * d.H + 7) / 8;
  hipLaunchKernelGGL((k_scan_bwd<TI, TI, D, C, BV>), dim3(groups * 8 * NVT), dim3(256), 0, s,
                     d, in, static_cast<const TI*>(dO), seg_begin, seg_end, ops, st, carry_in,
                     carry_out);
  return hipGetLastError();
}

#define KDA_DISPATCH(FN, ...)                                              \
  if (dtype == 0) {                                                        \
    if (D == 64 && C == 16) return FN<float, 64, 16>(__VA_ARGS__);         \
    if (D == 64 && C == 32) return FN<float, 64, 32>(__VA_ARGS__);         \
    if (D == 64 && C == 64) return FN<float, 64, 64>(__VA_ARGS__);         \
    if (D == 128 && C == 16) return FN<float, 128, 16>(__VA_ARGS__);       \
    if (D == 128 && C == 32) return FN<float, 128, 32>(__VA_ARGS__);       \
    if (D == 128 && C == 64) return FN<float, 128, 64>(__VA_ARGS__);       \
  } else {                                                                 \
    if (D == 64 && C == 32) return FN<bf16, 64, 32>(__VA_ARGS__);          \
    if (D == 64 && C == 64) return FN<bf16, 64, 64>(__VA_ARGS__);          \
    if (D == 128 && C == 32) return FN<bf16, 128, 32>(__VA_ARGS__);        \
    if (D == 128 && C == 64) return FN<bf16, 128, 64>(__VA_ARGS__);        \
  }                                                                        \
  return hipErrorInvalidValue;

hipError_t launch_scan_fwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           int seg_begin, int seg_end, const ChunkOps& ops, void* out_o,
                           const SegStates* st, const float* carry_in, float* carry_out,
                           hipStream_t s) {
  KDA_DISPATCH(launch_sf, d, in, seg_begin, seg_end, ops, out_o, st, carry_in, carry_out, s)
}

hipError_t launch_scan_bwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           const void* dO, int seg_begin, int seg_end, const ChunkOps& ops,
                           const SegStates& st, const float* carry_in, float* carry_out,
                           hipStream_t s) {
  KDA_DISPATCH(launch_sb, d, in, dO, seg_begin, seg_end, ops, st, carry_in, carry_out, s)
}

}  // namespace kda
