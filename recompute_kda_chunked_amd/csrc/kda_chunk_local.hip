// Chunk-local kernel: one block per (chunk, head) of a segment.
//
// Builds the per-chunk operands of the chunked gated delta rule, following
// the per-chunk operation table of "KDA at the production shape..." section
// 2.1 (aqk, akk, the triangular inverse, w, u) and the state-loop pieces of
// section 1.1 (the state is decayed by the last cumulative gate of the chunk):
//   G    = cumulative sum of g within the chunk (fp32)
//   P    [r,s] = sum_k kh_rk kh_sk exp(G_rk - G_sk)        (s < r)
//   Akk  [r,s] = beta_r P[r,s]
//   Aqk  [r,s] = sum_k qh_rk kh_sk exp(G_rk - G_sk)        (s <= r)
//   T    = (I + Akk)^-1   (unit lower triangular, fp32)
//   W    = T (beta * kh * e^G),  U = T (beta * v)
//   qg   = qh * e^G,  kg = kh * e^{G_c - G},  gamma = e^{G_c}
// The u row of that table is garbled in the extracted text; the reading here
// is U = T (beta * v), the only one consistent with the token recurrence.
//
// Overflow safety: exp(G_r - G_s) is never split as exp(G_r) * exp(-G_s) over
// a whole chunk (the cumulative gate of a 64-row chunk reaches -320 at the -5
// bound, past the fp32 exponent range; the pages note the same limit for
// 17+ steps). Rows are grouped in 16-row blocks; for a block pair (I, J <= I)
// the factor is taken around the first row b of block I:
//   exp(G_r - G_s) = exp(G_r - G_b) * exp(G_b - G_s)
// with G_r - G_b in [-75, 0] for r in block I, and G_b - G_s <= 0 for s in an
// earlier block, or in [0, 75] for s in block I. Every factor is finite.
//
// Operands for the MFMA products are generated on the fly from the inputs and
// the fp32 cumulative gate held in LDS; nothing but the outputs below is
// written to memory.
#include "kda_prologue.h"

namespace kda {

template <typename TI, typename OpT, int D, int C, bool BWD>
__global__ void __launch_bounds__(256) k_chunk_local(Dims d, Inputs in, int seg_begin,
                                                     ChunkOps ops) {
  using M = Mma<OpT>;
  constexpr int K = D, V = D, NB = C / 16, KPL = M::KPL, KS = M::KS;
  constexpr int LDG = D + 4;   // Gs row stride (floats)
  constexpr int LDM = C + 4;   // fp32 C x C stride
  constexpr int LDT = C + 8;   // operand C x C stride (16-byte aligned rows)
  constexpr int SZ_M = C * LDM * 4, SZ_TB = C * LDT * (int)sizeof(OpT);
  constexpr int SZ_R = SZ_M > SZ_TB ? SZ_M : SZ_TB;
  __shared__ float Gs[C * LDG];
  __shared__ __attribute__((aligned(16))) unsigned char regM[SZ_R];  // P, then Tb
  __shared__ float As[C * LDM];                                         // Aqk, then T
  __shared__ float Sx[16 * C];
  __shared__ float rq[C], rqs[C], rk[C], be[C];
  __shared__ float ptot[4 * D];
  float* Ms = reinterpret_cast<float*>(regM);
  OpT* Tb = reinterpret_cast<OpT*>(regM);
  float* Ts = As;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int lc = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const ChunkLoc L = locate<C>(in, d.N, seg_begin + lc);
  const size_t idx = static_cast<size_t>(lc) * d.H + h;
  const size_t ts = static_cast<size_t>(d.H) * D;
  const TI* qr = static_cast<const TI*>(in.q) + L.t0 * ts + static_cast<size_t>(h) * D;
  const TI* kr = static_cast<const TI*>(in.k) + L.t0 * ts + static_cast<size_t>(h) * D;
  const TI* vr = static_cast<const TI*>(in.v) + L.t0 * ts + static_cast<size_t>(h) * D;

  for (int e = tid; e < C * LDM; e += 256) {
    Ms[e] = 0.f;
    As[e] = 0.f;
  }
  auto G = [&](int r, int kk) -> float& { return Gs[r * LDG + kk]; };
  prologue_rows<TI, D, C, 4>(d, in, h, L, rq, rqs, rk, be, G);
  __syncthreads();
  cumsum_rows<D, C, 256>(G, ptot);

  // ---- gated products P (= Akk / beta) and Aqk, 16x16 block pairs
  for (int p = w; p < NB * (NB + 1) / 2; p += 4) {
    int I = 0, J = p;
    while (J > I) { J -= I + 1; ++I; }
    const int ra = 16 * I + i, rb = 16 * J + i;
    const bool va = ra < L.len, vb = rb < L.len;
    f32x4 accP = zero4(), accQ = zero4();
    for (int k0 = 0; k0 < K; k0 += KS) {
      const int kk = k0 + g * KPL;
      float qa[KPL], ka[KPL], kb[KPL], ea[KPL], eb[KPL];
      if (va) {
        load_row_f<TI, KPL>(qr + ra * ts + kk, qa);
        load_row_f<TI, KPL>(kr + ra * ts + kk, ka);
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) qa[j] = ka[j] = 0.f;
      }
      if (vb) load_row_f<TI, KPL>(kr + rb * ts + kk, kb);
      else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) kb[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const float gb = Gs[16 * I * LDG + kk + j];
        ea[j] = kexp<OpT>(Gs[ra * LDG + kk + j] - gb);
        eb[j] = kexp<OpT>(gb - Gs[rb * LDG + kk + j]);
      }
      const float sq = rqs[ra], sk = rk[ra], sb = rk[rb];
      const auto fq = M::make([&](int j) { return qa[j] * sq * ea[j]; });
      const auto fk = M::make([&](int j) { return ka[j] * sk * ea[j]; });
      const auto fb = M::make([&](int j) { return kb[j] * sb * eb[j]; });
      accP = M::mma(fk, fb, accP);
      accQ = M::mma(fq, fb, accQ);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 16 * I + 4 * g + rr, s = 16 * J + i;
      Ms[r * LDM + s] = (s < r) ? accP[rr] : 0.f;
      As[r * LDM + s] = (s <= r) ? accQ[rr] : 0.f;
    }
  }
  __syncthreads();

  // ---- elementwise outputs and the C x C matrices that leave before the inverse
  {
    OpT* aq = static_cast<OpT*>(BWD ? ops.AqkT : ops.Aqk) + idx * C * C;
    for (int e = tid; e < C * C; e += 256) {
      const int a = e / C, b = e % C;
      aq[e] = from_f<OpT>(BWD ? As[b * LDM + a] : As[a * LDM + b]);
    }
    if (BWD) {
      OpT* P = static_cast<OpT*>(ops.P) + idx * C * C;
      for (int e = tid; e < C * C; e += 256) P[e] = from_f<OpT>(Ms[(e / C) * LDM + e % C]);
    }
    float* gam = ops.gam + idx * K;
    for (int kk = tid; kk < K; kk += 256) gam[kk] = kexp<OpT>(Gs[(C - 1) * LDG + kk]);
    // Element-wise outputs. All global loads of a loop are issued before its
    // stores (the output and input pointers may alias as far as the compiler
    // knows, which would otherwise serialise every load behind a store).
    constexpr int PER = C * K / 256;
    // row-major [C][K] outputs: qg (forward) or kg (backward)
    {
      float src[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j, r = e / K, kk = e % K;
        src[j] = r < L.len ? to_f((BWD ? kr : qr)[r * ts + kk]) : 0.f;
      }
      OpT* rowm = static_cast<OpT*>(BWD ? ops.kg : ops.qg) + idx * C * K;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j, r = e / K, kk = e % K;
        const float gr = Gs[r * LDG + kk];
        const float val = BWD ? src[j] * rk[r] * kexp<OpT>(Gs[(C - 1) * LDG + kk] - gr)
                              : src[j] * rqs[r] * kexp<OpT>(gr);
        rowm[e] = from_f<OpT>(val);
      }
    }
    // transposed [K][C] outputs: kgT always, qgT for the backward
    {
      float ks[PER], qs[BWD ? PER : 1];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j, kk = e / C, r = e % C;
        ks[j] = r < L.len ? to_f(kr[r * ts + kk]) : 0.f;
        if (BWD) qs[j] = r < L.len ? to_f(qr[r * ts + kk]) : 0.f;
      }
      OpT* kgT = static_cast<OpT*>(ops.kgT) + idx * K * C;
      OpT* qgT = BWD ? static_cast<OpT*>(ops.qgT) + idx * K * C : nullptr;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j, kk = e / C, r = e % C;
        const float gr = Gs[r * LDG + kk];
        kgT[e] = from_f<OpT>(ks[j] * rk[r] * kexp<OpT>(Gs[(C - 1) * LDG + kk] - gr));
        if (BWD) qgT[e] = from_f<OpT>(qs[j] * rqs[r] * kexp<OpT>(gr));
      }
    }
  }
  __syncthreads();

  // ---- T = (I + Akk)^-1: diagonal 16x16 blocks by forward substitution
  for (int e = tid; e < C * LDM; e += 256) Ts[e] = 0.f;
  __syncthreads();
  if (w < NB && lane < 16) {
    const int I = w, j = lane;
    float tcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int R = 16 * I + r;
      float t = (r == j) ? 1.f : 0.f;
      const float bR = be[R];
#pragma unroll
      for (int s = 0; s < r; ++s) t -= bR * Ms[R * LDM + 16 * I + s] * tcol[s];
      tcol[r] = t;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[(16 * I + r) * LDM + 16 * I + j] = tcol[r];
  }
  __syncthreads();
  // Off-diagonal blocks on fp32 MFMA (v_mfma_f32_16x16x4_f32), level by
  // level d = I - J (blocks of one level are independent):
  //   S[I, J] = sum_{J <= M < I} A[I, M] T[M, J],   T[I, J] = -T[I, I] S[I, J]
  // with A[r, s] = beta_r P[r, s]. Sx holds one 16x16 S block per block of
  // the level.
  for (int dl = 1; dl < NB; ++dl) {
    for (int b = w; b < NB - dl; b += 4) {
      const int J = b, I = J + dl;
      f32x4 acc = zero4();
      const float bI = be[16 * I + i];
      for (int Mb = J; Mb < I; ++Mb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = bI * Ms[(16 * I + i) * LDM + 16 * Mb + k0 + g];
          const float t = Ts[(16 * Mb + k0 + g) * LDM + 16 * J + i];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, t, acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) Sx[b * 256 + (4 * g + rr) * 16 + i] = acc[rr];
    }
    __syncthreads();
    for (int b = w; b < NB - dl; b += 4) {
      const int J = b, I = J + dl;
      f32x4 acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float a = Ts[(16 * I + i) * LDM + 16 * I + k0 + g];
        const float sx = Sx[b * 256 + (k0 + g) * 16 + i];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sx, acc, 0, 0, 0);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) Ts[(16 * I + 4 * g + rr) * LDM + 16 * J + i] = -acc[rr];
    }
    __syncthreads();
  }
  // operand copy of T (overwrites P), and T^T for the backward
  for (int e = tid; e < C * C; e += 256) {
    const int r = e / C, s = e % C;
    Tb[r * LDT + s] = from_f<OpT>(Ts[r * LDM + s]);
  }
  if (BWD) {
    OpT* TT = static_cast<OpT*>(ops.TT) + idx * C * C;
    for (int e = tid; e < C * C; e += 256) TT[e] = from_f<OpT>(Ts[(e % C) * LDM + e / C]);
  }
  __syncthreads();

  // ---- W = T Kb and U = T Bv (MFMA). Kb^T / Bv^T fragments are generated:
  // lane (i, g) holds column i (a channel) and k-slots s = s0 + g*KPL + j.
  // The raw k / v values a wave needs are loaded up front (strided reads of
  // the chunk tile, all in flight together).
  constexpr int NSF = C / KS;  // fragments along the chunk
  constexpr int NMW = (K / 16 + 3) / 4;
  OpT* Wn = static_cast<OpT*>(ops.Wn) + idx * C * K;
  {
    float raw[NMW][NSF][KPL], vraw[NMW][NSF][KPL];
#pragma unroll
    for (int jm = 0; jm < NMW; ++jm) {
      const int kk = 16 * (w + 4 * jm) + i;
#pragma unroll
      for (int f = 0; f < NSF; ++f)
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int s_ = f * KS + g * KPL + j;
          const bool ok = s_ < L.len && w + 4 * jm < K / 16;
          raw[jm][f][j] = ok ? to_f(kr[s_ * ts + kk]) : 0.f;
          vraw[jm][f][j] = ok ? to_f(vr[s_ * ts + kk]) : 0.f;
        }
    }
#pragma unroll
    for (int jm = 0; jm < NMW; ++jm) {
      const int mk = w + 4 * jm;
      if (mk >= K / 16) break;
      const int kk = 16 * mk + i;
      f32x4 acc[NB], acc2[NB], accu[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] = acc2[n] = accu[n] = zero4();
#pragma unroll
      for (int f = 0; f < NSF; ++f) {
        const int s0 = f * KS;
        const auto gk = M::make([&](int j) {
          const int s_ = s0 + g * KPL + j;
          return be[s_] * rk[s_] * raw[jm][f][j] * kexp<OpT>(Gs[s_ * LDG + kk]);
        });
        const auto gv = M::make([&](int j) { return be[s0 + g * KPL + j] * vraw[jm][f][j]; });
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const auto tb = M::load(Tb + (16 * n + i) * LDT + s0 + g * KPL);
          acc[n] = M::mma(gk, tb, acc[n]);              // W^T tile (k rows, r cols)
          if (BWD) acc2[n] = M::mma(tb, gk, acc2[n]);   // W tile (r rows, k cols)
          if (BWD) accu[n] = M::mma(gv, tb, accu[n]);   // U^T tile: U[16n + i][16mk + 4g + rr]
          else accu[n] = M::mma(tb, gv, accu[n]);       // U tile: U[16n + 4g + rr][16mk + i]
        }
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        // acc[n][rr] = W[16n + i][16mk + 4g + rr]
        OpT* dst = Wn + (16 * n + i) * K + 16 * mk + 4 * g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f<OpT>(-acc[n][rr]);
        if (BWD) {
          // acc2[n][rr] = W[16n + 4g + rr][16mk + i]  ->  WnT[k][r..r+3]
          OpT* dT = static_cast<OpT*>(ops.WnT) + idx * K * C + (16 * mk + i) * C + 16 * n + 4 * g;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) dT[rr] = from_f<OpT>(-acc2[n][rr]);
        }
        OpT* du = BWD ? static_cast<OpT*>(ops.U) + idx * C * V + (16 * n + i) * V + 16 * mk + 4 * g
                      : static_cast<OpT*>(ops.UT) + idx * V * C + (16 * mk + i) * C + 16 * n + 4 * g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) du[rr] = from_f<OpT>(accu[n][rr]);
      }
    }
  }
}

template <typename TI, typename OpT, int D, int C>
static hipError_t launch_cl(bool bwd, const Dims& d, const Inputs& in, int seg_begin,
                            int seg_chunks, const ChunkOps& ops, hipStream_t s) {
  const dim3 grid(seg_chunks * d.H), block(256);
  if (bwd)
    hipLaunchKernelGGL((k_chunk_local<TI, OpT, D, C, true>), grid, block, 0, s, d, in,
                       seg_begin, ops);
  else
    hipLaunchKernelGGL((k_chunk_local<TI, OpT, D, C, false>), grid, block, 0, s, d, in,
                       seg_begin, ops);
  return hipGetLastError();
}

hipError_t launch_chunk_local(int dtype, int D, int C, bool bwd, const Dims& d,
                              const Inputs& in, int seg_begin, int seg_chunks,
                              const ChunkOps& ops, hipStream_t s) {
#define KDA_CL(TI, DD, CC) \
  if (D == DD && C == CC) return launch_cl<TI, TI, DD, CC>(bwd, d, in, seg_begin, seg_chunks, ops, s);
  if (dtype == 0) {
    KDA_CL(float, 64, 16) KDA_CL(float, 64, 32) KDA_CL(float, 64, 64)
    KDA_CL(float, 128, 16) KDA_CL(float, 128, 32) KDA_CL(float, 128, 64)
  } else {
    KDA_CL(bf16, 64, 32) KDA_CL(bf16, 64, 64) KDA_CL(bf16, 128, 32) KDA_CL(bf16, 128, 64)
  }
#undef KDA_CL
  return hipErrorInvalidValue;
}

}  // namespace kda
