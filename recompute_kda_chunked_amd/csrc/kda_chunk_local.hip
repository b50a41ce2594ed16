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
    // row-major [C][K] outputs: qg (forward) or kg (backward)
    OpT* rowm = static_cast<OpT*>(BWD ? ops.kg : ops.qg) + idx * C * K;
    for (int e = tid; e < C * K; e += 256) {
      const int r = e / K, kk = e % K;
      float val = 0.f;
      if (r < L.len) {
        const float gr = Gs[r * LDG + kk];
        val = BWD ? to_f(kr[r * ts + kk]) * rk[r] * kexp<OpT>(Gs[(C - 1) * LDG + kk] - gr)
                  : to_f(qr[r * ts + kk]) * rqs[r] * kexp<OpT>(gr);
      }
      rowm[e] = from_f<OpT>(val);
    }
    // transposed [K][C] outputs: kgT always, qgT for the backward
    OpT* kgT = static_cast<OpT*>(ops.kgT) + idx * K * C;
    OpT* qgT = BWD ? static_cast<OpT*>(ops.qgT) + idx * K * C : nullptr;
    for (int e = tid; e < K * C; e += 256) {
      const int kk = e / C, r = e % C;
      float vk = 0.f, vq = 0.f;
      if (r < L.len) {
        const float gr = Gs[r * LDG + kk];
        vk = to_f(kr[r * ts + kk]) * rk[r] * kexp<OpT>(Gs[(C - 1) * LDG + kk] - gr);
        if (BWD) vq = to_f(qr[r * ts + kk]) * rqs[r] * kexp<OpT>(gr);
      }
      kgT[e] = from_f<OpT>(vk);
      if (BWD) qgT[e] = from_f<OpT>(vq);
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
  // off-diagonal blocks, one block row at a time:
  //   T[I, J] = -T[I, I] * sum_{J <= M < I} A[I, M] T[M, J]
  for (int I = 1; I < NB; ++I) {
    const int ncol = 16 * I;
    for (int e = tid; e < 16 * ncol; e += 256) {
      const int r = e / ncol, cc = e % ncol;
      const int R = 16 * I + r;
      float s = 0.f;
      for (int m = (cc / 16) * 16; m < ncol; ++m) s += Ms[R * LDM + m] * Ts[m * LDM + cc];
      Sx[r * C + cc] = be[R] * s;
    }
    __syncthreads();
    for (int e = tid; e < 16 * ncol; e += 256) {
      const int r = e / ncol, cc = e % ncol;
      const int R = 16 * I + r;
      float s = 0.f;
      for (int r2 = 0; r2 <= r; ++r2) s += Ts[R * LDM + 16 * I + r2] * Sx[r2 * C + cc];
      Ts[R * LDM + cc] = -s;
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
  OpT* Wn = static_cast<OpT*>(ops.Wn) + idx * C * K;
  for (int mk = w; mk < K / 16; mk += 4) {
    f32x4 acc[NB], acc2[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = acc2[n] = zero4();
    const int kk = 16 * mk + i;
    for (int s0 = 0; s0 < C; s0 += KS) {
      const auto gen = M::make([&](int j) {
        const int s = s0 + g * KPL + j;
        return s < L.len ? be[s] * rk[s] * to_f(kr[s * ts + kk]) * kexp<OpT>(Gs[s * LDG + kk])
                         : 0.f;
      });
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const auto tb = M::load(Tb + (16 * n + i) * LDT + s0 + g * KPL);
        acc[n] = M::mma(gen, tb, acc[n]);      // W^T tile (k rows, r cols)
        if (BWD) acc2[n] = M::mma(tb, gen, acc2[n]);  // W tile (r rows, k cols)
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
    }
  }
  for (int mv = w; mv < V / 16; mv += 4) {
    f32x4 acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = zero4();
    const int vv = 16 * mv + i;
    for (int s0 = 0; s0 < C; s0 += KS) {
      const auto gen = M::make([&](int j) {
        const int s = s0 + g * KPL + j;
        return s < L.len ? be[s] * to_f(vr[s * ts + vv]) : 0.f;
      });
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const auto tb = M::load(Tb + (16 * n + i) * LDT + s0 + g * KPL);
        if (BWD) acc[n] = M::mma(gen, tb, acc[n]);  // U^T tile: U[16n + i][16mv + 4g + rr]
        else acc[n] = M::mma(tb, gen, acc[n]);      // U tile: U[16n + 4g + rr][16mv + i]
      }
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      OpT* dst = BWD ? static_cast<OpT*>(ops.U) + idx * C * V + (16 * n + i) * V + 16 * mv + 4 * g
                     : static_cast<OpT*>(ops.UT) + idx * V * C + (16 * mv + i) * C + 16 * n + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr] = from_f<OpT>(acc[n][rr]);
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
