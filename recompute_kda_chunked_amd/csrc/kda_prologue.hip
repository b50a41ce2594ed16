// Chunk table and the standalone prologue kernel.
#include "kda_prologue.h"

namespace kda {

// coff[n] = number of chunks (of length C) in sequences 0..n-1; coff[N] is the
// total. One block; each thread owns a contiguous run of sequences. The
// threads' chunk counts are prefix-summed by a shuffle scan in each wave,
// then the four wave totals are added in wave order.
__global__ void __launch_bounds__(256) k_chunk_table(const int32_t* cu, int N, int C, int NC,
                                                     int32_t* coff, int2* cloc) {
  __shared__ int32_t wsum[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (N + 255) / 256;
  const int b = min(N, t * per), e = min(N, b + per);
  int32_t local = 0;
  for (int n = b; n < e; ++n) local += (cu[n + 1] - cu[n] + C - 1) / C;
  int32_t incl = local;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int32_t woff = 0;
  for (int i = 0; i < w; ++i) woff += wsum[i];
  if (t == 255) coff[N] = woff + incl;
  int32_t run = woff + incl - local;
  for (int n = b; n < e; ++n) {
    coff[n] = run;
    run += (cu[n + 1] - cu[n] + C - 1) / C;
  }
  // the block's coff stores are complete and visible after the barrier
  __syncthreads();
  for (int c = t; c < NC; c += 256) {
    const int n = find_seq(coff, N, c);
    const int t0 = cu[n] + (c - coff[n]) * C, rem = cu[n + 1] - t0;
    cloc[c] = int2{t0, rem < C ? rem : C};
  }
}

hipError_t launch_chunk_table(const int32_t* cu, int N, int C, int NC, int32_t* coff, int2* cloc,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, s, cu, N, C, NC, coff, cloc);
  return hipGetLastError();
}

// One block per (chunk, head): prologue rows, chunk-local cumulative gate sum,
// written out as fp32 qh, kh, beta and gcum.
template <typename TI, int D, int C>
__global__ void __launch_bounds__(256) k_prologue(Dims d, Inputs in, float* qh, float* kh,
                                                  float* beta, float* gcum) {
  typedef typename GateT<TI>::T GV;
  constexpr int LDG = D + 4;
  __shared__ GV Gs[C * LDG];
  __shared__ float rq[C], rqs[C], rk[C], be[C];
  __shared__ GV ptot[4 * D];
  const int c = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const ChunkLoc L = locate<C>(in, d.N, c);
  auto G = [&](int r, int kk) -> GV& { return Gs[r * LDG + kk]; };
  prologue_rows<TI, D, C, 4>(d, in, h, L, rq, rqs, rk, be, G);
  __syncthreads();
  cumsum_rows<D, C, 256>(G, ptot);
  const size_t ts = static_cast<size_t>(d.H) * D;
  const TI* q = static_cast<const TI*>(in.q) + L.t0 * ts + static_cast<size_t>(h) * D;
  const TI* k = static_cast<const TI*>(in.k) + L.t0 * ts + static_cast<size_t>(h) * D;
  for (int idx = threadIdx.x; idx < L.len * D; idx += 256) {
    const int r = idx / D, kk = idx % D;
    const size_t o = (L.t0 + r) * ts + static_cast<size_t>(h) * D + kk;
    qh[o] = to_f(q[r * ts + kk]) * rqs[r];
    kh[o] = to_f(k[r * ts + kk]) * rk[r];
    gcum[o] = static_cast<float>(Gs[r * LDG + kk]);
  }
  for (int r = threadIdx.x; r < L.len; r += 256) beta[(L.t0 + r) * d.H + h] = be[r];
}

template <typename TI, int D, int C>
static hipError_t launch_pro(const Dims& d, const Inputs& in, int n_chunks, float* qh,
                             float* kh, float* beta, float* gcum, hipStream_t s) {
  hipLaunchKernelGGL((k_prologue<TI, D, C>), dim3(n_chunks * d.H), dim3(256), 0, s, d, in,
                     qh, kh, beta, gcum);
  return hipGetLastError();
}

hipError_t launch_prologue(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           int64_t n_chunks, float* qh, float* kh, float* beta, float* gcum,
                           hipStream_t s) {
  const int nc = static_cast<int>(n_chunks);
#define KDA_PRO(TI, DD, CC) \
  if (D == DD && C == CC) return launch_pro<TI, DD, CC>(d, in, nc, qh, kh, beta, gcum, s);
  if (dtype == 0) {
    KDA_PRO(float, 64, 16) KDA_PRO(float, 64, 32) KDA_PRO(float, 64, 64)
    KDA_PRO(float, 128, 16) KDA_PRO(float, 128, 32) KDA_PRO(float, 128, 64)
  } else {
    KDA_PRO(bf16, 64, 16) KDA_PRO(bf16, 64, 32) KDA_PRO(bf16, 64, 64)
    KDA_PRO(bf16, 128, 16) KDA_PRO(bf16, 128, 32) KDA_PRO(bf16, 128, 64)
  }
#undef KDA_PRO
  return hipErrorInvalidValue;
}

}  // namespace kda
