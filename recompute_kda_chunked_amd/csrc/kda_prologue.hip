// Chunk table and the standalone prologue kernel.
#include "kda_prologue.h"

namespace kda {

// Exclusive prefix sum over n in [0, N) of f(n), by one block of 256
// threads: out(n, sum of f over [0, n)) for every n; returns the total. Each
// thread owns a contiguous run of n; the runs' sums are prefix-summed by a
// shuffle scan in each wave, then the four wave totals are added in wave
// order. Every thread of the block must call it.
template <typename F, typename O>
__device__ int32_t block_scan(int N, F f, O out, int32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int per = (N + 255) / 256;
  const int b = min(N, t * per), e = min(N, b + per);
  int32_t local = 0;
  for (int n = b; n < e; ++n) local += f(n);
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
  const int32_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  int32_t run = woff + incl - local;
  for (int n = b; n < e; ++n) {
    const int32_t x = f(n);
    out(n, run);
    run += x;
  }
  // wsum is free again, and this block's stores are visible to it
  __syncthreads();
  return total;
}

// The chunk table (TableArgs in kda_internal.h). The last block handles the
// per-sequence tables (and, for a plan in sequence order, cloc); for a plan
// by windows, block sg < NS lays out segment sg: sequence n's chunks at
// positions [sg * win, (sg + 1) * win) follow those of sequences 0..n-1, and
// the segment follows every chunk at a position below sg * win.
__global__ void __launch_bounds__(256) k_chunk_table(TableArgs a) {
  __shared__ int32_t wsum[4];
  const int32_t* cu = a.cu;
  const int N = a.N, C = a.C;
  auto nchunks = [&](int n) { return (cu[n + 1] - cu[n] + C - 1) / C; };
  auto put_loc = [&](int P, int n, int pos) {
    const int t0 = cu[n] + pos * C, rem = cu[n + 1] - t0;
    a.cloc[P] = int2{t0, rem < C ? rem : C};
  };
  if (static_cast<int>(blockIdx.x) == static_cast<int>(gridDim.x) - 1) {
    const int32_t nc = block_scan(N, nchunks, [&](int n, int32_t pre) {
      a.coff[n] = pre;
      if (!a.ck_win) a.ckt[n] = int2{pre, 0};
    }, wsum);
    if (threadIdx.x == 0) a.coff[N] = nc;
    if (a.ck_win) {
      // checkpoint slots sequence by sequence: one per window start after
      // the first
      const int E = a.ck_every;
      block_scan(N, [&](int n) { return max(0, (nchunks(n) + E - 1) / E - 1); },
                 [&](int n, int32_t pre) { a.ckt[n] = int2{0, pre - 1}; }, wsum);
    }
    if (a.win) {
      block_scan(N, [&](int n) { return nchunks(n) > a.win ? 1 : 0; },
                 [&](int n, int32_t pre) { a.xr[n] = pre; }, wsum);
    } else {
      // coff is complete and visible after block_scan's closing barrier
      for (int c = threadIdx.x; c < a.NC; c += 256) {
        const int n = find_seq(a.coff, N, c);
        put_loc(c, n, c - a.coff[n]);
      }
    }
    return;
  }
  const int sg = blockIdx.x, W = a.win, p0 = sg * W;
  const int32_t base = block_scan(N, [&](int n) { return min(nchunks(n), p0); },
                                  [](int, int32_t) {}, wsum);
  int32_t* row = a.pst + static_cast<size_t>(sg) * (N + 1);
  const int32_t cnt = block_scan(N, [&](int n) { return min(max(nchunks(n) - p0, 0), W); },
                                 [&](int n, int32_t pre) { row[n] = base + pre; }, wsum);
  if (threadIdx.x == 0) row[N] = base + cnt;
  __syncthreads();
  for (int j = threadIdx.x; j < cnt && base + j < a.NC; j += 256) {
    const int n = find_seq(row, N, base + j);
    put_loc(base + j, n, p0 + (base + j - row[n]));
  }
}

hipError_t launch_chunk_table(const TableArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_table, dim3(a.win ? a.NS + 1 : 1), dim3(256), 0, s, a);
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
