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

// A [D][C] tile (channel rows, chunk-row columns) staged in LDS: written as
// packed row pairs by the element-wise pass, read as MFMA operand fragments
// (KPL consecutive chunk rows of one channel) or drained to memory in
// fragment-major order (contiguous vectors).
template <typename OpT, int D, int C>
struct TileT;

// bf16: unpadded rows of C elements; the 16-byte units of a row are permuted
// by an XOR of channel bits so that both the packed-pair writes (16 lanes on
// channels 8 apart) and the fragment reads (8 lanes on consecutive channels)
// spread over the LDS banks.
template <int D, int C>
struct TileT<bf16, D, C> {
  static_assert(C == 32 || C == 64, "bf16 tiles hold 32 or 64 chunk rows");
  static constexpr int NU = C / 8;                // 16-byte units per row
  static constexpr int R = C == 64 ? 0 : 1;       // log2(rows per 32 banks)
  static constexpr int kElems = D * C;
  static constexpr int kBytes = kElems * 2;
  static __device__ __forceinline__ int swz(int kk) { return ((kk >> R) ^ (kk >> 3)) & (NU - 1); }
  static __device__ __forceinline__ int off(int kk, int s) {
    return kk * C + 8 * ((s >> 3) ^ swz(kk)) + (s & 7);
  }
  // rows s and s + 1 (s even) of channel kk, as a packed pair
  typedef __attribute__((ext_vector_type(2))) __bf16 Pair;
  static __device__ __forceinline__ void put2(bf16* t, int kk, int s, Pair v) {
    *reinterpret_cast<Pair*>(t + off(kk, s)) = v;
  }
  // rows s .. s + 7 (s a multiple of 8) of channel kk
  static __device__ __forceinline__ bf16x8 frag(const bf16* t, int kk, int s) {
    return *reinterpret_cast<const bf16x8*>(t + off(kk, s));
  }
  // slot e of the fragment-major [D][C] array: channel 16 rb + (e & 15),
  // rows sf * 32 + 8 * ((e >> 4) & 3) .. + 7
  static __device__ __forceinline__ void drain(const bf16* t, bf16* dst, int tid) {
    for (int e = tid; e < D * NU; e += 256) {
      const int blk = e >> 6, lane = e & 63;
      const int kk = 16 * (blk / (C / 32)) + (lane & 15), s = 32 * (blk % (C / 32)) + 8 * (lane >> 4);
      vstore<true>(reinterpret_cast<bf16x8*>(dst + 8 * e), frag(t, kk, s));
    }
  }
};

// fp32: rows padded to C + 1 words.
template <int D, int C>
struct TileT<float, D, C> {
  static constexpr int LD = C + 1;
  static constexpr int kElems = D * LD;
  static constexpr int kBytes = kElems * 4;
  typedef __attribute__((ext_vector_type(2))) float Pair;
  static __device__ __forceinline__ void put2(float* t, int kk, int s, Pair v) {
    t[kk * LD + s] = v[0];
    t[kk * LD + s + 1] = v[1];
  }
  static __device__ __forceinline__ float frag(const float* t, int kk, int s) { return t[kk * LD + s]; }
  // fragment-major [D][C]: element 4 e + q is channel 16 rb + (4 e + q) % 16,
  // row 4 sf + ((4 e) >> 4) % 4, four consecutive channels per vector
  static __device__ __forceinline__ void drain(const float* t, float* dst, int tid) {
    for (int e = tid; e < D * C / 4; e += 256) {
      const int blk = e >> 4, l0 = (4 * e) & 63;
      const int kk = 16 * (blk / (C / 4)) + (l0 & 15), s = 4 * (blk % (C / 4)) + (l0 >> 4);
      const float* src = t + kk * LD + s;
      vstore<true>(reinterpret_cast<f32x4*>(dst + 4 * e), f32x4{src[0], src[LD], src[2 * LD], src[3 * LD]});
    }
  }
};

// BWD: backward layouts (AqkT, kg, qgT, WnT, TT, P as well). STATE (forward
// layout only): just the operands of the state recurrence (Wn, U, kg^T,
// gamma), for a pass that only carries the state. PH: a gate per head
// (Dims::gate_head), equal in every channel, so each gate factor is one
// exponential per row instead of one per element.
// G2: GDN-2 ("KDA at the production shape...", section 1.6 and the table of
// section 2.1: akk = (b k Gamma)(k / Gamma)^T, w = M^-1 (b k Gamma),
// u = M^-1 (w v)): a per-channel erase gate b = sigmoid(raw_b) and write gate
// w = sigmoid(raw_w) replace beta. The row side of the k.k products carries
// b, so P is Akk itself (beta = 1 below), Kb = b kh e^G and Bv = w v.
// The per-chunk operands leave with the non-temporal hint: the scans and the
// gradient kernel read them later from HBM, and with the hint the output scan
// runs about 5% and the recording scan about 7% faster, with this kernel's
// own time unchanged.
template <typename TI, typename OpT, int D, int C, bool BWD, bool STATE, bool PH, bool G2>
__global__ void __launch_bounds__(256, 2) k_chunk_local(Dims d, Inputs in, int seg_begin,
                                                     ChunkOps ops) {
  using M = Mma<OpT>;
  constexpr int K = D, V = D, NB = C / 16, KPL = M::KPL, KS = M::KS;
  constexpr int LDG = D + 4;   // Gs row stride (floats)
  constexpr int LDM = C + 4;   // fp32 C x C stride
  constexpr int LDT = C + 8;   // operand C x C stride (16-byte aligned rows)
  constexpr int SZ_M = C * LDM * 4, SZ_TB = C * LDT * (int)sizeof(OpT);
  constexpr int SZ_R = SZ_M > SZ_TB ? SZ_M : SZ_TB;
  using TL = TileT<OpT, D, C>;
  typedef typename GateT<OpT>::T GV;
  constexpr int SZ_G = C * LDG * (int)sizeof(GV), SZ_S = 2 * TL::kBytes;
  constexpr int SZ_T = (C * LDM + 16 * C) * 4;
  constexpr int SZ_GR = SZ_G > SZ_S ? SZ_G : SZ_S;
  // The cumulative gate; then the staging area of the transposed kg^T (qg^T)
  // tiles; then T (fp32) and the inverse's scratch; then the staged operands
  // of W and U. Aqk leaves from registers, so at most the gate region, P and
  // the row scalars are live at once (54 KB at D = 128, C = 64: three blocks
  // per CU).
  __shared__ __attribute__((aligned(16))) unsigned char regG[SZ_GR > SZ_T ? SZ_GR : SZ_T];
  __shared__ __attribute__((aligned(16))) unsigned char regM[SZ_R];  // P, then Tb
  __shared__ __attribute__((aligned(16))) float rq[C], rqs[C], rk[C], be[C];
  __shared__ GV ptot[256];  // cumulative-sum partials: (256 / D) parts of D channels
  GV* Gs = reinterpret_cast<GV*>(regG);
  OpT* tile0 = reinterpret_cast<OpT*>(regG);
  OpT* tile1 = tile0 + TL::kElems;
  float* Ms = reinterpret_cast<float*>(regM);
  OpT* Tb = reinterpret_cast<OpT*>(regM);
  float* Ts = reinterpret_cast<float*>(regG);
  float* Sx = Ts + C * LDM;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int lc = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const ChunkLoc L = locate<C>(in, d.N, seg_begin + lc);
  const size_t idx = static_cast<size_t>(lc) * d.H + h;
  const size_t ts = static_cast<size_t>(d.H) * D;
  const TI* qr = static_cast<const TI*>(in.q) + L.t0 * ts + static_cast<size_t>(h) * D;
  const TI* kr = static_cast<const TI*>(in.k) + L.t0 * ts + static_cast<size_t>(h) * D;
  const TI* vr = static_cast<const TI*>(in.v) + L.t0 * ts + static_cast<size_t>(h) * D;
  // GDN-2 gate rows (raw), [T][H][K] and [T][H][V]
  const TI* bkr = G2 ? static_cast<const TI*>(in.bk) + L.t0 * ts + static_cast<size_t>(h) * D : nullptr;
  const TI* wvr = G2 ? static_cast<const TI*>(in.wv) + L.t0 * ts + static_cast<size_t>(h) * D : nullptr;

  static_assert(C * LDM % 4 == 0, "the fp32 C x C buffers clear in 16-byte pieces");
  for (int e = tid; e < C * LDM / 4; e += 256) reinterpret_cast<f32x4*>(Ms)[e] = zero4();
  auto G = [&](int r, int kk) -> GV& { return Gs[r * LDG + kk]; };
  // the gate in GateUnits (base 2 for bf16): every exponential below is of a
  // difference of these values
  using GU = GateUnits<OpT>;
  prologue_rows<TI, D, C, 4>(d, in, h, L, rq, rqs, rk, be, G, static_cast<GV>(GU::scale));

  // ---- gated products P (= Akk / beta) and Aqk, 16x16 block pairs. Wave w
  // takes pairs w, w + 4, ...; the raw rows of its next pair are loaded while
  // the current one is computed (two register sets), and those of its first
  // pair while the cumulative sum runs. With four row blocks the pairs are
  // numbered so that a wave's pairs share rows: wave 0 takes (3,0), (3,1),
  // (3,2), wave 1 the diagonal (1,1), (2,2), (3,3), wave 2 (2,0), (2,1) and
  // wave 3 (0,0), (1,0); rows the wave already holds are copied, not loaded
  // again (76 KB of row loads per chunk-head instead of 120 KB).
  constexpr int NPAIR = NB * (NB + 1) / 2, PPW = (NPAIR + 3) / 4, NKS = K / KS;
  struct PairRows {
    typename M::frag xa[NKS], xk[NKS], xb[NKS];
    typename M::frag xe[G2 ? NKS : 1];  // GDN-2: raw erase gate of the row-side rows
  };
  auto pair_blocks = [](int p, int& I, int& J) {
    if constexpr (NB == 4) {
      // 4 bits per pair: I = {3,1,2,0,3,2,2,1,3,3}, J = {0,1,0,0,1,2,1,0,2,3}
      I = static_cast<int>((0x3312230213ull >> (4 * p)) & 15);
      J = static_cast<int>((0x3201210010ull >> (4 * p)) & 15);
    } else {
      I = 0;
      J = p;
      while (J > I) { J -= I + 1; ++I; }
    }
  };
  // Rows past the chunk's end read the last valid row (their scales rqs / rk
  // are zero). prev holds pair pp (the wave's previous pair, or pp < 0):
  // its row side is reused when the row block is the same, and the column
  // side's k rows come from the row side (a diagonal pair) or from prev.
  auto load_pair = [&](PairRows& f, int p, const PairRows& prev, int pp) {
    if (p >= NPAIR) return;
    int I, J, Ip = -1, Jp = -1;
    pair_blocks(p, I, J);
    if (pp >= 0 && pp < NPAIR) pair_blocks(pp, Ip, Jp);
    const int ra = 16 * I + i, rb = 16 * J + i;
    const int rac = ra < L.len ? ra : L.len - 1, rbc = rb < L.len ? rb : L.len - 1;
    if (Ip == I) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (!STATE) f.xa[ks] = prev.xa[ks];
        f.xk[ks] = prev.xk[ks];
        if constexpr (G2) f.xe[ks] = prev.xe[ks];
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int kk = ks * KS + g * KPL;
        if (!STATE) f.xa[ks] = M::load(qr + rac * ts + kk);
        f.xk[ks] = M::load(kr + rac * ts + kk);
        if constexpr (G2) f.xe[ks] = M::load(bkr + rac * ts + kk);
      }
    }
    if (J == I) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.xb[ks] = f.xk[ks];
    } else if (J == Jp) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.xb[ks] = prev.xb[ks];
    } else if (J == Ip) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.xb[ks] = prev.xk[ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) f.xb[ks] = M::load(kr + rbc * ts + ks * KS + g * KPL);
    }
  };
  // forward layout of a bf16 problem: Aqk as a bf16 pair (see do_pair, store_aqk)
  constexpr bool HL = !BWD && !STATE && sizeof(OpT) == 2;
  auto el = [](const typename M::frag& f, int j) -> float {
    if constexpr (KPL == 1) return to_f(f);
    else return to_f(f[j]);
  };
  // The Aqk tile of pair p is returned in aq (masked), to be stored after all
  // of the phase's loads are issued: forward, transposed (MFMA operands
  // swapped: aq[rr] = Aqk[16I + i][16J + 4g + rr]); backward, as Aqk^T rows
  // (aq[rr] = Aqk[16I + 4g + rr][16J + i] = Aqk^T[16J + i][16I + 4g + rr]).
  // Either way the lane's four values are consecutive in the stored matrix.
  auto do_pair = [&](const PairRows& f, int p, f32x4& aq) {
    int I, J;
    pair_blocks(p, I, J);
    const int ra = 16 * I + i, rb = 16 * J + i;
    // Row-side operands (rows ra, factors exp(G_ra - G_b) <= 1) are formed
    // without their rows' L2-norm scales, which multiply the products
    // instead (one per output row); column-side operands keep theirs, since
    // their factors reach exp(75) on the diagonal blocks.
    const float sq = rqs[ra], sb = rk[rb];
    f32x4 accP = zero4(), accQ = zero4();
    // per-head gate: the factors of rows ra and rb (every channel alike)
    float ea0 = 0.f, eb0 = 0.f;
    if constexpr (PH) {
      const GV gb = Gs[16 * I * LDG];
      ea0 = GU::ex(Gs[ra * LDG] - gb);
      eb0 = GU::ex(gb - Gs[rb * LDG]);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kk = ks * KS + g * KPL;
      float ea[KPL], eb[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if constexpr (PH) {
          ea[j] = ea0;
          eb[j] = eb0;
        } else {
          const GV gb = Gs[16 * I * LDG + kk + j];
          ea[j] = GU::ex(Gs[ra * LDG + kk + j] - gb);
          eb[j] = GU::ex(gb - Gs[rb * LDG + kk + j]);
        }
      }
      // the row side of P carries the erase gate under GDN-2 (P = Akk)
      const auto fk = M::make([&](int j) {
        const float e = G2 ? sigmoidf(el(f.xe[ks], j)) : 1.f;
        return el(f.xk[ks], j) * ea[j] * e;
      });
      if constexpr (HL) {
        // Aqk of the forward layout from bf16 pairs of both operands (hi hi,
        // lo hi, hi lo): the output takes Aqk directly, and rounding its
        // operands to bf16 alone would add about one bf16 rounding's worth of
        // error to O. P (for the inverse) keeps single bf16 operands.
        float bq[KPL], qv[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          bq[j] = el(f.xb[ks], j) * sb * eb[j];
          qv[j] = el(f.xa[ks], j) * ea[j];
        }
        const auto fb = M::make([&](int j) { return bq[j]; });
        const auto fq = M::make([&](int j) { return qv[j]; });
        const auto fbl = M::make([&](int j) { return bq[j] - el(fb, j); });
        const auto fql = M::make([&](int j) { return qv[j] - el(fq, j); });
        accP = M::mma(fk, fb, accP);
        accQ = M::mma(fb, fq, accQ);
        accQ = M::mma(fbl, fq, accQ);
        accQ = M::mma(fb, fql, accQ);
      } else {
        const auto fb = M::make([&](int j) { return el(f.xb[ks], j) * sb * eb[j]; });
        accP = M::mma(fk, fb, accP);
        if (!STATE) {
          const auto fq = M::make([&](int j) { return el(f.xa[ks], j) * ea[j]; });
          accQ = BWD ? M::mma(fq, fb, accQ) : M::mma(fb, fq, accQ);
        }
      }
    }
    // the row scales: P's rows 16I + 4g + rr (operand A); Aqk's row-side
    // operand is B in the forward layout (output column i: row ra) and A in
    // the backward layout (output row 16I + 4g + rr)
    const f32x4 sk4 = *reinterpret_cast<const f32x4*>(rk + 16 * I + 4 * g);
    const f32x4 sq4 = *reinterpret_cast<const f32x4*>(rqs + 16 * I + 4 * g);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      accP[rr] *= sk4[rr];
      accQ[rr] *= BWD ? sq4[rr] : sq;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 16 * I + 4 * g + rr, s = 16 * J + i;
      Ms[r * LDM + s] = (s < r) ? accP[rr] : 0.f;
      // Aqk[r'][s'] = 0 for s' > r': forward r' = 16I + i, s' = 16J + 4g + rr
      aq[rr] = (BWD ? s <= r : 16 * J + 4 * g + rr <= ra) ? accQ[rr] : 0.f;
    }
  };
  // Aqk (forward) or Aqk^T (backward), fragment-major: the tiles of the
  // wave's pairs, and zeros in the blocks above (Aqk) or below (Aqk^T) the
  // diagonal that share a fragment with entries the scans use (the scans
  // load no fragment that lies wholly in the zero triangle). The forward
  // layout of a bf16 problem also stores what rounding Aqk to bf16 dropped
  // (Aqk_lo), so that the output's intra-chunk product sees Aqk to about
  // 2^-17 of its value.
  auto lo4 = [](const f32x4& v) {
    f32x4 r;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r[rr] = v[rr] - to_f(from_f<OpT>(v[rr]));
    return r;
  };
  auto store_aqk = [&](const f32x4 (&aqv)[PPW]) {
    OpT* dst = static_cast<OpT*>(BWD ? ops.AqkT : ops.Aqk) + idx * C * C;
    OpT* dlo = HL ? static_cast<OpT*>(ops.Aqk_lo) + idx * C * C : nullptr;
#pragma unroll
    for (int it = 0; it < PPW; ++it) {
      const int p = w + 4 * it;
      if (p >= NPAIR) break;
      int I, J;
      pair_blocks(p, I, J);
      if (BWD) {
        store4_fm<OpT, true>(dst, 16 * J + i, 16 * I + 4 * g, C, aqv[it]);
      } else {
        store4_fm<OpT, true>(dst, 16 * I + i, 16 * J + 4 * g, C, aqv[it]);
        if constexpr (HL) store4_fm<OpT, true>(dlo, 16 * I + i, 16 * J + 4 * g, C, lo4(aqv[it]));
      }
    }
    for (int zb = w; zb < NB * (NB - 1) / 2; zb += 4) {
      int I = 1, J = zb;  // zb-th block pair with J < I
      while (J >= I) { J -= I; ++I; }
      // only blocks inside a fragment that a scan wave loads (one that also
      // holds its row block's triangle); the others are never read
      const bool read = BWD ? (16 * J) / KS >= (16 * I) / KS : (16 * I) / KS < (16 * (J + 1) + KS - 1) / KS;
      if (!read) continue;
      if (BWD) {
        store4_fm<OpT, true>(dst, 16 * I + i, 16 * J + 4 * g, C, zero4());
      } else {
        store4_fm<OpT, true>(dst, 16 * J + i, 16 * I + 4 * g, C, zero4());
        if constexpr (HL) store4_fm<OpT, true>(dlo, 16 * J + i, 16 * I + 4 * g, C, zero4());
      }
    }
  };
  // ---- the element-wise pass after the pairs works on (row pair, VE
  // channels) items read as vectors of q, k, v; in the forward layout those
  // loads are issued with the wave's last pair, so they arrive while the
  // pairs finish (the backward layout keeps more registers live and issues
  // them after the pairs: holding them longer would halve its occupancy)
  typedef typename Vec16<TI>::T VT;
  constexpr int VE = 16 / sizeof(TI), LPR = D / VE;
  constexpr int NITEM = (C / 2) * LPR, IPT = (NITEM + 255) / 256;
  VT xq[IPT][2], xk[IPT][2], xv[IPT][2];
  VT xe[G2 ? IPT : 1][2], xw[G2 ? IPT : 1][2];  // GDN-2 raw gate rows
  auto load_items = [&]() {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + 256 * it, rp = item / LPR, c0 = (item % LPR) * VE;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        // rows past the chunk's end read the last valid row (no branch);
        // their scales rqs, rk and beta are zero
        const int r = 2 * rp + h2, rc = (item < NITEM && r < L.len) ? r : L.len - 1;
        const int cc = item < NITEM ? c0 : 0;
        if (!STATE) xq[it][h2] = *reinterpret_cast<const VT*>(qr + rc * ts + cc);
        xk[it][h2] = *reinterpret_cast<const VT*>(kr + rc * ts + cc);
        xv[it][h2] = *reinterpret_cast<const VT*>(vr + rc * ts + cc);
        if constexpr (G2) {
          xe[it][h2] = *reinterpret_cast<const VT*>(bkr + rc * ts + cc);
          xw[it][h2] = *reinterpret_cast<const VT*>(wvr + rc * ts + cc);
        }
      }
    }
  };

  PairRows pa, pb;
  f32x4 aqv[PPW];
  load_pair(pa, w, pb, -1);
  __syncthreads();
  cumsum_rows<D, C, 256>(G, ptot);
#pragma unroll
  for (int it = 0; it < PPW; ++it) {
    const int p = w + 4 * it;
    PairRows& cur = (it & 1) ? pb : pa;
    PairRows& nxt = (it & 1) ? pa : pb;
    if (it + 1 < PPW) load_pair(nxt, p + 4, cur, p);
    else if (!BWD) load_items();
    aqv[it] = zero4();
    if (p < NPAIR) do_pair(cur, p, aqv[it]);
  }
  __syncthreads();
  if (BWD) load_items();

  // ---- outputs that leave before the inverse: Aqk (or its transpose), P^T,
  // gamma, then one pass over the items computing every gated element-wise
  // operand:
  //   qg = qh e^G, kg = kh e^{G_c - G}, Kb = beta kh e^G, Bv = beta v
  // The untransposed ones (qg or kg) are stored directly, fragment-major;
  // transposed ones are staged in LDS (row pairs packed) and leave as
  // contiguous vectors, or wait in registers as the operands of W and U.
  // staged values per item: [0] kg (both), [1] Kb, [2] Bv, [3] qg (backward)
  constexpr int NSV = BWD ? 4 : 3;
  // held in the operand type (bf16 pairs pack into one register): they are
  // rounded to it when staged anyway
  typename TL::Pair sv[IPT][NSV][VE];
  {
    // stores of this phase follow all of its loads (loads and stores share one
    // completion counter)
    if (!STATE) store_aqk(aqv);
    {
      if (BWD) {
        // P^T, so that the gradient kernel reads a lane's four rows of one
        // column as one vector; each thread writes 16-byte pieces of its rows.
        // P is strictly lower triangular: 16x16 blocks of P^T below the block
        // diagonal are zero and are not written (the gradient kernel reads
        // only blocks (ns, m) with ns <= m).
        OpT* PT = static_cast<OpT*>(ops.PT) + idx * C * C;
        constexpr int PV = 16 / (int)sizeof(OpT);  // elements per piece
        static_assert(C % PV == 0 && 16 % PV == 0, "P^T rows split into 16-byte pieces");
        for (int e = tid; e < C * C / PV; e += 256) {
          const int a = e / (C / PV), b0 = (e % (C / PV)) * PV;  // P^T[a][b0 ..] = P[b0 ..][a]
          if (a / 16 > b0 / 16) continue;
          typedef std::conditional_t<sizeof(OpT) == 2, bf16x8, f32x4> PVec;
          PVec v;
#pragma unroll
          for (int j = 0; j < PV; ++j) v[j] = from_f<OpT>(Ms[(b0 + j) * LDM + a]);
          *reinterpret_cast<PVec*>(PT + a * C + b0) = v;
        }
      }
      float* gam = ops.gam + idx * K;
      for (int kk = tid; kk < K; kk += 256) gam[kk] = GU::ex(Gs[(C - 1) * LDG + kk]);
    }
    OpT* rowm = static_cast<OpT*>(BWD ? ops.kg : ops.qg) + idx * C * K;
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + 256 * it, rp = item / LPR, c0 = (item % LPR) * VE;
      if (item >= NITEM) break;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r = 2 * rp + h2;
        const float sq = rqs[r], sk = rk[r], b = be[r];
        float eGr = 0.f, eGcr = 0.f;  // per-head gate: one pair per row
        if constexpr (PH) {
          const GV gr = Gs[r * LDG];
          eGr = GU::ex(gr);
          eGcr = GU::ex(Gs[(C - 1) * LDG] - gr);
        }
        VT out;
#pragma unroll
        for (int j = 0; j < VE; ++j) {
          float eG = eGr, eGc = eGcr;
          if constexpr (!PH) {
            const GV gr = Gs[r * LDG + c0 + j];
            eG = GU::ex(gr);
            eGc = GU::ex(Gs[(C - 1) * LDG + c0 + j] - gr);
          }
          const float kh = to_f(xk[it][h2][j]) * sk;
          const float qg = STATE ? 0.f : to_f(xq[it][h2][j]) * sq * eG;
          const OpT kg = from_f<OpT>(kh * eGc);
          // beta, or under GDN-2 the channel's erase (Kb) and write (Bv) gates
          // (b is then 1 on valid rows, 0 past the chunk's end)
          float bk = b, bw = b;
          if constexpr (G2) {
            bk = b * sigmoidf(to_f(xe[it][h2][j]));
            bw = b * sigmoidf(to_f(xw[it][h2][j]));
          }
          sv[it][0][j][h2] = kg;
          sv[it][1][j][h2] = from_f<OpT>(bk * kh * eG);
          sv[it][2][j][h2] = from_f<OpT>(bw * to_f(xv[it][h2][j]));
          if (BWD) sv[it][NSV - 1][j][h2] = from_f<OpT>(qg);
          out[j] = BWD ? kg : from_f<OpT>(qg);
        }
        if (!STATE) {
          // fragment-major [C][K] in row-parity order (FragMajor::pslot): the
          // VE channels are one lane slot (bf16) or VE slots 16 apart (fp32)
          OpT* dst = rowm + FragMajor<OpT>::off_p(r, c0, K);
          if constexpr (VE == KPL) {
            vstore<true>(reinterpret_cast<VT*>(dst), out);
          } else {
#pragma unroll
            for (int j = 0; j < VE; ++j) vstore<true>(dst + 16 * j, out[j]);
          }
        }
      }
    }
  }
  __syncthreads();  // the gate region is free from here
  // first staging pass: kg^T (and qg^T) leave through the staging area
  auto stage = [&](OpT* tile, int which) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + 256 * it, rp = item / LPR, c0 = (item % LPR) * VE;
      if (item >= NITEM) break;
#pragma unroll
      for (int j = 0; j < VE; ++j)
        TL::put2(tile, c0 + j, 2 * rp, sv[it][which][j]);
    }
  };
  stage(tile0, 0);
  if (BWD) stage(tile1, NSV - 1);
  __syncthreads();
  TL::drain(tile0, static_cast<OpT*>(ops.kgT) + idx * K * C, tid);
  if (BWD) TL::drain(tile1, static_cast<OpT*>(ops.qgT) + idx * K * C, tid);
  __syncthreads();

  // ---- T = (I + Akk)^-1 (in the staging area, free again), diagonal 16x16
  // blocks by forward substitution. The operands of W and U wait in
  // registers (sv) meanwhile.
  for (int e = tid; e < C * LDM / 4; e += 256) reinterpret_cast<f32x4*>(Ts)[e] = zero4();
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
  // operand copy of T (overwrites P), four elements per thread and step,
  // and T^T for the backward
  static_assert(LDM % 4 == 0 && LDT % 4 == 0, "T rows copy in 4-element pieces");
  for (int e = tid; e < C * C / 4; e += 256) {
    const int r = e / (C / 4), s = (e % (C / 4)) * 4;
    store4<OpT>(Tb + r * LDT + s, *reinterpret_cast<const f32x4*>(Ts + r * LDM + s));
  }
  if (BWD) {
    // T^T, fragment-major, one lane slot per thread. T is lower triangular,
    // so fragments wholly left of T^T's diagonal are zero; they are not
    // written (the gradient kernel skips them: tt_frag_nonzero).
    typedef typename M::frag F;
    F* TT = reinterpret_cast<F*>(static_cast<OpT*>(ops.TT) + idx * C * C);
    for (int e = tid; e < C * C / KPL; e += 256) {
      const int blk = e >> 6, lane = e & 63;
      if (!tt_frag_nonzero<OpT>(blk / (C / KS), blk % (C / KS))) continue;
      const int a = 16 * (blk / (C / KS)) + (lane & 15), b = KS * (blk % (C / KS)) + KPL * (lane >> 4);
      TT[e] = M::make([&](int j) { return Ts[(b + j) * LDM + a]; });
    }
  }
  __syncthreads();
  // second staging pass: the operands of W and U into the staging area (T is in Tb)
  stage(tile0, 1);
  stage(tile1, 2);
  // The forward layout keeps U in fp32 (the state-only pass as well, so that
  // the states it recomputes equal those the output scan carries, bit for
  // bit). T has a unit diagonal (exactly 1 in
  // bf16), so the diagonal term of U = T Bv is Bv itself: what rounding Bv =
  // beta * v to the operand type dropped is added back at each U element,
  // from v rows read again here (four values of row 16n + i per tile).
  constexpr int NMW = (K / 16 + 3) / 4;
  constexpr bool UFIX = !BWD && sizeof(OpT) == 2;
  uint32_t vfix[UFIX ? NMW : 1][UFIX ? NB : 1][4];
  uint32_t wfix[UFIX && G2 ? NMW : 1][UFIX && G2 ? NB : 1][4];  // GDN-2 write gate
  if constexpr (UFIX) {
#pragma unroll
    for (int jm = 0; jm < NMW; ++jm) {
      const int mk = (w + 4 * jm) % (K / 16);  // waves past the last key block: loaded, unused
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int r = 16 * n + i, rc = r < L.len ? r : L.len - 1;
        load4_raw<TI>(vr + rc * ts + 16 * mk + 4 * g, vfix[jm][n]);
        if constexpr (G2) load4_raw<TI>(wvr + rc * ts + 16 * mk + 4 * g, wfix[jm][n]);
      }
    }
  }
  __syncthreads();

  // ---- W = T Kb and U = T Bv (MFMA). Kb^T / Bv^T fragments come from the
  // staged tiles: lane (i, g) holds channel i and k-slots s0 + g*KPL + j.
  constexpr int NSF = C / KS;  // fragments along the chunk
  OpT* Wn = static_cast<OpT*>(ops.Wn) + idx * C * K;
  {
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
        const auto gk = TL::frag(tile0, kk, s0 + g * KPL);
        const auto gv = TL::frag(tile1, kk, s0 + g * KPL);
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          if (s0 >= 16 * (n + 1)) continue;  // T[16n + i][s] = 0 for s > 16n + 15
          const auto tb = M::load(Tb + (16 * n + i) * LDT + s0 + g * KPL);
          acc[n] = M::mma(gk, tb, acc[n]);              // W^T tile (k rows, r cols)
          if (BWD) acc2[n] = M::mma(tb, gk, acc2[n]);   // W tile (r rows, k cols)
          accu[n] = M::mma(gv, tb, accu[n]);            // U^T tile: U[16n + i][16mk + 4g + rr]
        }
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        // acc[n][rr] = W[16n + i][16mk + 4g + rr]; all three fragment-major
        store4_fm<OpT, true>(Wn, 16 * n + i, 16 * mk + 4 * g, K, -acc[n]);
        if (BWD) {
          // acc2[n][rr] = W[16n + 4g + rr][16mk + i]  ->  WnT[k][r..r+3]
          store4_fm<OpT, true>(static_cast<OpT*>(ops.WnT) + idx * K * C, 16 * mk + i, 16 * n + 4 * g, C,
                         -acc2[n]);
        }
        if constexpr (BWD) {
          store4_fm<OpT, true>(static_cast<OpT*>(ops.U) + idx * C * V, 16 * n + i, 16 * mk + 4 * g, V, accu[n]);
        } else {
          // fp32 in 16x16 blocks (ChunkOps::Uf): accu[n][rr] = U[16n + i][16mk + 4g + rr]
          f32x4 u = accu[n];
          if constexpr (UFIX) {
            const int r = 16 * n + i;
            const f32x4 v4 = unpack4<TI>(vfix[jm][n]);
            f32x4 w4 = f32x4{1.f, 1.f, 1.f, 1.f};
            if constexpr (G2) {
              const f32x4 x4 = unpack4<TI>(wfix[jm][n]);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) w4[rr] = sigmoidf(x4[rr]);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              // as staged (element pass)
              const float bw = G2 ? be[r] * w4[rr] : be[r];
              const float bv = bw * v4[rr];
              u[rr] += bv - to_f(from_f<OpT>(bv));
            }
          }
          vstore<true>(reinterpret_cast<f32x4*>(ops.Uf + idx * C * V + (n * (V / 16) + mk) * 256 + i * 16 + 4 * g), u);
        }
      }
    }
  }
}

template <typename TI, typename OpT, int D, int C, bool PH, bool G2>
static hipError_t launch_cl(int mode, const Dims& d, const Inputs& in, int seg_begin,
                            int seg_chunks, const ChunkOps& ops, hipStream_t s) {
  const dim3 grid(seg_chunks * d.H), block(256);
  if (mode == KL_BWD)
    hipLaunchKernelGGL((k_chunk_local<TI, OpT, D, C, true, false, PH, G2>), grid, block, 0, s, d,
                       in, seg_begin, ops);
  else if (mode == KL_STATE)
    hipLaunchKernelGGL((k_chunk_local<TI, OpT, D, C, false, true, PH, G2>), grid, block, 0, s, d,
                       in, seg_begin, ops);
  else
    hipLaunchKernelGGL((k_chunk_local<TI, OpT, D, C, false, false, PH, G2>), grid, block, 0, s,
                       d, in, seg_begin, ops);
  return hipGetLastError();
}

hipError_t launch_chunk_local(int dtype, int D, int C, int mode, const Dims& d,
                              const Inputs& in, int seg_begin, int seg_chunks,
                              const ChunkOps& ops, hipStream_t s) {
#define KDA_CL(TI, DD, CC)                                                                   \
  if (D == DD && C == CC)                                                                    \
    return d.gdn2 ? launch_cl<TI, TI, DD, CC, false, true>(mode, d, in, seg_begin, seg_chunks, ops, s) \
           : d.gate_head                                                                     \
               ? launch_cl<TI, TI, DD, CC, true, false>(mode, d, in, seg_begin, seg_chunks, ops, s) \
               : launch_cl<TI, TI, DD, CC, false, false>(mode, d, in, seg_begin, seg_chunks, ops, s);
  if (dtype == 0) {
    KDA_CL(float, 64, 16) KDA_CL(float, 64, 32) KDA_CL(float, 64, 64)
    KDA_CL(float, 128, 16) KDA_CL(float, 128, 32)
  } else {
    KDA_CL(bf16, 64, 32) KDA_CL(bf16, 64, 64) KDA_CL(bf16, 128, 32) KDA_CL(bf16, 128, 64)
  }
#undef KDA_CL
  return hipErrorInvalidValue;
}

}  // namespace kda
