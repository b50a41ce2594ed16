// Inter-chunk state scans: one block (4 waves) per (sequence, head, value
// tile).
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
// MFMA accumulator tiles; a bf16 (or fp32) operand copy sits in LDS.
//
// Work split: wave w owns row block m = w of the chunk (Vn, O or dVn tiles,
// all value blocks of the tile) and MKW row blocks of the state. State, Vn
// and O tiles are held transposed (lane (i, g) has four consecutive value
// columns of one key channel or chunk row), so that every store of them to
// memory is one 4-element vector per tile. The serial
// chunk loop is software-pipelined: the per-chunk operands a wave needs
// (rows of W, qg, Aqk, kg^T, U, gamma, dO, ...) for chunk c+1 are loaded into
// registers while chunk c is computed (two alternating register sets), so the
// global-load latency stays off the recurrence.
// The prefetched values stay raw until use: converting them at load time
// would make the wave wait for the loads right away.
//
// Block-to-XCD mapping: blocks are dealt round-robin to the 8 XCDs, so the
// NVT value tiles of one (sequence, head) get block ids that are equal mod 8
// and share that XCD's L2 for the per-chunk operands they all read.
#include <type_traits>

#include "kda_prologue.h"

namespace kda {

// Block -> (sequence n of the segment's range [n0, n1), head h, value tile vt).
template <int NVT>
__device__ __forceinline__ bool scan_program(const Seg& sg, int H, int& n, int& h, int& vt) {
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  vt = slot % NVT;
  const int nh = (slot / NVT) * 8 + xcd;
  if (nh >= (sg.n1 - sg.n0) * H) return false;
  n = sg.n0 + nh / H;
  h = nh % H;
  return true;
}

// Sequence n's chunks in a segment: chunk-order indices [cb, ce), chunk cb
// at position pos of the sequence; first / last: the segment holds the
// sequence's first / last chunk.
struct SeqRange {
  int cb, ce, pos;
  bool first, last;
};
__device__ __forceinline__ SeqRange seq_range(const Seg& sg, int coff0, int coff1, int n) {
  SeqRange r;
  if (sg.pst) {
    // inside the segment's range whatever the table holds
    r.cb = min(max(sg.pst[n], sg.c0), sg.c1);
    r.ce = min(max(sg.pst[n + 1], r.cb), sg.c1);
    r.pos = sg.pos0;
  } else {
    r.cb = max(coff0, sg.c0);
    r.ce = min(coff1, sg.c1);
    r.pos = r.cb - coff0;
  }
  r.first = r.pos == 0;
  r.last = r.pos + (r.ce - r.cb) == coff1 - coff0;
  return r;
}

// Slot of sequence n's state at the boundary before its chunk `pos`.
__device__ __forceinline__ size_t carry_slot(const CarryMap& m, int n, int pos) {
  int k = 0;
  if (m.ckt) {
    const int2 e = m.ckt[n];
    k = e.y + (e.x + pos) / m.every;
  } else if (m.xr) {
    k = m.xr[n];
  }
  return static_cast<size_t>(min(max(k, 0), m.nslots - 1));
}

// Tile geometry shared by both scans.
template <typename OpT, int D, int C, int BV>
struct ScanGeo {
  using M = Mma<OpT>;
  static constexpr int K = D, V = D, NB = C / 16, NVT = V / BV, BVT = BV / 16;
  static constexpr int NHT = (K / 16) * BVT;  // state tiles
  static constexpr int HPW = NHT / 4;          // state tiles per wave
  static constexpr int MKW = HPW / BVT;        // state row blocks per wave
  static constexpr int NKF = K / M::KS;        // fragments along K
  static constexpr int NCF = C / M::KS;        // fragments along C
  static constexpr int LDH = K + 8, LDC = C + 8;
  static_assert(NHT % 4 == 0 && HPW % BVT == 0, "state tiles must split over 4 waves");
};

// Operands of one chunk for one wave of the forward scan.
template <typename OpT, int D, int C, int BV>
struct FwdOps {
  using G = ScanGeo<OpT, D, C, BV>;
  using F = typename G::M::frag;
  F w[G::NKF];                // W rows of block m (negated: -W)
  F q[G::NKF];                // qg rows of block m (output only)
  F a[G::NCF];                // Aqk rows of block m (output only)
  F al[G::NCF];               // Aqk_lo rows of block m (output, bf16 only)
  uint32_t u[G::BVT][4];      // U[r][v..v+3] at the lane's Vn^T tile entries, raw
                              // bits (converted at use, so the prefetch does not
                              // wait for its loads): fp32 (forward layout) or
                              // the operand type (backward layout, REC)
  F kt[G::MKW][G::NCF];       // kg^T rows of the wave's state row blocks
  float gm[G::MKW];           // gamma at the lane's key channel of each row block
};

// The chunk operands are fragment-major (FragMajor): each fragment load below
// is one contiguous 64-slot run. PART selects the operands of one phase of a
// chunk step (0: W and U; 1: qg and Aqk; 2: kg^T and gamma; -1: all), so
// that a step can issue the next operands in portions between its phases
// instead of all at once (a wave that issues many loads back to back stalls
// until the memory pipeline accepts them).
template <typename OpT, int D, int C, int BV, bool OUT_O, bool REC, int PART = -1>
__device__ __forceinline__ void load_fwd_ops(FwdOps<OpT, D, C, BV>& f, const ChunkOps& ops,
                                             size_t idx, int v0, int w, int i, int g) {
  using G = ScanGeo<OpT, D, C, BV>;
  using M = typename G::M;
  using FM = FragMajor<OpT>;
  constexpr int K = G::K, V = G::V;
  const int lane = i + 16 * g;
  // waves past the last row block (C < 64) load that block's rows again and
  // leave them unused: the loads stay unconditional
  const int m = w < G::NB ? w : G::NB - 1;
  if (PART < 0 || PART == 0) {
    const OpT* Wn = static_cast<const OpT*>(ops.Wn) + idx * C * K;
#pragma unroll
    for (int j = 0; j < G::NKF; ++j) f.w[j] = M::load(Wn + FM::frag(m, j, K, lane));
    if constexpr (REC) {
      const OpT* U = static_cast<const OpT*>(ops.U) + idx * C * V;
#pragma unroll
      for (int nv = 0; nv < G::BVT; ++nv) load4_fm_raw<OpT>(U, 16 * m + i, v0 + 16 * nv + 4 * g, V, f.u[nv]);
    } else {
      // fp32 U in 16x16 blocks (ChunkOps::Uf): block (m, v0/16 + nv), row i, columns 4g ..
      const float* U = ops.Uf + idx * C * V + (m * (V / 16) + v0 / 16) * 256 + i * 16 + 4 * g;
#pragma unroll
      for (int nv = 0; nv < G::BVT; ++nv) load4_raw<float>(U + 256 * nv, f.u[nv]);
    }
  }
  if (OUT_O && (PART < 0 || PART == 1)) {
    const OpT* qg = static_cast<const OpT*>(ops.qg) + idx * C * K;
#pragma unroll
    for (int j = 0; j < G::NKF; ++j) f.q[j] = M::load(qg + FM::frag_p(m, j, K, lane));  // row-parity order
    const OpT* aq = static_cast<const OpT*>(ops.Aqk) + idx * C * C;
    // Aqk[r][s] = 0 for s > r: fragments past the wave's diagonal are never
    // used, and load the last used one again (lines already in flight, so no
    // new misses; the loads stay unconditional)
    const int nf = (16 * (m + 1) + G::M::KS - 1) / G::M::KS;
#pragma unroll
    for (int j = 0; j < G::NCF; ++j) f.a[j] = M::load(aq + FM::frag(m, j < nf ? j : nf - 1, C, lane));
    if constexpr (sizeof(OpT) == 2) {
      const OpT* al = static_cast<const OpT*>(ops.Aqk_lo) + idx * C * C;
#pragma unroll
      for (int j = 0; j < G::NCF; ++j) f.al[j] = M::load(al + FM::frag(m, j < nf ? j : nf - 1, C, lane));
    }
  }
  if (PART < 0 || PART == 2) {
    const OpT* kgT = static_cast<const OpT*>(ops.kgT) + idx * K * C;
    const float* gam = ops.gam + idx * K;
#pragma unroll
    for (int jm = 0; jm < G::MKW; ++jm) {
      const int mk = w * G::MKW + jm;
#pragma unroll
      for (int j = 0; j < G::NCF; ++j) f.kt[jm][j] = M::load(kgT + FM::frag(mk, j, C, lane));
      f.gm[jm] = gam[16 * mk + i];
    }
  }
}

template <typename TI, typename OpT, int D, int C, int BV, bool OUT_O, bool REC>
__global__ void __launch_bounds__(256) k_scan_fwd(Dims d, Inputs in, Seg sgm, ChunkOps ops,
                                                  TI* o, SegStates st, const float* carry_in,
                                                  float* carry_out, CarryMap cm,
                                                  ScanStates ss) {
  using G = ScanGeo<OpT, D, C, BV>;
  using M = typename G::M;
  constexpr int K = G::K, V = G::V, NB = G::NB, NVT = G::NVT, BVT = G::BVT;
  constexpr int HPW = G::HPW, MKW = G::MKW, LDH = G::LDH, LDC = G::LDC, KS = M::KS, KPL = M::KPL;
  // The output's intra-chunk product Aqk Vn of a bf16 problem takes both
  // factors as bf16 pairs (hi + lo, three MFMAs: hi hi, hi lo, lo hi): a
  // plain bf16 rounding of either would add one bf16 rounding's worth of
  // error to O. The state update keeps the single bf16 Vn.
  constexpr bool HL = OUT_O && sizeof(OpT) == 2;
  __shared__ __attribute__((aligned(16))) OpT hT_s[BV * LDH];
  __shared__ __attribute__((aligned(16))) OpT VnT_s[BV * LDC];
  __shared__ __attribute__((aligned(16))) OpT VnTlo_s[HL ? BV * LDC : 1];

  int n, h, vt;
  if (!scan_program<NVT>(sgm, d.H, n, h, vt)) return;
  // sequence bounds read once: the loop's stores could alias them as far as
  // the compiler knows, and a reload would wait for every prefetch in flight
  const SeqRange R = seq_range(sgm, in.coff[n], in.coff[n + 1], n);
  const int64_t tok0 = in.cu[n], tok1 = in.cu[n + 1];
  const int cb = R.cb, ce = R.ce, pofs = R.pos - R.cb;  // chunk c is at position c + pofs
  if (cb >= ce) return;
  const int seg_begin = sgm.c0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int v0 = vt * BV;
  const size_t ts = static_cast<size_t>(d.H) * V, hkv = static_cast<size_t>(d.H) * K * V;
  // U: fp32 in the forward layout, the operand type in the backward one (REC)
  using UT = std::conditional_t<REC, OpT, float>;

  // state tile j of this wave: row block mk = w*MKW + j/BVT, value block
  // nv = j%BVT, held transposed: hs[j][rr] = h[16mk + i][v0 + 16nv + 4g + rr].
  // At the sequence's first chunk the state is its initial state (or zero),
  // otherwise the carry of the previous segment.
  f32x4 hs[HPW];
  const float* hin = !R.first ? carry_in + carry_slot(cm, n, R.pos) * hkv
                     : (ss.init ? ss.init + static_cast<size_t>(n) * hkv : nullptr);
  const bool zero_in = hin == nullptr;
  // offset of the lane's four state values in a [H][K][V] array
  auto hoff = [&](int j) {
    const int mk = w * MKW + j / BVT, nv = j % BVT;
    return (static_cast<size_t>(h) * K + 16 * mk + i) * V + v0 + 16 * nv + 4 * g;
  };
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    hs[j] = zero_in ? zero4() : *reinterpret_cast<const f32x4*>(hin + hoff(j));
  // states entering the backward's segments: chunk c has checkpoint key
  // kofs + c, a checkpoint where the key is a multiple of ck_map.every
  const int ck_every = ss.ck_map.every;
  const int2 ckn = ss.ck ? ss.ck_map.ckt[n] : int2{0, 0};
  const int kofs = ckn.x + pofs;
  int next_ck = ss.ck ? (kofs + cb + ck_every - 1) / ck_every * ck_every - kofs : 0x7fffffff;
  auto put_state = [&]() {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int mk = w * MKW + j / BVT, nv = j % BVT;
      OpT* dst = hT_s + (16 * nv + 4 * g) * LDH + 16 * mk + i;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr * LDH] = from_f<OpT>(hs[j][rr]);
    }
  };
  put_state();

  // Two operand sets alternate so that chunk c + 1 is being loaded while
  // chunk c is computed (the loop is unrolled by two, no register copies).
  // A third set in flight (chunk c + 2) ran no faster and pushed the
  // operand sets into AGPRs (296 registers per wave instead of 200).
  using Ops = FwdOps<OpT, D, C, BV>;
  Ops s0, s1;
  const size_t idx0 = static_cast<size_t>(cb - seg_begin) * d.H + h;
  load_fwd_ops<OpT, D, C, BV, OUT_O, REC>(s0, ops, idx0, v0, w, i, g);
  __syncthreads();

  auto step = [&](int c, const Ops& cur, Ops& fill) {
    const size_t idx = static_cast<size_t>(c - seg_begin) * d.H + h;
    // operands of chunk c + 1, in three portions over the step; unconditional
    // (the last chunk again past the end): on every path the same number of
    // loads follows each set, so the waits before a set's use can leave the
    // next set in flight
    const size_t idx2 = static_cast<size_t>(min(c + 1, ce - 1) - seg_begin) * d.H + h;
    load_fwd_ops<OpT, D, C, BV, OUT_O, REC, 0>(fill, ops, idx2, v0, w, i, g);
    if (c == next_ck) {
      // the state entering chunk c, needed only where c is inside the sequence
      if (c + pofs > 0) {
        const int k = min(max(ckn.y + (kofs + c) / ck_every, 0), ss.ck_map.nslots - 1);
        float* dst = ss.ck + static_cast<size_t>(k) * hkv;
#pragma unroll
        for (int j = 0; j < HPW; ++j) *reinterpret_cast<f32x4*>(dst + hoff(j)) = hs[j];
      }
      next_ck += ck_every;
    }
    if (REC) {
      // entering state h_n, fragment-major [K][V]
      OpT* hd = static_cast<OpT*>(st.h) + idx * K * V;
#pragma unroll
      for (int j = 0; j < HPW; ++j)
        store4_fm<OpT>(hd, 16 * (w * MKW + j / BVT) + i, v0 + 16 * (j % BVT) + 4 * g, V, hs[j]);
    }
    // Vn = U - W h and the inter part qg h of O: row block m = w, all value
    // blocks, as transposed tiles: accV[rr] = Vn[16m + i][v0 + 16nv + 4g + rr]
    f32x4 accO[BVT];
    if (w < NB) {
      const int m = w;
#pragma unroll
      for (int nv = 0; nv < BVT; ++nv) {
        f32x4 accV = unpack4<UT>(cur.u[nv]);
        accO[nv] = zero4();
        const OpT* bh = hT_s + (16 * nv + i) * LDH + g * KPL;
#pragma unroll
        for (int j = 0; j < G::NKF; ++j) {
          const auto b = M::load(bh + j * KS);
          accV = M::mma(b, cur.w[j], accV);
          if (OUT_O) accO[nv] = M::mma(b, cur.q[j], accO[nv]);
        }
        OpT* dst = VnT_s + (16 * nv + 4 * g) * LDC + 16 * m + i;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const OpT hi = from_f<OpT>(accV[rr]);
          dst[rr * LDC] = hi;
          if constexpr (HL) VnTlo_s[(16 * nv + 4 * g + rr) * LDC + 16 * m + i] = from_f<OpT>(accV[rr] - to_f(hi));
        }
        if (REC)
          store4_fm<OpT>(static_cast<OpT*>(st.Vn) + idx * C * V, 16 * m + i, v0 + 16 * nv + 4 * g, V, accV);
      }
    }
    load_fwd_ops<OpT, D, C, BV, OUT_O, REC, 1>(fill, ops, idx2, v0, w, i, g);
    __syncthreads();
    if (OUT_O && w < NB) {
      const int m = w;
      const int64_t t0 = tok0 + static_cast<int64_t>(c + pofs) * C;
      const int len = static_cast<int>(min(static_cast<int64_t>(C), tok1 - t0));
      const int nf = (16 * (m + 1) + KS - 1) / KS;  // Aqk[r][s] = 0 for s > r
      const int r = 16 * m + i;
#pragma unroll
      for (int nv = 0; nv < BVT; ++nv) {
        const OpT* bv = VnT_s + (16 * nv + i) * LDC + g * KPL;
        const OpT* bvl = VnTlo_s + (HL ? (16 * nv + i) * LDC + g * KPL : 0);
#pragma unroll
        for (int j = 0; j < G::NCF; ++j)
          if (j < nf) {
            const auto vh = M::load(bv + j * KS);
            accO[nv] = M::mma(vh, cur.a[j], accO[nv]);
            if constexpr (HL) {
              accO[nv] = M::mma(M::load(bvl + j * KS), cur.a[j], accO[nv]);
              accO[nv] = M::mma(vh, cur.al[j], accO[nv]);
            }
          }
        // accO[nv][rr] = O[r][v0 + 16nv + 4g + rr]
        if constexpr (BVT % 2 != 0)
          if (r < len) store4<TI>(o + (t0 + r) * ts + static_cast<size_t>(h) * V + v0 + 16 * nv + 4 * g, accO[nv]);
      }
      if constexpr (BVT % 2 == 0) {
        // Pairs of value blocks leave as 8 contiguous columns per lane: two
        // lane swaps (upper 32 lanes of the first block with the lower 32 of
        // the second, then odd 16-lane rows of the first with even rows of
        // the second) give the lanes of row group g columns 8g .. 8g + 7 of
        // the pair, so a row's 32 columns are one 64-byte run.
        constexpr int NWD = sizeof(TI) == 2 ? 2 : 4;  // 32-bit words per four values
#pragma unroll
        for (int nv = 0; nv < BVT; nv += 2) {
          uint32_t x[NWD], y[NWD];
          pack4<TI>(accO[nv], x);
          pack4<TI>(accO[nv + 1], y);
#pragma unroll
          for (int k = 0; k < NWD; ++k) {
            const auto a = __builtin_amdgcn_permlane32_swap(x[k], y[k], false, false);
            const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
            x[k] = b[0];
            y[k] = b[1];
          }
          if (r < len) {
            TI* dst = o + (t0 + r) * ts + static_cast<size_t>(h) * V + v0 + 16 * nv + 8 * g;
            if constexpr (NWD == 2) {
              *reinterpret_cast<uint4*>(dst) = make_uint4(x[0], x[1], y[0], y[1]);
            } else {
              *reinterpret_cast<uint4*>(dst) = make_uint4(x[0], x[1], x[2], x[3]);
              *reinterpret_cast<uint4*>(dst + 4) = make_uint4(y[0], y[1], y[2], y[3]);
            }
          }
        }
      }
    }
    load_fwd_ops<OpT, D, C, BV, OUT_O, REC, 2>(fill, ops, idx2, v0, w, i, g);
    // h <- Diag(gamma) h + kg^T Vn, on the transposed tiles
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int jm = j / BVT, nv = j % BVT;
      f32x4 acc;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[rr] = cur.gm[jm] * hs[j][rr];
      const OpT* bv = VnT_s + (16 * nv + i) * LDC + g * KPL;
#pragma unroll
      for (int jj = 0; jj < G::NCF; ++jj) acc = M::mma(M::load(bv + jj * KS), cur.kt[jm][jj], acc);
      hs[j] = acc;
    }
    // hT_s was last read before the barrier above; the barrier below also
    // keeps the next chunk's VnT_s writes behind this chunk's VnT_s reads
    put_state();
    __syncthreads();
  };
  // whole pairs of chunks in the loop (every step issues the same loads, so
  // each wait leaves the newer operand set in flight), then the last chunk
  int c = cb;
  for (; c + 1 < ce; c += 2) {
    step(c, s0, s1);
    step(c + 1, s1, s0);
  }
  if (c < ce) step(c, s0, s1);
  // the state leaves as the next segment's carry, or as the sequence's final state
  float* hout = !R.last ? (carry_out ? carry_out + carry_slot(cm, n, ce + pofs) * hkv : nullptr)
                        : (ss.fin ? ss.fin + static_cast<size_t>(n) * hkv : nullptr);
  if (hout) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) *reinterpret_cast<f32x4*>(hout + hoff(j)) = hs[j];
  }
}

// Operands of one chunk for one wave of the reverse scan.
template <typename TI, typename OpT, int D, int C, int BV>
struct BwdOps {
  using G = ScanGeo<OpT, D, C, BV>;
  using F = typename G::M::frag;
  typedef typename Vec16<TI>::T VT;
  static constexpr int VE = 16 / sizeof(TI);      // dO elements per 16-byte vector
  static constexpr int NVEC = C * BV / VE;        // vectors in the dO tile
  static constexpr int NDO = (NVEC + 255) / 256;  // vectors per thread
  F at[G::NCF];               // Aqk^T rows of block m
  F kg[G::NKF];               // kg rows of block m
  F qt[G::MKW][G::NCF];       // qg^T rows of the wave's state row blocks
  F wt[G::MKW][G::NCF];       // -W^T rows of the wave's state row blocks
  float gm[G::MKW];           // gamma at the lane's key channel of each row block
  VT dOv[NDO];                // dO tile vectors this thread stages into LDS (raw)
};

// PART: 0 the dO tile, 1 Aqk^T and kg, 2 qg^T, -W^T and gamma, -1 all (issued
// in portions over a step, as in the forward scan).
template <typename TI, typename OpT, int D, int C, int BV, int PART = -1>
__device__ __forceinline__ void load_bwd_ops(BwdOps<TI, OpT, D, C, BV>& f, const ChunkOps& ops,
                                             size_t idx, const TI* dO, int64_t t0, int len,
                                             size_t ts, int h, int v0, int tid, int w, int i,
                                             int g) {
  using G = ScanGeo<OpT, D, C, BV>;
  using M = typename G::M;
  using FM = FragMajor<OpT>;
  constexpr int K = G::K, V = G::V;
  const int lane = i + 16 * g;
  if (PART < 0 || PART == 1) {
    const int m = w < G::NB ? w : G::NB - 1;  // unconditional, as in the forward
    const OpT* at = static_cast<const OpT*>(ops.AqkT) + idx * C * C;
    const int f_lo = (16 * m) / G::M::KS;  // Aqk^T[r][s] = 0 for s < r: unused fragments re-load f_lo
#pragma unroll
    for (int j = 0; j < G::NCF; ++j) f.at[j] = M::load(at + FM::frag(m, j < f_lo ? f_lo : j, C, lane));
    const OpT* kg = static_cast<const OpT*>(ops.kg) + idx * C * K;
#pragma unroll
    for (int j = 0; j < G::NKF; ++j) f.kg[j] = M::load(kg + FM::frag_p(m, j, K, lane));  // row-parity order
  }
  if (PART < 0 || PART == 2) {
    const OpT* qgT = static_cast<const OpT*>(ops.qgT) + idx * K * C;
    const OpT* WnT = static_cast<const OpT*>(ops.WnT) + idx * K * C;
    const float* gam = ops.gam + idx * K;
#pragma unroll
    for (int jm = 0; jm < G::MKW; ++jm) {
      const int mk = w * G::MKW + jm;
#pragma unroll
      for (int j = 0; j < G::NCF; ++j) {
        f.qt[jm][j] = M::load(qgT + FM::frag(mk, j, C, lane));
        f.wt[jm][j] = M::load(WnT + FM::frag(mk, j, C, lane));
      }
      f.gm[jm] = gam[16 * mk + i];
    }
  }
  if (PART >= 1) return;
  // rows past the chunk's end read its last row (unconditional loads stay
  // where they are issued; a conditional one would be moved to its use and
  // waited for there) and are zeroed where they are used
  using O = BwdOps<TI, OpT, D, C, BV>;
#pragma unroll
  for (int j = 0; j < O::NDO; ++j) {
    // threads past the tile's vectors load its last one again (unused)
    const int e0 = tid + 256 * j, e = e0 < O::NVEC ? e0 : O::NVEC - 1;
    const int r = e / (BV / O::VE), c0 = (e % (BV / O::VE)) * O::VE, rc = r < len ? r : len - 1;
    f.dOv[j] = *reinterpret_cast<const typename O::VT*>(dO + (t0 + rc) * ts + static_cast<size_t>(h) * V + v0 + c0);
  }
}

template <typename TI, typename OpT, int D, int C, int BV>
__global__ void __launch_bounds__(256) k_scan_bwd(Dims d, Inputs in, const TI* dO, Seg sgm,
                                                  ChunkOps ops, SegStates st,
                                                  const float* carry_in, float* carry_out,
                                                  CarryMap cm, ScanStates ss) {
  using G = ScanGeo<OpT, D, C, BV>;
  using M = typename G::M;
  using Ops = BwdOps<TI, OpT, D, C, BV>;
  constexpr int K = G::K, V = G::V, NB = G::NB, NVT = G::NVT, BVT = G::BVT;
  constexpr int HPW = G::HPW, MKW = G::MKW, LDH = G::LDH, LDC = G::LDC, KS = M::KS, KPL = M::KPL;
  static_assert(C * BV % 256 == 0, "dO tile split");
  __shared__ __attribute__((aligned(16))) OpT dhT_s[BV * LDH];
  __shared__ __attribute__((aligned(16))) OpT dVnT_s[BV * LDC];
  __shared__ __attribute__((aligned(16))) OpT dOT_s[BV * LDC];

  int n, h, vt;
  if (!scan_program<NVT>(sgm, d.H, n, h, vt)) return;
  // sequence bounds read once: the loop's stores could alias them as far as
  // the compiler knows, and a reload would wait for every prefetch in flight
  const SeqRange R = seq_range(sgm, in.coff[n], in.coff[n + 1], n);
  const int64_t tok0 = in.cu[n], tok1 = in.cu[n + 1];
  const int cb = R.cb, ce = R.ce, pofs = R.pos - R.cb;  // chunk c is at position c + pofs
  if (cb >= ce) return;
  const int seg_begin = sgm.c0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int v0 = vt * BV;
  const size_t ts = static_cast<size_t>(d.H) * V, hkv = static_cast<size_t>(d.H) * K * V;
  auto chunk_t0 = [&](int c) {
    return tok0 + static_cast<int64_t>(c + pofs) * C;
  };
  auto chunk_len = [&](int64_t t0) {
    return static_cast<int>(min(static_cast<int64_t>(C), tok1 - t0));
  };

  // dh' (gradient of the state leaving the current chunk), transposed tiles
  // as in the forward scan: hs[j][rr] = dh'[16mk + i][v0 + 16nv + 4g + rr].
  // After the sequence's last chunk it is the final state's gradient (or
  // zero), otherwise the carry of the following segment.
  f32x4 hs[HPW];
  const float* hin = !R.last ? carry_in + carry_slot(cm, n, ce + pofs) * hkv
                     : (ss.init ? ss.init + static_cast<size_t>(n) * hkv : nullptr);
  const bool zero_in = hin == nullptr;
  auto hoff = [&](int j) {
    const int mk = w * MKW + j / BVT, nv = j % BVT;
    return (static_cast<size_t>(h) * K + 16 * mk + i) * V + v0 + 16 * nv + 4 * g;
  };
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    hs[j] = zero_in ? zero4() : *reinterpret_cast<const f32x4*>(hin + hoff(j));
  auto put_state = [&]() {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int mk = w * MKW + j / BVT, nv = j % BVT;
      OpT* dst = dhT_s + (16 * nv + 4 * g) * LDH + 16 * mk + i;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) dst[rr * LDH] = from_f<OpT>(hs[j][rr]);
    }
  };
  put_state();

  // two alternating operand sets: chunk c - 1 loads while chunk c is computed
  Ops s0, s1;
  auto load = [&](Ops& f, int c, auto part) {
    const int64_t t0 = chunk_t0(c);
    load_bwd_ops<TI, OpT, D, C, BV, decltype(part)::value>(
        f, ops, static_cast<size_t>(c - seg_begin) * d.H + h, dO, t0, chunk_len(t0), ts, h, v0,
        tid, w, i, g);
  };
  using All = std::integral_constant<int, -1>;
  load(s0, ce - 1, All{});
  auto step = [&](int c, const Ops& cur, Ops& fill) {
    const size_t idx = static_cast<size_t>(c - seg_begin) * d.H + h;
    // unconditional (the first chunk again past the start), as in the forward
    // scan, and in three portions over the step
    const int c2 = max(c - 1, cb);
    load(fill, c2, std::integral_constant<int, 0>{});
    // dO tile, transposed into LDS ([BV][C]); padded rows are zero
    const int len = chunk_len(chunk_t0(c));
#pragma unroll
    for (int j = 0; j < Ops::NDO; ++j) {
      const int e = tid + 256 * j, r = e / (BV / Ops::VE), c0 = (e % (BV / Ops::VE)) * Ops::VE;
      if (e < Ops::NVEC) {
#pragma unroll
        for (int q = 0; q < Ops::VE; ++q)
          dOT_s[(c0 + q) * LDC + r] = from_f<OpT>(r < len ? static_cast<float>(cur.dOv[j][q]) : 0.f);
      }
    }
    {
      // dh', fragment-major [K][V]
      OpT* hd = static_cast<OpT*>(st.dh) + idx * K * V;
#pragma unroll
      for (int j = 0; j < HPW; ++j)
        store4_fm<OpT>(hd, 16 * (w * MKW + j / BVT) + i, v0 + 16 * (j % BVT) + 4 * g, V, hs[j]);
    }
    load(fill, c2, std::integral_constant<int, 1>{});
    __syncthreads();
    if (w < NB) {
      const int m = w;
      const int f_lo = (16 * m) / KS;  // Aqk^T[r][s] = 0 for s < r
#pragma unroll
      for (int nv = 0; nv < BVT; ++nv) {
        f32x4 acc = zero4();
        const OpT* bo = dOT_s + (16 * nv + i) * LDC + g * KPL;
#pragma unroll
        for (int j = 0; j < G::NCF; ++j)
          if (j >= f_lo) acc = M::mma(cur.at[j], M::load(bo + j * KS), acc);
        const OpT* bd = dhT_s + (16 * nv + i) * LDH + g * KPL;
#pragma unroll
        for (int j = 0; j < G::NKF; ++j) acc = M::mma(cur.kg[j], M::load(bd + j * KS), acc);
        store4<OpT>(dVnT_s + (16 * nv + i) * LDC + 16 * m + 4 * g, acc);
        // dVn^T, fragment-major [V][C]
        store4_fm<OpT>(static_cast<OpT*>(st.dVnT) + idx * V * C, v0 + 16 * nv + i, 16 * m + 4 * g, C, acc);
      }
    }
    load(fill, c2, std::integral_constant<int, 2>{});
    __syncthreads();
    // dh = Diag(gamma) dh' + qg^T dO - W^T dVn, on the transposed tiles
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int jm = j / BVT, nv = j % BVT;
      f32x4 acc;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[rr] = cur.gm[jm] * hs[j][rr];
      const OpT* bo = dOT_s + (16 * nv + i) * LDC + g * KPL;
      const OpT* bv = dVnT_s + (16 * nv + i) * LDC + g * KPL;
#pragma unroll
      for (int jj = 0; jj < G::NCF; ++jj) {
        acc = M::mma(M::load(bo + jj * KS), cur.qt[jm][jj], acc);
        acc = M::mma(M::load(bv + jj * KS), cur.wt[jm][jj], acc);
      }
      hs[j] = acc;
    }
    __syncthreads();  // every wave is done reading dhT_s / dOT_s / dVnT_s of this chunk
    put_state();
  };
  // whole pairs of chunks in the loop, then the first chunk
  int c = ce - 1;
  for (; c - 1 >= cb; c -= 2) {
    step(c, s0, s1);
    step(c - 1, s1, s0);
  }
  if (c >= cb) step(c, s0, s1);
  // the gradient leaves as the previous segment's carry, or, past the
  // sequence's first chunk, as the initial state's gradient
  float* hout = !R.first ? carry_out + carry_slot(cm, n, R.pos) * hkv
                         : (ss.fin ? ss.fin + static_cast<size_t>(n) * hkv : nullptr);
  if (hout) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) *reinterpret_cast<f32x4*>(hout + hoff(j)) = hs[j];
  }
}

// Value-tile width of both scans. The scans are bound by the chunk operands
// each block pulls through its CU (every value tile of a head loads all of
// them), so the width trades CUs in use against operand bytes per state
// column: 32 columns while the (sequence, head) pairs with chunks in the
// segment give at most one such block per CU, 64 columns (half the operand
// bytes per column) once they would give more. Measured per launch on
// MI355X: 1 x 8192 x H64 (256 blocks of 32): 64 columns are 1.4x slower, 16
// columns (512 blocks) 1.55x slower; 8 packed sequences x H16 in windows (512
// blocks of 32, two per CU): 64 columns take the forward scan 0.258 -> 0.218
// ms, the reverse 0.139 -> 0.114 and the recording scan 0.098 -> 0.088; H96
// (384 blocks of 32): forward 0.150 -> 0.128 ms, reverse 0.181 -> 0.144.
static bool wide_tiles(int pairs, int D) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const long groups = (static_cast<long>(pairs) + 7) / 8;
  return groups * 8 * (D / 32) > cus;
}

// Blocks of a scan over segment sg: every (sequence, head) pair of its
// sequence range, in groups of 8 (one per XCD), times the value tiles.
static dim3 scan_grid(const Seg& sg, int H, int NVT) {
  const int groups = ((sg.n1 - sg.n0) * H + 7) / 8;
  return dim3(groups * 8 * NVT);
}

template <typename TI, int D, int C, int BV>
static hipError_t launch_sf_bv(const Dims& d, const Inputs& in, const Seg& sg,
                               const ChunkOps& ops, void* o, const SegStates* st,
                               const float* carry_in, float* carry_out, const CarryMap& cm,
                               const ScanStates& ss, hipStream_t s) {
  const dim3 grid = scan_grid(sg, d.H, D / BV), block(256);
  SegStates z{};
  if (o)
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, true, false>), grid, block, 0, s, d, in, sg,
                       ops, static_cast<TI*>(o), z, carry_in, carry_out, cm, ss);
  else if (st)
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, false, true>), grid, block, 0, s, d, in, sg,
                       ops, nullptr, *st, carry_in, carry_out, cm, ss);
  else
    hipLaunchKernelGGL((k_scan_fwd<TI, TI, D, C, BV, false, false>), grid, block, 0, s, d, in, sg,
                       ops, nullptr, z, carry_in, carry_out, cm, ss);
  return hipGetLastError();
}

template <typename TI, int D, int C>
static hipError_t launch_sf(const Dims& d, const Inputs& in, const Seg& sg, int active,
                            const ChunkOps& ops, void* o, const SegStates* st,
                            const float* carry_in, float* carry_out, const CarryMap& cm,
                            const ScanStates& ss, hipStream_t s) {
  if (sg.n1 <= sg.n0) return hipSuccess;
  if (D >= 64 && wide_tiles(active * d.H, D))
    return launch_sf_bv<TI, D, C, 64>(d, in, sg, ops, o, st, carry_in, carry_out, cm, ss, s);
  return launch_sf_bv<TI, D, C, 32>(d, in, sg, ops, o, st, carry_in, carry_out, cm, ss, s);
}

template <typename TI, int D, int C, int BV>
static hipError_t launch_sb_bv(const Dims& d, const Inputs& in, const void* dO, const Seg& sg,
                               const ChunkOps& ops, const SegStates& st,
                               const float* carry_in, float* carry_out, const CarryMap& cm,
                               const ScanStates& ss, hipStream_t s) {
  hipLaunchKernelGGL((k_scan_bwd<TI, TI, D, C, BV>), scan_grid(sg, d.H, D / BV), dim3(256), 0, s,
                     d, in, static_cast<const TI*>(dO), sg, ops, st, carry_in, carry_out, cm, ss);
  return hipGetLastError();
}

template <typename TI, int D, int C>
static hipError_t launch_sb(const Dims& d, const Inputs& in, const void* dO, const Seg& sg,
                            int active, const ChunkOps& ops, const SegStates& st,
                            const float* carry_in, float* carry_out, const CarryMap& cm,
                            const ScanStates& ss, hipStream_t s) {
  if (sg.n1 <= sg.n0) return hipSuccess;
  if (D >= 64 && wide_tiles(active * d.H, D))
    return launch_sb_bv<TI, D, C, 64>(d, in, dO, sg, ops, st, carry_in, carry_out, cm, ss, s);
  return launch_sb_bv<TI, D, C, 32>(d, in, dO, sg, ops, st, carry_in, carry_out, cm, ss, s);
}

#define KDA_DISPATCH(FN, ...)                                              \
  if (dtype == 0) {                                                        \
    if (D == 64 && C == 16) return FN<float, 64, 16>(__VA_ARGS__);         \
    if (D == 64 && C == 32) return FN<float, 64, 32>(__VA_ARGS__);         \
    if (D == 64 && C == 64) return FN<float, 64, 64>(__VA_ARGS__);         \
    if (D == 128 && C == 16) return FN<float, 128, 16>(__VA_ARGS__);       \
    if (D == 128 && C == 32) return FN<float, 128, 32>(__VA_ARGS__);       \
  } else {                                                                 \
    if (D == 64 && C == 32) return FN<bf16, 64, 32>(__VA_ARGS__);          \
    if (D == 64 && C == 64) return FN<bf16, 64, 64>(__VA_ARGS__);          \
    if (D == 128 && C == 32) return FN<bf16, 128, 32>(__VA_ARGS__);        \
    if (D == 128 && C == 64) return FN<bf16, 128, 64>(__VA_ARGS__);        \
  }                                                                        \
  return hipErrorInvalidValue;

hipError_t launch_scan_fwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           const Seg& sg, int active, const ChunkOps& ops, void* out_o,
                           const SegStates* st, const float* carry_in, float* carry_out,
                           const CarryMap& cm, const ScanStates& ss, hipStream_t s) {
  KDA_DISPATCH(launch_sf, d, in, sg, active, ops, out_o, st, carry_in, carry_out, cm, ss, s)
}

hipError_t launch_scan_bwd(int dtype, int D, int C, const Dims& d, const Inputs& in,
                           const void* dO, const Seg& sg, int active, const ChunkOps& ops,
                           const SegStates& st, const float* carry_in, float* carry_out,
                           const CarryMap& cm, const ScanStates& ss, hipStream_t s) {
  KDA_DISPATCH(launch_sb, d, in, dO, sg, active, ops, st, carry_in, carry_out, cm, ss, s)
}

// Sequences with no tokens: their outgoing state (final state, or the
// initial state's gradient) is the incoming one, or zero. One block per
// (sequence, head); non-empty sequences exit at once.
__global__ void __launch_bounds__(256) k_state_passthrough(const int32_t* cu, int H, int KV,
                                                           const float* src, float* dst) {
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  if (cu[n] != cu[n + 1]) return;
  const size_t off = (static_cast<size_t>(n) * H + h) * KV;
  for (int e = threadIdx.x; e < KV; e += 256) dst[off + e] = src ? src[off + e] : 0.f;
}

hipError_t launch_state_passthrough(const int32_t* cu, int N, int H, int KV, const float* src,
                                    float* dst, hipStream_t s) {
  hipLaunchKernelGGL(k_state_passthrough, dim3(N * H), dim3(256), 0, s, cu, H, KV, src, dst);
  return hipGetLastError();
}

}  // namespace kda
