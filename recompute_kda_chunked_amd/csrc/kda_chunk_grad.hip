// Token-parallel gradient kernel: one block per (chunk, head) of a segment,
// full K and V per block, so every contraction over the value or key
// dimension finishes on chip and each gradient is written once, in its final
// dtype (the tensor-lifetime rule the FROST page credits for its memory
// advantage: no full-sequence fp32 stage buffers, no overlapping old/new
// gradient arrays; "KDA Memory with Recompute...", sections "What are FP32
// stage buffers..." and "Why the larger FROST state series still wins").
//
// Inputs per chunk: the raw q, k, v, raw gate, raw beta and dO; from the
// recompute scans the entering state h_n and leaving-state gradient dh'_n,
// Vn and dVn; from the chunk-local kernel T^T, P, U and -W. Reverse-mode
// differentiation of the chunk operations (notation of the chunk-local
// kernel; Kb = beta*kh*e^G, Bv = beta*v, qg = qh*e^G, kg = kh*e^{G_c-G}):
//   dBv  = T^T dVn          dv   = beta * dBv
//   dKb  = -dBv h^T          (= T^T dW with dW = -dVn h^T)
//   dqg  = dO h^T            dkg  = Vn dh'^T
//   dAqk = tril(dO Vn^T)     dAkk = stril(-dBv U^T - dKb W^T)
//   dbeta = rowsum(dBv*v) + rowsum(dKb*kh*e^G) + rowsum(dAkk*P)
// and for each gated product X[r,s] = sum_k a_rk c_sk e^{G_rk - G_sk} with
// upstream dX ((beta_r dAkk, kh, kh) and (dAqk, qh, kh)):
//   da_r += sum_s dX[r,s] c_s e^{G_r-G_s},  dc_s += sum_r dX[r,s] a_r e^{G_r-G_s}
//   dG_r += a_r * (first sum),              dG_s -= c_s * (second sum)
// plus dqh += dqg e^G, dkh += dkg e^{G_c-G} + beta dKb e^G, the matching dG
// terms, dG_c += sum_r dkg*kg + gamma * rowsum(h * dh'). dg is the reverse
// cumulative sum of dG within the chunk; then the prologue is differentiated
// (L2 normalisation, sigmoid, gate map). Gate-parameter gradients leave as
// per-chunk partials for a fixed-order reduction.
#include <type_traits>

#include "kda_prologue.h"

namespace kda {

template <typename OpT>
__device__ __forceinline__ float frag_at(const typename Mma<OpT>::frag& f, int j);
template <>
__device__ __forceinline__ float frag_at<bf16>(const bf16x8& f, int j) { return static_cast<float>(f[j]); }
template <>
__device__ __forceinline__ float frag_at<float>(const float& f, int) { return f; }

typedef __attribute__((ext_vector_type(4))) double f64x4;

// Arithmetic of the gated-product VJP and of dG. Each gated pair (r, s)
// enters dG twice, +X at row r and -X at row s, and only the pairs that span
// a row survive the reverse cumulative sum; the rest must cancel. For bf16
// problems the pair products run on bf16 MFMA and both sides use identically
// rounded operand values, so the cancellation is exact up to fp32
// accumulation. For fp32 problems (tolerance 1e-5) the products run on fp64
// MFMA (v_mfma_f64_16x16x4_f64, exact products of fp32 operands) and dG is
// kept in fp64.
template <typename OpT>
struct Vjp;
template <>
struct Vjp<bf16> {
  typedef float T;
  typedef f32x4 acc;
  typedef bf16x8 frag;
  static constexpr int KS = 32, KPL = 8;
  static __device__ __forceinline__ acc zero() { return zero4(); }
  static __device__ __forceinline__ acc mma(frag a, frag b, acc c) { return Mma<bf16>::mma(a, b, c); }
  static __device__ __forceinline__ frag load(const bf16* p) { return Mma<bf16>::load(p); }
  template <class F>
  static __device__ __forceinline__ frag make(F f) { return Mma<bf16>::make(f); }
  static __device__ __forceinline__ T rnd(T x) { return to_f(static_cast<bf16>(x)); }
  // of a difference of cumulative gates, kept in base-2 units (GateUnits)
  static __device__ __forceinline__ T ex(T x) { return __builtin_amdgcn_exp2f(x); }
  static __device__ __forceinline__ T sig(T x) { return sigmoidf(x); }
  static __device__ __forceinline__ acc fix(acc x) { return x; }
};
template <>
struct Vjp<float> {
  typedef double T;
  typedef f64x4 acc;
  typedef double frag;
  static constexpr int KS = 4, KPL = 1;
  static __device__ __forceinline__ acc zero() { return acc{0.0, 0.0, 0.0, 0.0}; }
  static __device__ __forceinline__ acc mma(frag a, frag b, acc c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return static_cast<double>(*p); }
  template <class F>
  static __device__ __forceinline__ frag make(F f) { return f(0); }
  static __device__ __forceinline__ T rnd(T x) { return x; }
  static __device__ __forceinline__ T ex(T x) { return exp(x); }
  static __device__ __forceinline__ T sig(T x) { return 1.0 / (1.0 + exp(-x)); }
  // The f64 16x16 accumulator holds row 4r + g in register r of lane group g;
  // move it to the common layout (row 4g + r): the value for row 4g + r sits
  // in lane (i, r), register g.
  static __device__ __forceinline__ acc fix(acc x) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    acc out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int src = i + 16 * r;
      const double v0 = __shfl(x[0], src, kWave), v1 = __shfl(x[1], src, kWave);
      const double v2 = __shfl(x[2], src, kWave), v3 = __shfl(x[3], src, kWave);
      out[r] = g == 0 ? v0 : (g == 1 ? v1 : (g == 2 ? v2 : v3));
    }
    return out;
  }
};

// SPLIT * D / 16 waves: wave w owns key block kb = w % (D/16) (16 channels)
// and row group half = w / (D/16) (one of SPLIT contiguous runs of the
// chunk's 16-row blocks) for every per-element accumulator, and shares the
// chunk-level products with the other waves.
template <int D>
constexpr int grad_split() { return D >= 128 ? 1 : 2; }

// PH: a gate per head (Dims::gate_head): one raw gate value and one gate
// VJP per row.
// G2: GDN-2 (per-channel erase gate b and write gate w instead of beta; the
// chunk-local kernel's P is then Akk, the product of the erase-gated rows
// b kh with kh). The gradient of beta, a row sum that beta could be hoisted
// out of, becomes a per-channel accumulation ("KDA at the production
// shape...", section 1.6): dv = w dBv and dw = v dBv per value channel;
// the erase gate collects kh (dKb e^G) from the W path and kh (row-side sum)
// from the gated-pair VJP of Akk, whose row operand is b kh. dbeta then
// receives draw_b [T][H][K] and dw draw_w [T][H][V].
template <typename TI, typename OpT, int D, int C, bool PH, bool G2>
__global__ void __launch_bounds__(D * 4 * grad_split<D>()) k_chunk_grad(Dims d, Inputs in, const TI* dO,
                                                    int seg_begin, ChunkOps ops, SegStates st,
                                                    TI* dq, TI* dk, TI* dv, TI* dg, TI* dbeta,
                                                    TI* dw, double* partials) {
  using M = Mma<OpT>;
  using VJ = Vjp<OpT>;
  using TG = typename VJ::T;
  typedef typename GateT<OpT>::T GV;  // cumulative gate (fp64 for fp32 problems)
  static_assert(sizeof(GV) == sizeof(TG), "dG reuses the cumulative-gate buffer");
  constexpr int K = D, V = D, NB = C / 16, KPL = M::KPL, KS = M::KS;
  constexpr int SPLIT = grad_split<D>();
  constexpr int NKB = D / 16, NW = SPLIT * NKB, NT = NW * 64;
  constexpr int MR = (NB + SPLIT - 1) / SPLIT;  // row blocks per wave
  constexpr int LDG = C + 4;         // GT [K][LDG] fp32
  constexpr int LDQ = C + 8;         // qT, kT [K][LDQ]
  constexpr int LDA = D + 8;         // [C][LDA] operand buffers
  constexpr int LDX = C + 8;         // [C][LDX] dX buffers
  // GDN-2: the erase gate, transposed like q and k, follows the dX buffers in S6
  constexpr int SZBT = G2 ? K * LDQ * (int)sizeof(TI) : 0;
  constexpr int SZ1 = 4 * C * LDA * (int)sizeof(OpT), SZ2 = 4 * C * LDX * (int)sizeof(OpT) + SZBT;
  constexpr int SZU = SZ1 > SZ2 ? SZ1 : SZ2;
  // after the VJP the operand region holds the scratch of the reverse
  // cumulative sum and of the partial reductions
  constexpr int OFF_S = 0;
  constexpr int OFF_X = (OFF_S + (int)sizeof(TG) * (NT + 64) + 15) / 16 * 16;
  static_assert(OFF_X + C * LDA * (int)sizeof(TI) <= SZU, "LDS scratch must fit");
  __shared__ __attribute__((aligned(16))) GV GT[K * LDG];
  __shared__ __attribute__((aligned(16))) TI qT[K * LDQ];
  __shared__ __attribute__((aligned(16))) TI kT[K * LDQ];
  __shared__ __attribute__((aligned(16))) unsigned char uni[SZU];
  __shared__ __attribute__((aligned(16))) float rq[C], rqs[C], rk[C], be[C];
  __shared__ float dbp[NW][C];
  __shared__ float rowp[2][NKB][C];
  __shared__ float rsum[2][C];  // rowp summed over key blocks
  __shared__ GV ptot[NT];
  __shared__ TG csum[SPLIT][NKB][16];
  // per-head gate: the gate factors of S6 depend on rows only, one table for
  // the block: eblk[I][s] = exp(G_{16I} - G_s) for s < 16(I + 1) (0 above),
  // ediag[r] = exp(G_r - G_{16 floor(r/16)})
  __shared__ TG eblk[PH ? NB * C : 1];
  __shared__ TG ediag[PH ? C : 1];

  OpT* dBv_s = reinterpret_cast<OpT*>(uni);
  OpT* dO_s = dBv_s + C * LDA;
  OpT* Vn_s = dO_s + C * LDA;
  OpT* dKb_s = Vn_s + C * LDA;
  OpT* dXq = reinterpret_cast<OpT*>(uni);
  OpT* dXk = dXq + C * LDX;
  OpT* dXqT = dXk + C * LDX;
  OpT* dXkT = dXqT + C * LDX;
  TI* bT = reinterpret_cast<TI*>(dXkT + C * LDX);  // GDN-2 erase gate, [K][LDQ] (S6)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int kb = w % NKB, half = w / NKB, kk = 16 * kb + i;
  // Row order of the transposed tiles qT, kT and GT: the rows of channel c
  // are permuted in groups of 8 by an XOR with its channel bits from 3 up, so
  // that the transposing writes (lanes on channels 8 apart) spread over the
  // LDS banks; each 8-row group stays contiguous for the 16-byte reads.
  auto swz = [](int c) { return ((c >> 3) & (C / 8 - 1)) << 3; };
  const int swk = swz(kk);  // this lane's channel
  const int lc = blockIdx.x / d.H, h = blockIdx.x % d.H;
  const int cglob = seg_begin + lc;
  const ChunkLoc L = locate<C>(in, d.N, cglob);
  const size_t idx = static_cast<size_t>(lc) * d.H + h;
  const size_t ts = static_cast<size_t>(d.H) * D;
  const size_t hoff = static_cast<size_t>(h) * D;
  const TI* vr = static_cast<const TI*>(in.v) + L.t0 * ts + hoff;
  const TI* bkr = G2 ? static_cast<const TI*>(in.bk) + L.t0 * ts + hoff : nullptr;
  const TI* wvr = G2 ? static_cast<const TI*>(in.wv) + L.t0 * ts + hoff : nullptr;
  auto row_block = [&](int jm) { return half * MR + jm; };  // valid while < NB
  // Rows r0 .. r0 + 3 (r0 a multiple of 4) of this lane's channel in the
  // transposed tiles, read as one vector: the row permutation moves whole
  // groups of 8 rows, so four aligned rows stay adjacent. Likewise four
  // consecutive row scalars.
  typedef std::conditional_t<sizeof(GV) == 4, f32x4, f64x4> GV4;
  auto gt4 = [&](int r0) { return *reinterpret_cast<const GV4*>(GT + kk * LDG + (r0 ^ swk)); };
  auto tile4 = [&](const TI* t, int r0) {
    uint32_t u[4];
    load4_raw<TI>(t + kk * LDQ + (r0 ^ swk), u);
    return unpack4<TI>(u);
  };
  auto sc4 = [](const float* a, int r0) { return *reinterpret_cast<const f32x4*>(a + r0); };

  // Global loads come before any global store: first the prologue's rows
  // (raw q, k, gate, beta; the q and k vectors also feed the transposes of
  // S1), then those of S2/S3 (dVn^T, T^T, dO, Vn, v) during S1, so their
  // latency overlaps the prologue and the cumulative sum. Rows past the
  // chunk's end read the last valid row (no branch) and are masked where
  // they are used.
  static_assert(sizeof(TI) == sizeof(OpT), "inputs and operands share a type");
  typedef typename Vec16<TI>::T VT;
  constexpr int VE = 16 / sizeof(TI), NVR = D / VE, NV = C * NVR, VPT = (NV + NT - 1) / NT;
  constexpr int T2 = (V / 16) * NB, TPW = (T2 + NW - 1) / NW, NKS = C / KS;
  using PR = ProRows<TI, D, C, NW>;
  static_assert(PR::NIT == VPT && PR::LPR == NVR, "prologue rows are the transposes' vectors");
  PR pr;
  prologue_load<TI, D, C, NW>(d, in, h, L, pr);
  VT ldo[VPT], ldn[VPT];
  // wave w takes the TPW tiles w*TPW .. of dBv^T (value block mv, row block
  // nr); they share one value block, so its dVn^T rows are loaded once
  static_assert(NB % TPW == 0, "a wave's tiles share one value block");
  typename M::frag fa[NKS];
  // T^T is staged once per block in LDS (the dKb_s region, unused until S4):
  // every wave's tiles take all of its row blocks, and eight waves loading
  // the same fragments from global memory would pass 8x its bytes through
  // the CU's address unit. One 16-byte piece per thread.
  constexpr int NTT = C * C * (int)sizeof(OpT) / 16, TTPT = (NTT + NT - 1) / NT;
  constexpr int TT_PPF = 64 * KPL * (int)sizeof(OpT) / 16;  // 16-byte pieces per fragment
  uint4 ttv[TTPT];
  static_assert(C <= LDA && C * LDA * (int)sizeof(OpT) % 16 == 0, "T^T fits the dKb_s region");
  uint32_t vin[TPW][4];
  uint32_t win[G2 ? TPW : 1][4];  // GDN-2 write gate at the dv positions
  using FM = FragMajor<OpT>;
  // vector e of the fragment-major Vn: VE elements in slot order, row
  // vn_row(e), columns vn_col(e) .. + VE - 1 (bf16: one lane slot) or rows
  // vn_row(e) .. + 3 of column vn_col(e) (fp32: four lane slots)
  auto vn_row = [](int e) { const int sl = e * VE / KPL; return 16 * ((sl >> 6) / (V / KS)) + (sl & 15); };
  auto vn_col = [](int e) { const int sl = e * VE / KPL; return KS * ((sl >> 6) % (V / KS)) + KPL * ((sl & 63) >> 4); };
  // S2's operands (dVn^T, T^T, v) are requested once the prologue's rows are
  // in use, S3's (dO, Vn) after the transposes: the memory pipeline takes a
  // wave's loads at a bounded rate, and a wave issuing all of them at once
  // would stall before its first arithmetic.
  // ---- S1: prologue, transposed raw q/k, cumulative gate G^T
  auto Gf = [&](int r, int kk_) -> GV& { return GT[kk_ * LDG + (r ^ swz(kk_))]; };
  // G^T in GateUnits (base 2 for bf16: every exponential below is of G or of a
  // difference of G values, and takes a single v_exp_f32)
  prologue_compute<TI, D, C, NW>(d, L, pr, rq, rqs, rk, be, Gf, static_cast<GV>(GateUnits<OpT>::scale));
  {
    const OpT* dVnT = static_cast<const OpT*>(st.dVnT) + idx * V * C;
    const OpT* TT = static_cast<const OpT*>(ops.TT) + idx * C * C;
#pragma unroll
    for (int j = 0; j < TTPT; ++j) {
      // zero fragments (never written) are skipped where a fragment is one
      // wave's pieces, so the test is uniform across the wave; otherwise
      // (fp32) everything is copied and the zero fragments go unused
      const int e = tid + NT * j, blk = (e < NTT ? e : 0) / TT_PPF;
      if (TT_PPF < 64 || tt_frag_nonzero<OpT>(blk / (C / KS), blk % (C / KS)))
        ttv[j] = reinterpret_cast<const uint4*>(TT)[e < NTT ? e : 0];
    }
    {
      const int t = w * TPW < T2 ? w * TPW : 0, mv = t / NB;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) fa[ks] = M::load(dVnT + FM::frag(mv, ks, C, lane));
    }
#pragma unroll
    for (int jt = 0; jt < TPW; ++jt) {
      const int t0 = w * TPW + jt, t = t0 < T2 ? t0 : 0;
      const int mv = t / NB, nr = t % NB;
      const int r = 16 * nr + i, vv = 16 * mv + 4 * g;
      load4_raw<TI>(vr + (r < L.len ? r : L.len - 1) * ts + vv, vin[jt]);
      if constexpr (G2) load4_raw<TI>(wvr + (r < L.len ? r : L.len - 1) * ts + vv, win[jt]);
    }
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int e = tid + NT * j, r = e / NVR, c = (e % NVR) * VE;
    if (e < NV) {
      const bool ok = r < L.len;
#pragma unroll
      for (int q2 = 0; q2 < VE; ++q2) {
        const int rs = r ^ swz(c + q2);
        qT[(c + q2) * LDQ + rs] = ok ? pr.qv[j][q2] : static_cast<TI>(0.f);
        kT[(c + q2) * LDQ + rs] = ok ? pr.kv[j][q2] : static_cast<TI>(0.f);
      }
    }
  }
  {
    const TI* dOr = dO + L.t0 * ts + hoff;
    const OpT* Vn = static_cast<const OpT*>(st.Vn) + idx * C * V;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e0 = tid + NT * j, e = e0 < NV ? e0 : 0, r = e / NVR, c = (e % NVR) * VE;
      const int rc = r < L.len ? r : L.len - 1;
      ldo[j] = *reinterpret_cast<const VT*>(dOr + rc * ts + c);
      ldn[j] = *reinterpret_cast<const VT*>(Vn + e * VE);
    }
  }
  for (int e = tid; e < NW * C; e += NT) dbp[e / C][e % C] = 0.f;
  for (int e = tid; e < 2 * NKB * C; e += NT) (&rowp[0][0][0])[e] = 0.f;
  __syncthreads();
  // T^T goes to LDS between the cumulative sum's barriers: its loads have had
  // the prologue and half the sum to arrive
  cumsum_rows<D, C, NT>(Gf, ptot, [&]() {
#pragma unroll
    for (int j = 0; j < TTPT; ++j) {
      const int e = tid + NT * j, blk = e / TT_PPF;
      if (e < NTT && (TT_PPF < 64 || tt_frag_nonzero<OpT>(blk / (C / KS), blk % (C / KS))))
        reinterpret_cast<uint4*>(dKb_s)[e] = ttv[j];
    }
  });
  if constexpr (PH) {
    // every channel holds the same cumulative gate; channel 0's column of
    // G^T is stored in row order (its permutation is the identity). Read
    // first in S6, after several barriers.
    for (int e = tid; e < NB * C; e += NT) {
      const int I = e / C, s_ = e % C;
      eblk[e] = s_ < 16 * (I + 1) ? VJ::ex(static_cast<TG>(GT[16 * I]) - static_cast<TG>(GT[s_]))
                                  : TG(0);
    }
    for (int r = tid; r < C; r += NT)
      ediag[r] = VJ::ex(static_cast<TG>(GT[r]) - static_cast<TG>(GT[r & ~15]));
  }

  // ---- S2: dBv = T^T dVn (tiles of dBv^T: value rows, chunk-row columns),
  // ---- S3: dO and Vn tiles into LDS. The h, dh' fragments S4 needs are
  // requested before this phase's stores (loads and stores share one
  // completion counter, so a load issued after a store would wait for it).
  constexpr int NVS = V / KS;
  typename M::frag fh[NVS], fdh[NVS];
  uint32_t bsc[G2 ? MR : 1][4];  // GDN-2 erase gate (raw) at the S4 positions
  {
    f32x4 dvv[TPW];
    f32x4 dwv[G2 ? TPW : 1];
#pragma unroll
    for (int jt = 0; jt < TPW; ++jt) {
      const int t = w * TPW + jt;
      if (t >= T2) break;
      const int mv = t / NB, nr = t % NB;
      const int r = 16 * nr + i, vv = 16 * mv + 4 * g;
      f32x4 acc = zero4();
      // the whole reduction is taken (T^T[r][s] is stored as 0 for s < r)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        if (tt_frag_nonzero<OpT>(nr, ks)) acc = M::mma(fa[ks], M::load(dKb_s + FM::frag(nr, ks, C, lane)), acc);
      OpT* dst = dBv_s + r * LDA + vv;
      float part = 0.f;
      const f32x4 vv4 = unpack4<TI>(vin[jt]);
      store4<OpT>(dst, acc);
      if constexpr (G2) {
        // dv = w dBv, draw_w = v dBv w (1 - w), per value channel
        const f32x4 x4 = unpack4<TI>(win[jt]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float wg = sigmoidf(x4[rr]);
          dvv[jt][rr] = be[r] * wg * acc[rr];
          dwv[jt][rr] = acc[rr] * vv4[rr] * wg * (1.f - wg);
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          part += r < L.len ? acc[rr] * vv4[rr] : 0.f;
          dvv[jt][rr] = be[r] * acc[rr];
        }
        part = sum_groups(part);
        if (g == 0) dbp[w][r] += part;
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + NT * j, r = e / NVR, c = (e % NVR) * VE;
      if (e < NV) {
        VT zo;
#pragma unroll
        for (int q2 = 0; q2 < VE; ++q2) zo[q2] = r < L.len ? ldo[j][q2] : static_cast<TI>(0.f);
        *reinterpret_cast<VT*>(dO_s + r * LDA + c) = zo;
        const int rn = vn_row(e), cn = vn_col(e);
        if constexpr (VE == KPL) {
          *reinterpret_cast<VT*>(Vn_s + rn * LDA + cn) = ldn[j];
        } else {
#pragma unroll
          for (int q2 = 0; q2 < VE; ++q2) Vn_s[(rn + q2) * LDA + cn] = ldn[j][q2];
        }
      }
    }
    {
      // rows kk of h and dh' (fragment-major [K][V])
      const OpT* bh = static_cast<const OpT*>(st.h) + idx * K * V;
      const OpT* bdh = static_cast<const OpT*>(st.dh) + idx * K * V;
#pragma unroll
      for (int j = 0; j < NVS; ++j) {
        fh[j] = M::load(bh + FM::frag(kb, j, V, lane));
        fdh[j] = M::load(bdh + FM::frag(kb, j, V, lane));
      }
    }
    if constexpr (G2) {
      // the erase gate of this lane's channel at the rows S4 visits
#pragma unroll
      for (int jm = 0; jm < MR; ++jm) {
        const int m = row_block(jm) < NB ? row_block(jm) : NB - 1;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 16 * m + 4 * g + rr;
          bsc[jm][rr] = load_bits<TI>(bkr + (r < L.len ? r : L.len - 1) * ts + kk);
        }
      }
    }
    TI* dvo = dv + L.t0 * ts + hoff;
    TI* dwo = G2 ? dw + L.t0 * ts + hoff : nullptr;
#pragma unroll
    for (int jt = 0; jt < TPW; ++jt) {
      const int t = w * TPW + jt;
      if (t >= T2) break;
      const int mv = t / NB, nr = t % NB;
      const int r = 16 * nr + i, vv = 16 * mv + 4 * g;
      if (r < L.len) {
        store4<TI>(dvo + r * ts + vv, dvv[jt]);
        if constexpr (G2) store4<TI>(dwo + r * ts + vv, dwv[jt]);
      }
    }
  }
  __syncthreads();

  // ---- S4: products with the states for the wave's (key block, row blocks)
  f32x4 aq[MR], ak[MR];
  f32x4 ab[G2 ? MR : 1];  // GDN-2: gradient of the erase gate b (then draw_b)
  TG aG[MR][4];
#pragma unroll
  for (int jm = 0; jm < MR; ++jm) {
    aq[jm] = ak[jm] = zero4();
    if constexpr (G2) ab[jm] = zero4();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) aG[jm][rr] = 0;
  }
  TG hdh = 0;
  {
    // the wave's rows of h and dh' as B fragments (loaded during S2)
    float hd = 0.f;
#pragma unroll
    for (int j = 0; j < NVS; ++j) {
#pragma unroll
      for (int jj = 0; jj < KPL; ++jj) hd += frag_at<OpT>(fh[j], jj) * frag_at<OpT>(fdh[j], jj);
    }
    hdh = static_cast<TG>(sum_groups(hd));
    const GV Gc = GT[kk * LDG + ((C - 1) ^ swk)];
    TG colsum = 0;
    float vb[4 * MR];  // beta's per-row terms, summed over the row group after the loop
#pragma unroll
    for (int e = 0; e < 4 * MR; ++e) vb[e] = 0.f;
#pragma unroll
    for (int jm = 0; jm < MR; ++jm) {
      const int m = row_block(jm);
      if (m >= NB) break;
      f32x4 rKb = zero4(), rQg = zero4(), rKg = zero4();
#pragma unroll
      for (int j = 0; j < NVS; ++j) {
        const int ro = (16 * m + i) * LDA + j * KS + g * KPL;
        rKb = M::mma(M::load(dBv_s + ro), fh[j], rKb);
        rQg = M::mma(M::load(dO_s + ro), fh[j], rQg);
        rKg = M::mma(M::load(Vn_s + ro), fdh[j], rKg);
      }
      const int r0 = 16 * m + 4 * g;
      const GV4 G4 = gt4(r0);
      const f32x4 q4 = tile4(qT, r0), k4 = tile4(kT, r0);
      const f32x4 rqs4 = sc4(rqs, r0), rk4 = sc4(rk, r0), be4 = sc4(be, r0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = r0 + rr;
        const GV Gv = G4[rr];
        const float eG = GateUnits<OpT>::ex(Gv), eGc = GateUnits<OpT>::ex(Gc - Gv);
        const float qh = q4[rr] * rqs4[rr];
        const float kh = k4[rr] * rk4[rr];
        const float dqg = rQg[rr], dkg = rKg[rr], dKb = -rKb[rr];
        // beta; under GDN-2 the channel's erase gate (be is 1 on valid rows)
        const float b = G2 ? be4[rr] * sigmoidf(bits_to_f<TI>(bsc[jm][rr])) : be4[rr];
        aq[jm][rr] += dqg * eG;
        ak[jm][rr] += dkg * eGc + b * dKb * eG;
        // -kg*dkg here and +kg*dkg in the G_c row cancel in the reverse
        // cumulative sum: both use the same product value
        const TG kgdkg = static_cast<TG>(dkg) * kh * eGc;
        aG[jm][rr] += static_cast<TG>(dqg) * qh * eG - kgdkg + static_cast<TG>(dKb) * b * kh * eG;
        colsum += kgdkg;
        dKb_s[r * LDA + kk] = from_f<OpT>(dKb);
        if constexpr (G2) {
          ab[jm][rr] += dKb * kh * eG;
        } else {
          vb[4 * jm + rr] = dKb * kh * eG;
        }
      }
    }
    if constexpr (!G2) {
      const float pb = transpose_sum16<4 * MR>(vb);
      const int j = i % (4 * MR), m = row_block(j / 4);
      if (i < 4 * MR && m < NB) dbp[w][16 * m + 4 * g + j % 4] += pb;
    }
    colsum += __shfl_xor(colsum, 16, kWave);
    colsum += __shfl_xor(colsum, 32, kWave);
    if (g == 0) csum[half][kb][i] = colsum;
  }
  __syncthreads();

  // ---- S5: dAqk and dAkk, lower 16x16 blocks (m rows, ns columns)
  constexpr int NPAIR = NB * (NB + 1) / 2, PPW = (NPAIR + NW - 1) / NW;
  // Pair p of wave w is p = w + NW jp. With four row blocks and eight waves
  // only waves 0 and 1 take two pairs; they get (0,0), (1,0) and (2,0), (3,0),
  // whose U and W rows (block ns = 0) they load once.
  auto s5_pair = [](int p, int& m, int& ns) {
    if constexpr (NB == 4 && NW == 8) {
      // m = {0,2,1,2,3,2,3,3,1,3}, ns = {0,0,1,1,1,2,2,3,0,0}, 4 bits per pair
      m = static_cast<int>((0x3133232120ull >> (4 * p)) & 15);
      ns = static_cast<int>((0x32211100ull >> (4 * p)) & 15);
    } else {
      m = 0;
      ns = p;
      while (ns > m) { ns -= m + 1; ++m; }
    }
  };
  f32x4 xq[PPW], xk[PPW];
  // GDN-2: the erase gate rows, requested now and transposed into LDS for S6
  VT braw[G2 ? VPT : 1];
  if constexpr (G2) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e0 = tid + NT * j, e = e0 < NV ? e0 : 0, r = e / NVR, c = (e % NVR) * VE;
      braw[j] = *reinterpret_cast<const VT*>(bkr + (r < L.len ? r : L.len - 1) * ts + c);
    }
  }
  {
    const OpT* Ug = static_cast<const OpT*>(ops.U) + idx * C * V;
    const OpT* Wng = static_cast<const OpT*>(ops.Wn) + idx * C * K;
    const OpT* PTg = static_cast<const OpT*>(ops.PT) + idx * C * C;
    // beta's per-row terms of the wave's pairs (row block pm, -1 past the
    // last pair), summed over the row group after the loop
    static_assert(PPW == 1 || PPW == 2 || PPW == 4, "pairs per wave");
    float vb[4 * PPW];
    int pm[PPW];
    constexpr int NKV = V / KS;
    typename M::frag fu[NKV], fw[NKV];  // U and -W rows of block ns (kept while ns repeats)
    int ns_held = -1;
#pragma unroll
    for (int jp = 0; jp < PPW; ++jp) {
      const int p = w + NW * jp;
      xq[jp] = xk[jp] = zero4();
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vb[4 * jp + rr] = 0.f;
      pm[jp] = -1;
      if (p >= NPAIR) continue;
      int m, ns;
      s5_pair(p, m, ns);
      pm[jp] = m;
      // global operands of this pair first (U and -W rows of block ns, P^T)
      uint32_t pv[4];  // raw: converted at use
      if (ns != ns_held) {
#pragma unroll
        for (int j = 0; j < NKV; ++j) {
          fu[j] = M::load(Ug + FragMajor<OpT>::frag(ns, j, V, lane));  // both fragment-major
          fw[j] = M::load(Wng + FragMajor<OpT>::frag(ns, j, K, lane));
        }
        ns_held = ns;
      }
      load4_raw<OpT>(PTg + (16 * ns + i) * C + 16 * m + 4 * g, pv);  // P[16m + 4g + rr][16ns + i]
      const f32x4 aqk = tile_nt<OpT>(zero4(), dO_s + 16 * m * LDA, LDA, Vn_s + 16 * ns * LDA, LDA, 0, V, lane);
      f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int ao = (16 * m + i) * LDA + j * KS + g * KPL;
        a1 = M::mma(M::load(dBv_s + ao), fu[j], a1);
        a2 = M::mma(M::load(dKb_s + ao), fw[j], a2);
      }
      const f32x4 p4 = unpack4<OpT>(pv);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = 16 * m + 4 * g + rr, s_ = 16 * ns + i;
        xq[jp][rr] = (s_ <= r) ? aqk[rr] : 0.f;
        const float dakk = (s_ < r) ? (a2[rr] - a1[rr]) : 0.f;
        xk[jp][rr] = be[r] * dakk;
        if constexpr (!G2) vb[4 * jp + rr] = dakk * p4[rr];  // GDN-2: the erase gate takes it in S6
      }
    }
    if constexpr (!G2) {
      const float pb = transpose_sum16<4 * PPW>(vb);
      const int j = i % (4 * PPW);
      int m = -1;
#pragma unroll
      for (int jp = 0; jp < PPW; ++jp) m = (j / 4 == jp) ? pm[jp] : m;
      // two pairs of a wave may share a row block: the add is atomic
      if (i < 4 * PPW && m >= 0) atomicAdd(&dbp[w][16 * m + 4 * g + j % 4], pb);
    }
  }
  __syncthreads();  // operand buffers are dead; the dX buffers reuse their space
  {
    // the four dX buffers are cleared 16 bytes per store
    constexpr int NZ = 4 * C * LDX * (int)sizeof(OpT) / 16;
    static_assert(4 * C * LDX * (int)sizeof(OpT) % 16 == 0, "dX buffers clear in 16-byte pieces");
    uint4* z = reinterpret_cast<uint4*>(dXq);
    for (int e = tid; e < NZ; e += NT) z[e] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
#pragma unroll
  for (int jp = 0; jp < PPW; ++jp) {
    const int p = w + NW * jp;
    if (p >= NPAIR) break;
    int m, ns;
    s5_pair(p, m, ns);
    const int s_ = 16 * ns + i, r0 = 16 * m + 4 * g;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      dXq[(r0 + rr) * LDX + s_] = from_f<OpT>(xq[jp][rr]);
      dXk[(r0 + rr) * LDX + s_] = from_f<OpT>(xk[jp][rr]);
    }
    store4<OpT>(dXqT + s_ * LDX + r0, xq[jp]);  // four adjacent columns
    store4<OpT>(dXkT + s_ * LDX + r0, xk[jp]);
  }
  if constexpr (G2) {
    // b = sigmoid(raw_b), transposed and row-permuted like kT (0 past the end)
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + NT * j, r = e / NVR, c = (e % NVR) * VE;
      if (e < NV) {
#pragma unroll
        for (int q2 = 0; q2 < VE; ++q2)
          bT[(c + q2) * LDQ + (r ^ swz(c + q2))] =
              from_f<TI>(r < L.len ? sigmoidf(to_f(braw[j][q2])) : 0.f);
      }
    }
  }
  __syncthreads();

  // ---- S6: VJP of the gated products
  // Operands are generated from the raw inputs and G^T. For each block pair
  // (I, J <= I) the decay exp(G_r - G_s) is split around the first row b of
  // block I (as in the forward), so every generated factor is finite.
  {
    const GV* Gk = GT + kk * LDG;
    const TI* qk = qT + kk * LDQ;
    const TI* kq = kT + kk * LDQ;
    auto khat = [&](int r) { return static_cast<TG>(to_f(kq[r ^ swk])) * static_cast<TG>(rk[r]); };
    auto qhat = [&](int r) { return static_cast<TG>(to_f(qk[r ^ swk])) * static_cast<TG>(rqs[r]); };
    auto dec = [&](int r, int s_) {
      return VJ::ex(static_cast<TG>(Gk[r ^ swk]) - static_cast<TG>(Gk[s_ ^ swk]));
    };
    // Eight consecutive rows r0..r0+7 (r0 a multiple of 8) of this channel's
    // raw q or k, its row scale and G, read as 16-byte LDS vectors (bf16
    // operands; the fp32 path reads one row per lane).
    struct Rows8 {
      float x[8], sc[8], G[8];
    };
    auto rows8 = [&](const TI* col, const float* scale, int r0) {
      Rows8 o;
      if constexpr (VJ::KPL == 8) {
        const bf16x8 xv = *reinterpret_cast<const bf16x8*>(col + (r0 ^ swk));
        const f32x4 s0v = *reinterpret_cast<const f32x4*>(scale + r0);
        const f32x4 s1v = *reinterpret_cast<const f32x4*>(scale + r0 + 4);
        const f32x4 g0v = *reinterpret_cast<const f32x4*>(Gk + (r0 ^ swk));
        const f32x4 g1v = *reinterpret_cast<const f32x4*>(Gk + (r0 ^ swk) + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o.x[j] = to_f(xv[j]);
          o.x[j + 4] = to_f(xv[j + 4]);
          o.sc[j] = s0v[j];
          o.sc[j + 4] = s1v[j];
          o.G[j] = g0v[j];
          o.G[j + 4] = g1v[j];
        }
      }
      return o;
    };
#pragma unroll
    for (int jm = 0; jm < MR; ++jm) {
      const int I = row_block(jm);
      if (I >= NB) break;
      const int b0 = 16 * I;
      // row side: rows r of block I, reduction over s < 16(I + 1):
      //   raw[r] = sum_s dX[r][s] * kh_s exp(G_b - G_s)
      typename VJ::acc rq_ = VJ::zero(), rk_ = VJ::zero();
      const int s_hi = 16 * (I + 1);
#pragma unroll
      for (int s0 = 0; s0 < (s_hi + VJ::KS - 1) / VJ::KS * VJ::KS; s0 += VJ::KS) {
        typename VJ::frag fb;
        if constexpr (VJ::KPL == 8) {
          const int sb = s0 + g * 8;
          const Rows8 v = rows8(kq, rk, sb);
          const float gb = Gk[b0 ^ swk];
          fb = VJ::make([&](int j) {
            const TG e = PH ? eblk[I * C + sb + j] : VJ::ex(gb - v.G[j]);
            return sb + j < s_hi ? v.x[j] * v.sc[j] * e : TG(0);
          });
        } else {
          fb = VJ::make([&](int j) {
            const int s_ = s0 + g * VJ::KPL + j;
            return s_ < s_hi ? khat(s_) * (PH ? eblk[I * C + s_] : dec(b0, s_)) : TG(0);
          });
        }
        const int ao = (16 * I + i) * LDX + s0 + g * VJ::KPL;
        rq_ = VJ::mma(VJ::load(dXq + ao), fb, rq_);
        rk_ = VJ::mma(VJ::load(dXk + ao), fb, rk_);
      }
      rq_ = VJ::fix(rq_);
      rk_ = VJ::fix(rk_);
      const int r0 = b0 + 4 * g;
      const GV4 G4 = gt4(r0);
      const f32x4 q4 = tile4(qT, r0), k4 = tile4(kT, r0), rqs4 = sc4(rqs, r0), rk4 = sc4(rk, r0);
      const TG gb0 = static_cast<TG>(Gk[b0 ^ swk]);
      // GDN-2: the erase gate at rows r0 .. r0 + 3 (the row operand of Akk is b kh)
      f32x4 b4 = f32x4{1.f, 1.f, 1.f, 1.f};
      if constexpr (G2) b4 = tile4(bT, r0);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const TG f = PH ? ediag[r0 + rr] : VJ::ex(static_cast<TG>(G4[rr]) - gb0);  // exp(G_r - G_b)
        // dG takes the column side's operand values for this pair, rounded as
        // that side's MFMA operands are (see Vjp)
        const TG khr = static_cast<TG>(k4[rr]) * static_cast<TG>(rk4[rr]);
        const TG Aq = VJ::rnd(static_cast<TG>(q4[rr]) * static_cast<TG>(rqs4[rr]) * f),
                 Ak = VJ::rnd(khr * static_cast<TG>(b4[rr]) * f);
        aq[jm][rr] += static_cast<float>(rq_[rr] * f);
        ak[jm][rr] += static_cast<float>(rk_[rr] * f * static_cast<TG>(b4[rr]));
        if constexpr (G2) ab[jm][rr] += static_cast<float>(rk_[rr] * f * khr);
        aG[jm][rr] += Aq * rq_[rr] + Ak * rk_[rr];
      }
      if constexpr (G2) {
        // the erase gate's own gradient through its sigmoid: draw_b
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ab[jm][rr] *= b4[rr] * (1.f - b4[rr]);
      }
      // column side: rows s of block J = I here, reduction over r in blocks
      // I2 >= J; the 32-long reduction index u covers (beta*dAkk, kh) for
      // u < 16 and (dAqk, qh) above:  y[s] = sum_r dX[r][s] * a_r exp(G_r - G_b)
      const int J = I;
      TG cc[4] = {0, 0, 0, 0}, gs[4] = {0, 0, 0, 0};
      // rows s = 16J + 4g .. + 3: G_s, raw k and its scale, for every block I2
      const GV4 Gs4 = gt4(16 * J + 4 * g);
      const f32x4 ks4 = tile4(kT, 16 * J + 4 * g), rks4 = sc4(rk, 16 * J + 4 * g);
#pragma unroll
      for (int I2 = J; I2 < NB; ++I2) {
        const int c0 = 16 * I2;
        typename VJ::acc y = VJ::zero();
#pragma unroll
        for (int u0 = 0; u0 < 32; u0 += VJ::KS) {
          const int u = u0 + g * VJ::KPL;
          const OpT* ap = (u < 16 ? dXkT : dXqT) + (16 * J + i) * LDX + c0 + (u & 15);
          typename VJ::frag fb;
          if constexpr (VJ::KPL == 8) {
            // u is 0, 8, 16 or 24: rows c0 + (u & 15) .. + 7 of kh (u < 16) or qh
            const int rb = c0 + (u & 15);
            const Rows8 v = u < 16 ? rows8(kq, rk, rb) : rows8(qk, rqs, rb);
            const float gc = Gk[c0 ^ swk];
            float eg[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) eg[j] = 1.f;
            if constexpr (G2) {
              // the row operand of the Akk part is b kh
              if (u < 16) {
                const bf16x8 bv8 = *reinterpret_cast<const bf16x8*>(bT + kk * LDQ + (rb ^ swk));
#pragma unroll
                for (int j = 0; j < 8; ++j) eg[j] = to_f(bv8[j]);
              }
            }
            fb = VJ::make([&](int j) {
              return v.x[j] * v.sc[j] * eg[j] * (PH ? ediag[rb + j] : VJ::ex(v.G[j] - gc));
            });
          } else {
            fb = VJ::make([&](int j) {
              const int uu = u + j, r = c0 + (uu & 15);
              const TG e = (G2 && uu < 16) ? static_cast<TG>(to_f(bT[kk * LDQ + (r ^ swk)])) : TG(1);
              return (uu < 16 ? khat(r) : qhat(r)) * e * (PH ? ediag[r] : dec(r, c0));
            });
          }
          y = VJ::mma(VJ::load(ap), fb, y);
        }
        y = VJ::fix(y);
        const TG gc0 = static_cast<TG>(Gk[c0 ^ swk]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          // exp(G_b - G_s), b = c0
          const TG f = PH ? eblk[I2 * C + 16 * J + 4 * g + rr] : VJ::ex(gc0 - static_cast<TG>(Gs4[rr]));
          cc[rr] += y[rr] * f;
          // the row side's B operand value
          gs[rr] += VJ::rnd(static_cast<TG>(ks4[rr]) * static_cast<TG>(rks4[rr]) * f) * y[rr];
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        ak[jm][rr] += static_cast<float>(cc[rr]);
        aG[jm][rr] -= gs[rr];
      }
    }
  }

  // ---- S7: row reductions for the L2-norm VJP; G_c terms; reverse cumsum of dG
  // (the raw gate and dt_bias that S8 needs are loaded first, so their
  // latency overlaps this phase and no load follows a store in S8)
  constexpr int PER = (C * D + NT - 1) / NT;
  static_assert(NT % D == 0, "one channel per thread in the gate VJP");
  // The raw gate rows come in as 16-byte vectors and wait in LDS for the gate
  // VJP (whose thread-per-channel mapping would otherwise take a 2-byte load
  // per element); draw_g goes out the same way, staged in LDS. dq and dk
  // leave from the lanes that form them after a 4x4 transpose within each
  // quad of lanes (four channels of one row per lane): staging them through
  // LDS cost 32 two-byte LDS stores per lane on the phase's chain, and
  // storing each lane's four rows of one channel took 32 two-byte stores.
  // (a per-head gate is read in S8 instead)
  VT xrow[VPT];
  float dbias = 0.f;
  if constexpr (!PH) {
    dbias = in.dt_bias[hoff + tid % D];
    const TI* xr = static_cast<const TI*>(in.g) + L.t0 * ts + hoff;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e0 = tid + NT * j, e = e0 < NV ? e0 : 0, r = e / NVR, c = (e % NVR) * VE;
      const int rc = r < L.len ? r : L.len - 1;  // clamped row, masked at use
      xrow[j] = *reinterpret_cast<const VT*>(xr + rc * ts + c);
    }
  }
  // exp(A_log) in the gate's precision, as the forward's gate map takes it
  // (A_log[h] from the prologue's loads: a load issued here would wait
  // behind this phase's others)
  const TG eat = exp(static_cast<TG>(pr.alog));
  // the wave's per-row sums over its 16 channels: value 4 jm + rr of every
  // lane, summed across the lanes of its row group in one transposed sum
  // that leaves row value j in lane j
  float vq[4 * MR], vk[4 * MR];
#pragma unroll
  for (int jm = 0; jm < MR; ++jm) {
    const int m = row_block(jm);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) vq[4 * jm + rr] = vk[4 * jm + rr] = 0.f;
    if (m >= NB) continue;
    const int r0 = 16 * m + 4 * g;
    const f32x4 q4 = tile4(qT, r0), k4 = tile4(kT, r0), rq4 = sc4(rq, r0), rk4 = sc4(rk, r0);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      vq[4 * jm + rr] = q4[rr] * rq4[rr] * aq[jm][rr];
      vk[4 * jm + rr] = k4[rr] * rk4[rr] * ak[jm][rr];
    }
    // row C-1 holds G_c: add sum_r kg*dkg over all row groups and gamma * (h . dh')
    if (m == NB - 1 && g == 3) {
      const GV Gc = GT[kk * LDG + ((C - 1) ^ swk)];
      TG cs = 0;
#pragma unroll
      for (int hh = 0; hh < SPLIT; ++hh) cs += csum[hh][kb][i];
      aG[jm][3] += cs + static_cast<TG>(GateUnits<OpT>::ex(Gc)) * hdh;
    }
  }
  {
    const float pq = transpose_sum16<4 * MR>(vq), pk = transpose_sum16<4 * MR>(vk);
    const int j = i % (4 * MR), m = row_block(j / 4);
    if (i < 4 * MR && m < NB) {
      rowp[0][kb][16 * m + 4 * g + j % 4] = pq;
      rowp[1][kb][16 * m + 4 * g + j % 4] = pk;
    }
  }
  __syncthreads();  // all reads of GT as the cumulative gate are done
  // dG^T in LDS, in the VJP precision, over the cumulative gate (same type)
  TG* dGT = reinterpret_cast<TG*>(GT);
  TG* ptg = reinterpret_cast<TG*>(uni + OFF_S);
  TG* red = reinterpret_cast<TG*>(uni + OFF_S + sizeof(TG) * NT);
  // raw gate rows (then draw_g), [C][LDA]
  TI* xg_s = reinterpret_cast<TI*>(uni + OFF_X);
  if constexpr (!PH) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + NT * j, r = e / NVR, c = (e % NVR) * VE;
      if (e < NV) *reinterpret_cast<VT*>(xg_s + r * LDA + c) = xrow[j];
    }
  }
#pragma unroll
  for (int jm = 0; jm < MR; ++jm) {
    const int m = row_block(jm);
    if (m >= NB) break;
    {
      // rows 16m + 4g .. + 3 of this lane's channel, one vector store
      typedef std::conditional_t<sizeof(TG) == 4, f32x4, f64x4> TG4;
      TG4 v;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = aG[jm][rr];
      *reinterpret_cast<TG4*>(dGT + kk * LDG + 16 * m + 4 * g) = v;
    }
  }
  __syncthreads();
  {
    // reverse inclusive cumulative sum over rows, per channel (fixed order)
    constexpr int parts = NT / D, rp = C / parts;
    static_assert(C % parts == 0, "reverse cumulative sum layout");
    const int col = tid % D, part = tid / D;
    TG v[rp];
#pragma unroll
    for (int j = 0; j < rp; ++j) v[j] = dGT[col * LDG + part * rp + j];
    TG run = 0;
#pragma unroll
    for (int j = rp - 1; j >= 0; --j) {
      run += v[j];
      v[j] = run;
    }
    ptg[part * D + col] = run;
    __syncthreads();
    TG off = 0;
    for (int p2 = part + 1; p2 < parts; ++p2) off += ptg[p2 * D + col];
#pragma unroll
    for (int j = 0; j < rp; ++j) dGT[col * LDG + part * rp + j] = v[j] + off;
    if (tid < 2 * C) {
      const int which = tid / C, r = tid % C;
      float acc = 0.f;
      for (int k2 = 0; k2 < NKB; ++k2) acc += rowp[which][k2][r];
      rsum[which][r] = acc;
    }
    __syncthreads();
  }

  // ---- S8: prologue VJP and outputs. The gate map's VJP consumes the raw
  // gate loads before the first store of the phase (a load waited for after
  // a store would also wait for the store).
  {
    // the gate map's VJP and the gate-parameter sums run in the VJP precision
    // (fp64 for fp32 problems: the dA_log sum cancels heavily)
    TG pdt = 0, pA = 0;
    float dxv[PER];
    // dx = dg/dx and dA = dg/dA times dgv, for a raw gate plus bias xb
    auto gate_vjp = [&](TG xb, TG dgv, TG& dx, TG& dA) {
      if (d.gate_mode == 0) {
        // g = L sigmoid(z), z = e^A (x + b): dg/dx = e^A L s (1 - s), dg/dA = z L s (1 - s)
        const TG z = eat * xb, sz = VJ::sig(z);
        const TG dz = dgv * static_cast<TG>(d.lb) * sz * (1 - sz);
        dx = dz * eat;
        dA = dz * z;
      } else {
        // g = -e^A softplus(x + b) above the bound: dg/dx = -e^A sigmoid(x + b),
        // dg/dA = g; no gradient where the bound holds
        const TG c = -eat * softplus_t<TG>(xb);
        const bool act = c > static_cast<TG>(d.lb);
        dx = act ? -dgv * eat * VJ::sig(xb) : TG(0);
        dA = act ? dgv * c : TG(0);
      }
    };
    if constexpr (PH) {
      // one raw value per row: TPR threads share row hr, and the row's dG
      // summed over all channels (fixed order: a run of D / TPR channels per
      // thread, then a butterfly over the row's TPR lanes) drives the gate
      // map's VJP once
      constexpr int TPR = NT / C;
      static_assert(NT % C == 0 && D % TPR == 0 && TPR <= 64, "per-head gate VJP layout");
      const int hr = tid / TPR;
      const TI* xr = static_cast<const TI*>(in.g) + L.t0 * d.H + h;
      const uint32_t xhead = load_bits<TI>(xr + static_cast<size_t>(hr < L.len ? hr : L.len - 1) * d.H);
      dbias = in.dt_bias[h];
      TG sg = 0;
#pragma unroll
      for (int j = 0; j < D / TPR; ++j) sg += dGT[((tid % TPR) * (D / TPR) + j) * LDG + hr];
#pragma unroll
      for (int o = TPR / 2; o > 0; o >>= 1) sg += __shfl_xor(sg, o, kWave);
      const bool ok = hr < L.len && tid % TPR == 0;
      TG dx, dA;
      gate_vjp(static_cast<TG>(bits_to_f<TI>(xhead)) + static_cast<TG>(dbias), ok ? sg : TG(0),
               dx, dA);
      if (ok) dg[(L.t0 + hr) * d.H + h] = from_f<TI>(static_cast<float>(dx));
      pdt = dx;
      pA = dA;
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + NT * j, r = e / D, kc = e % D;
        const bool ok = e < C * D && r < L.len;
        const TG xb = static_cast<TG>(to_f(xg_s[(r < C ? r : 0) * LDA + kc])) + static_cast<TG>(dbias);
        const TG dgv = ok ? static_cast<TG>(dGT[kc * LDG + (r < C ? r : 0)]) : TG(0);
        TG dx, dA;
        gate_vjp(xb, dgv, dx, dA);
        dxv[j] = static_cast<float>(dx);
        pdt += dx;
        pA += dA;
      }
    }
    TI* dqo = dq + L.t0 * ts + hoff;
    TI* dko = dk + L.t0 * ts + hoff;
#pragma unroll
    for (int jm = 0; jm < MR; ++jm) {
      const int m = row_block(jm);
      if (m >= NB) break;
      const int r0 = 16 * m + 4 * g;
      const f32x4 q4 = tile4(qT, r0), k4 = tile4(kT, r0), rq4 = sc4(rq, r0), rk4 = sc4(rk, r0);
      f32x4 vq, vk;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = r0 + rr;
        const float qd = rsum[0][r], kd = rsum[1][r];
        const float qbar = q4[rr] * rq4[rr];
        const float khat_ = k4[rr] * rk4[rr];
        vq[rr] = rqs[r] * (aq[jm][rr] - qbar * qd);
        vk[rr] = rk[r] * (ak[jm][rr] - khat_ * kd);
      }
      // lane i = 4a + c then holds row r0 + c of channels 16 kb + 4a .. + 3:
      // one 4-element store per output instead of four scattered elements
      vq = quad_transpose(vq);
      vk = quad_transpose(vk);
      const int r = r0 + (i & 3), c0 = 16 * kb + (i & ~3);
      if (r < L.len) {
        store4<TI>(dqo + r * ts + c0, vq);
        store4<TI>(dko + r * ts + c0, vk);
      }
    }
    // draw_g over the raw gate: each element is read and rewritten by the
    // same thread
    if constexpr (!PH) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + NT * j, r = e / D, kc = e % D;
        if (e < C * D) xg_s[r * LDA + kc] = from_f<TI>(dxv[j]);
      }
    }
    // tid % D is this thread's channel for every e above (a per-head gate
    // leaves its row sums in these columns; the reduction adds them all)
    ptg[tid] = pdt;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pA += __shfl_xor(pA, o, kWave);
    if (lane == 0) red[w] = pA;
    if constexpr (!G2) {
      for (int r = tid; r < L.len; r += NT) {
        float db_ = 0.f;
        for (int w2 = 0; w2 < NW; ++w2) db_ += dbp[w2][r];
        dbeta[(L.t0 + r) * d.H + h] = from_f<TI>(db_ * be[r] * (1.f - be[r]));
      }
    }
    __syncthreads();
    double* part = partials + (static_cast<size_t>(cglob) * d.H + h) * (K + 1);
    if (tid < D) {
      TG s2 = 0;
      for (int p2 = 0; p2 < NT / D; ++p2) s2 += ptg[p2 * D + tid];
      part[tid] = static_cast<double>(s2);
    }
    if (tid == 0) {
      TG s2 = 0;
      for (int j = 0; j < NW; ++j) s2 += red[j];
      part[K] = static_cast<double>(s2);
    }
    TI* dgo = dg + L.t0 * ts + hoff;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int e = tid + NT * j, r = e / NVR, c = (e % NVR) * VE;
      if (e < NV && r < L.len) {
        if constexpr (!PH)
          *reinterpret_cast<VT*>(dgo + r * ts + c) = *reinterpret_cast<const VT*>(xg_s + r * LDA + c);
      }
    }
    if constexpr (G2) {
      // draw_b [T][H][K] from the per-channel accumulators
      TI* dbo = dbeta + L.t0 * ts + hoff;
#pragma unroll
      for (int jm = 0; jm < MR; ++jm) {
        const int m = row_block(jm);
        if (m >= NB) break;
        f32x4 vb;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) vb[rr] = ab[jm][rr];
        vb = quad_transpose(vb);  // as dq above
        const int r = 16 * m + 4 * g + (i & 3);
        if (r < L.len) store4<TI>(dbo + r * ts + 16 * kb + (i & ~3), vb);
      }
    }
  }
}

template <typename TI, int D, int C, bool PH, bool G2>
static hipError_t launch_cg(const Dims& d, const Inputs& in, const void* dO, int seg_begin,
                            int seg_chunks, const ChunkOps& ops, const SegStates& st, void* dq,
                            void* dk, void* dv, void* dg, void* dbeta, void* dw,
                            double* partials, hipStream_t s) {
  // GDN-2's fp32 erase-gate tile does not fit beside the others at fp32,
  // D = 64, C = 64 (the host rejects that combination)
  if constexpr (G2 && sizeof(TI) == 4 && D == 64 && C == 64) return hipErrorNotSupported;
  else hipLaunchKernelGGL((k_chunk_grad<TI, TI, D, C, PH, G2>), dim3(seg_chunks * d.H), dim3(D * 4 * grad_split<D>()), 0, s, d,
                     in, static_cast<const TI*>(dO), seg_begin, ops, st, static_cast<TI*>(dq),
                     static_cast<TI*>(dk), static_cast<TI*>(dv), static_cast<TI*>(dg),
                     static_cast<TI*>(dbeta), static_cast<TI*>(dw), partials);
  return hipGetLastError();
}

hipError_t launch_chunk_grad(int dtype, int D, int C, const Dims& d, const Inputs& in,
                             const void* dO, int seg_begin, int seg_chunks,
                             const ChunkOps& ops, const SegStates& st, void* dq, void* dk,
                             void* dv, void* dg, void* dbeta, void* dw, double* partials,
                             hipStream_t s) {
#define KDA_CG(TI, DD, CC)                                                                     \
  if (D == DD && C == CC)                                                                      \
    return d.gdn2 ? launch_cg<TI, DD, CC, false, true>(d, in, dO, seg_begin, seg_chunks, ops, st, \
                                                       dq, dk, dv, dg, dbeta, dw, partials, s)  \
           : d.gate_head ? launch_cg<TI, DD, CC, true, false>(d, in, dO, seg_begin, seg_chunks, ops, st, \
                                                     dq, dk, dv, dg, dbeta, dw, partials, s)    \
                       : launch_cg<TI, DD, CC, false, false>(d, in, dO, seg_begin, seg_chunks, ops, \
                                                      st, dq, dk, dv, dg, dbeta, dw, partials, s);
  if (dtype == 0) {
    KDA_CG(float, 64, 16) KDA_CG(float, 64, 32) KDA_CG(float, 64, 64)
    KDA_CG(float, 128, 16) KDA_CG(float, 128, 32)
  } else {
    KDA_CG(bf16, 64, 32) KDA_CG(bf16, 64, 64) KDA_CG(bf16, 128, 32) KDA_CG(bf16, 128, 64)
  }
#undef KDA_CG
  return hipErrorInvalidValue;
}

// dA_log[h] and ddt_bias[h, :] from per-chunk partials (fp64). Block (h, kg)
// covers 64 columns of head h; its four waves sum interleaved chunk subsets
// in order and the four results are added in wave order (deterministic).
__global__ void __launch_bounds__(256) k_gate_reduce(int D, int H, int n_chunks,
                                                     const double* partials, float* dA_log,
                                                     float* ddt_bias) {
  __shared__ double red[4][64];
  const int h = blockIdx.x, l = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int k = blockIdx.y * 64 + l;
  double s = 0.0;
  if (k <= D) {
#pragma unroll 8
    for (int c = part; c < n_chunks; c += 4) s += partials[(static_cast<size_t>(c) * H + h) * (D + 1) + k];
  }
  red[part][l] = s;
  __syncthreads();
  if (part == 0 && k <= D) {
    const double t = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
    if (k < D) ddt_bias[static_cast<size_t>(h) * D + k] = static_cast<float>(t);
    else dA_log[h] = static_cast<float>(t);
  }
}

// The per-head gate's dA_log[h] and ddt_bias[h]: block h of 512 threads.
// Column k of the partials (k <= D) is summed by four threads over the
// chunks c = part, part + 4, ... in order; the four parts are added in part
// order, then thread 0 adds the D gate columns in order (deterministic).
__global__ void __launch_bounds__(512) k_gate_reduce_head(int D, int H, int n_chunks,
                                                          const double* partials, float* dA_log,
                                                          float* ddt_bias) {
  __shared__ double red[4][129];
  const int h = blockIdx.x, part = threadIdx.x >> 7;
  for (int k = threadIdx.x & 127; k <= D; k += 128) {
    double s = 0.0;
#pragma unroll 8
    for (int c = part; c < n_chunks; c += 4) s += partials[(static_cast<size_t>(c) * H + h) * (D + 1) + k];
    red[part][k] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < D; ++k) t += ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
    ddt_bias[h] = static_cast<float>(t);
    dA_log[h] = static_cast<float>(((red[0][D] + red[1][D]) + red[2][D]) + red[3][D]);
  }
}

hipError_t launch_gate_reduce(int D, int H, int n_chunks, int gate_head,
                              const double* partials, float* dA_log, float* ddt_bias,
                              hipStream_t s) {
  if (gate_head)
    hipLaunchKernelGGL(k_gate_reduce_head, dim3(H), dim3(512), 0, s, D, H, n_chunks, partials,
                       dA_log, ddt_bias);
  else
    hipLaunchKernelGGL(k_gate_reduce, dim3(H, (D + 1 + 63) / 64), dim3(256), 0, s, D, H,
                       n_chunks, partials, dA_log, ddt_bias);
  return hipGetLastError();
}

}  // namespace kda
