// Device helpers for the gfx950 KDA kernels: element conversion, 64-lane
// wavefront reductions and 16x16 MFMA tile products.
//
// Tile convention used by every kernel: a 16x16 output tile Y is held by one
// wavefront as an f32x4 per lane; lane l = 16*g + i holds Y[4*g + r][i] for
// r = 0..3 (the CDNA 16x16 accumulator layout). Products are written "NT":
//   Y[m][n] = sum_kk A[m][kk] * B[n][kk]
// with both operands stored kk-contiguous, so each lane reads its k-slots
// (8 consecutive bf16, or 1 fp32) with one vector load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }

// Raw element bits held in a full register. A 16-bit load that fills only
// half a register would depend on the register's old contents (and make the
// wave wait for earlier loads); these loads zero-extend instead.
template <typename T>
__device__ __forceinline__ uint32_t load_bits(const T* p);
template <>
__device__ __forceinline__ uint32_t load_bits<bf16>(const bf16* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
template <>
__device__ __forceinline__ uint32_t load_bits<float>(const float* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
template <typename T>
__device__ __forceinline__ float bits_to_f(uint32_t b);
template <>
__device__ __forceinline__ float bits_to_f<bf16>(uint32_t b) { return __uint_as_float(b << 16); }
template <>
__device__ __forceinline__ float bits_to_f<float>(uint32_t b) { return __uint_as_float(b); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// DPP lane move (a VALU operand modifier: no LDS traffic, unlike a shuffle).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N = 2, 4, 8, 16 or 32),
// every lane of a group receiving the group's sum: swaps within quads
// (quad_perm [1,0,3,2], [2,3,0,1]), then mirrors within 8 and 16 lanes
// (row_half_mirror, row_mirror); lanes 16 apart are combined by a shuffle.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "lane group size");
  if (N >= 2) x += dpp_mov<0xB1>(x);
  if (N >= 4) x += dpp_mov<0x4E>(x);
  if (N >= 8) x += dpp_mov<0x141>(x);
  if (N >= 16) x += dpp_mov<0x140>(x);
  if (N >= 32) x += __shfl_xor(x, 16, kWave);
  return x;
}

// N sums at once over each aligned group of 16 lanes (N = 1, 2, 4, 8 or 16
// values per lane): on return lane l holds its group's sum of v[l % N].
// Partners are taken in turn across the row mirror, the half-row mirror and
// the quad swaps by 2 and by 1 (each an involution that pairs lanes differing
// in lane bit 3, 2, 1, 0). While a lane holds fewer values than that level
// can split, it adds its partner's copy of every value; otherwise it keeps
// the half its lane bit selects and adds its partner's copy of that half, so
// the values halve level by level (recursive halving). Sixteen values take
// 45 lane moves and selects instead of the 64 moves of sixteen group_sum<16>
// calls, and every lane ends with a different sum.
template <int N, int CTRL, int BIT>
__device__ __forceinline__ void halving_level(float (&a)[16], int l) {
  if constexpr (2 * BIT > N) {
#pragma unroll
    for (int j = 0; j < N; ++j) a[j] += dpp_mov<CTRL>(a[j]);
  } else {
    constexpr int H = N / 2;
    const bool up = (l & BIT) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float keep = up ? a[j + H] : a[j], send = up ? a[j] : a[j + H];
      a[j] = keep + dpp_mov<CTRL>(send);
    }
  }
}
// 4x4 transpose within each quad of lanes (lanes 4a .. 4a + 3): lane c of a
// quad holds x[0..3] on entry and, on return, at index k what lane k held
// at index c. Two block-swap steps, with the partner lane c ^ 1 and then
// c ^ 2 (quad_perm [1,0,3,2] and [2,3,0,1]): at index r a lane takes the
// partner's value at index r ^ b where bit b of r and of c differ.
template <int CTRL, int B>
__device__ __forceinline__ f32x4 quad_swap_step(const f32x4& x, int c) {
  f32x4 t, y;
#pragma unroll
  for (int r = 0; r < 4; ++r) t[r] = dpp_mov<CTRL>(x[r]);
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = ((r & B) != (c & B)) ? t[r ^ B] : x[r];
  return y;
}
__device__ __forceinline__ f32x4 quad_transpose(const f32x4& x) {
  const int c = static_cast<int>(threadIdx.x) & 3;
  return quad_swap_step<0x4E, 2>(quad_swap_step<0xB1, 1>(x, c), c);
}

template <int N>
__device__ __forceinline__ float transpose_sum16(const float (&v)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "values per lane");
  float a[16];
#pragma unroll
  for (int j = 0; j < N; ++j) a[j] = v[j];
  const int l = static_cast<int>(threadIdx.x) & 15;
  constexpr int N1 = 16 > N ? N : N / 2;
  constexpr int N2 = 8 > N1 ? N1 : N1 / 2;
  constexpr int N3 = 4 > N2 ? N2 : N2 / 2;
  halving_level<N, 0x140, 8>(a, l);
  halving_level<N1, 0x141, 4>(a, l);
  halving_level<N2, 0x4E, 2>(a, l);
  halving_level<N3, 0xB1, 1>(a, l);
  return a[0];
}

// Sum over the four lane groups g (lanes i, i+16, i+32, i+48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---------------------------------------------------------------- MFMA traits

template <typename OpT>
struct Mma;

// bf16 operands, fp32 accumulate: v_mfma_f32_16x16x32_bf16 (gfx950).
// Lane (i, g) supplies k-slots 8g..8g+7 of row i for A and of column i for B.
template <>
struct Mma<bf16> {
  static constexpr int KS = 32;  // reduction length per instruction
  static constexpr int KPL = 8;  // k-slots per lane
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  template <class F>
  static __device__ __forceinline__ frag make(F f) {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = static_cast<bf16>(f(j));
    return r;
  }
};

// fp32 operands: v_mfma_f32_16x16x4_f32. Lane (i, g) supplies k-slot g.
template <>
struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  template <class F>
  static __device__ __forceinline__ frag make(F f) { return f(0); }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Four consecutive values from raw bits (bf16: two words, low half first;
// fp32: four words), their raw load, and a four-value vector store (8 or 16
// bytes).
template <typename T>
__device__ __forceinline__ f32x4 unpack4(const uint32_t (&u)[4]) {
  if constexpr (sizeof(T) == 2) {
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                 __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
  } else {
    return f32x4{__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                 __uint_as_float(u[3])};
  }
}
template <typename T>
__device__ __forceinline__ void load4_raw(const T* p, uint32_t (&u)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    u[0] = x.x;
    u[1] = x.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    u[0] = x.x;
    u[1] = x.y;
    u[2] = x.z;
    u[3] = x.w;
  }
}
// A store with or without the non-temporal hint. NT = true suits a
// kernel's output that only a later kernel reads: the hint lets the line
// leave the caches rather than being kept for reuse that never comes, and the
// streaming kernels that consume it then run measurably faster.
template <bool NT, typename V>
__device__ __forceinline__ void vstore(V* p, const V& v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
template <typename T, bool NT = false>
__device__ __forceinline__ void store4(T* p, const f32x4& v) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 b;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) b[rr] = static_cast<bf16>(v[rr]);
    vstore<NT>(reinterpret_cast<bf16x4*>(p), b);
  } else {
    vstore<NT>(reinterpret_cast<f32x4*>(p), v);
  }
}

// Four values as 32-bit words of the storage type, rounded as store4 rounds
// them (bf16: two words, the lower-addressed value in the low half; fp32:
// four words).
template <typename T>
__device__ __forceinline__ void pack4(const f32x4& v, uint32_t (&w)[sizeof(T) == 2 ? 2 : 4]) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 b;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) b[rr] = static_cast<bf16>(v[rr]);
    const uint2 u = __builtin_bit_cast(uint2, b);
    w[0] = u.x;
    w[1] = u.y;
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) w[rr] = __float_as_uint(v[rr]);
  }
}

// Fragment-major operand arrays. An [R][S] matrix that is read as MFMA
// operand fragments (rows in blocks of 16, the reduction dimension S in
// pieces of KS) is stored one fragment after another: fragment (rb, sf) is
// 64 lane slots of KPL elements, slot (i, g) = i + 16 g holding row 16 rb + i,
// columns sf KS + g KPL .. + KPL - 1. A wave's fragment load is then one
// contiguous run of 64 KPL elements instead of 16 strided row pieces.
// R is a multiple of 16 and S of KS.
template <typename OpT>
struct FragMajor {
  using M = Mma<OpT>;
  // element (r, s)
  static __device__ __forceinline__ int off(int r, int s, int S) {
    return (((r >> 4) * (S / M::KS) + s / M::KS) * 64 + (r & 15) + 16 * ((s % M::KS) / M::KPL)) *
               M::KPL + s % M::KPL;
  }
  // the lane's slot of fragment (rb, sf)
  static __device__ __forceinline__ int frag(int rb, int sf, int S, int lane) {
    return ((rb * (S / M::KS) + sf) * 64 + lane) * M::KPL;
  }
  // elements (r, s0 .. s0 + 3), s0 a multiple of 4: contiguous for bf16
  // (within one slot), 16 slots apart for fp32
  static constexpr int kStep4 = M::KPL >= 4 ? 1 : 16;
  // Row-parity order (bf16): within each fragment the slot of (row i, piece
  // g) is placed at ((i >> 3) * 2 + (i & 1)) * 16 + ((i >> 1) & 3) * 4 + g,
  // so that four rows of one parity with all their pieces fill 256
  // contiguous bytes. A reader still covers one whole fragment per wave; a
  // writer holding rows 2p + h (h fixed per store) writes whole lines. fp32
  // fragments keep the plain order.
  static __device__ __forceinline__ int pslot(int i, int g) {
    if constexpr (M::KPL >= 4) return (((i >> 3) << 1) + (i & 1)) * 16 + ((i >> 1) & 3) * 4 + g;
    else return i + 16 * g;
  }
  static __device__ __forceinline__ int off_p(int r, int s, int S) {
    if constexpr (M::KPL >= 4)
      return (((r >> 4) * (S / M::KS) + s / M::KS) * 64 + pslot(r & 15, (s % M::KS) / M::KPL)) * M::KPL +
             s % M::KPL;
    else return off(r, s, S);
  }
  static __device__ __forceinline__ int frag_p(int rb, int sf, int S, int lane) {
    return ((rb * (S / M::KS) + sf) * 64 + pslot(lane & 15, lane >> 4)) * M::KPL;
  }
};

template <typename OpT, bool NT = false>
__device__ __forceinline__ void store4_fm(OpT* a, int r, int s0, int S, const f32x4& v) {
  OpT* p = a + FragMajor<OpT>::off(r, s0, S);
  if constexpr (FragMajor<OpT>::kStep4 == 1) {
    store4<OpT, NT>(p, v);
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) vstore<NT>(p + 16 * rr, static_cast<OpT>(v[rr]));
  }
}
template <typename OpT>
__device__ __forceinline__ void load4_fm_raw(const OpT* a, int r, int s0, int S, uint32_t (&u)[4]) {
  const OpT* p = a + FragMajor<OpT>::off(r, s0, S);
  if constexpr (FragMajor<OpT>::kStep4 == 1) {
    load4_raw<OpT>(p, u);
  } else {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) u[rr] = __float_as_uint(p[16 * rr]);
  }
}

// Whether fragment (row block rb, reduction piece sf) of the fragment-major
// T^T (T lower triangular, so T^T[r][s] = 0 for s < r) holds a nonzero:
// its last column reaches the block's first row.
template <typename OpT>
__device__ __forceinline__ bool tt_frag_nonzero(int rb, int sf) {
  return Mma<OpT>::KS * (sf + 1) > 16 * rb;
}

// acc += sum_{kk in [k_lo, k_hi)} A[i][kk] * B[i'][kk] for one 16x16 tile.
// A and B point at the first row of the tile; lda/ldb are row strides in
// elements. k_lo and k_hi - k_lo are multiples of Mma<OpT>::KS.
template <typename OpT>
__device__ __forceinline__ f32x4 tile_nt(f32x4 acc, const OpT* A, int lda, const OpT* B,
                                         int ldb, int k_lo, int k_hi, int lane) {
  using M = Mma<OpT>;
  const int i = lane & 15, g = lane >> 4;
  const OpT* a = A + i * lda + g * M::KPL;
  const OpT* b = B + i * ldb + g * M::KPL;
  for (int k0 = k_lo; k0 < k_hi; k0 += M::KS) acc = M::mma(M::load(a + k0), M::load(b + k0), acc);
  return acc;
}

// Round a reduction bound up to the instruction's reduction length.
template <typename OpT>
__device__ __forceinline__ constexpr int kround(int x) {
  return (x + Mma<OpT>::KS - 1) / Mma<OpT>::KS * Mma<OpT>::KS;
}

// Sequence lookup: the sequence n containing global chunk c (coff[n] <= c <
// coff[n+1]); empty sequences have coff[n] == coff[n+1] and are skipped.
__device__ __forceinline__ int find_seq(const int32_t* coff, int N, int c) {
  int lo = 0, hi = N;  // answer in [0, N)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (coff[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace kda
