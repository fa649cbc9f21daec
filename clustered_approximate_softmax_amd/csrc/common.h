// Shared device/host definitions for the MuSe HIP library (gfx950 / CDNA4).
//
// MFMA convention used by every kernel: v_mfma_f32_16x16x32_bf16.
//   lane l, column n = l % 16, lane group g = l / 16 (0..3)
//   A operand (16 x 32): lane holds A[row = l%16][k-slot 8g..8g+7]
//   B operand (32 x 16): lane holds B[k-slot 8g..8g+7][col = l%16]
//   C/D (16 x 16):       lane holds D[row = 4g + i][col = l%16], i = 0..3
// The k-slots of A and B pair up by (g, j), so any one-to-one map from
// slots to the contraction index works as long as both operands use it.
// When a product's B operand is built from a previous MFMA result held in
// registers, the 32 contraction indices of two 16-row result tiles are
// mapped as slot(8g + j) = 4g + j (j < 4) and 16 + 4g + (j - 4) (j >= 4);
// the matching A operand then reads two 4-element runs from LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MUSE_MAXLEV 32
#define MUSE_MAXC 256

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

namespace muse {

// ---------------------------------------------------------------------------
// Problem plan.  One plan describes every acausal MuSe problem of a call:
// acausal: one problem per head with queries and keys = all N rows;
// causal: level l has span m = block * 2^l and segments t with
// 2mt + m < N; keys are rows [2mt, 2mt + m), queries rows
// [2mt + m, min(2mt + 2m, N)).  (Hierarchical block decomposition of the
// causal case: newx.sg page, Abstract.)
// ---------------------------------------------------------------------------
// C is the storage count of every per-cluster array, max(cq, ck): the
// side with fewer clusters simply has empty clusters beyond its own count.
struct Plan {
  int32_t B, Hq, Hkv, N, D, C, Cq, Ck;
  int32_t nlev, P;          // levels, problems per head
  int32_t causal, blk, iters, topk, k1w, dipole;   // dipole: 0 monopole, 1 dipole, 2 exact tilt
  int32_t warm;             // 1: k-means starts from the centroids already in the state
  int32_t v4;               // 1: causal spatial blocks with accumulated summaries (one problem per head)
  int32_t nb, topk2, k2w;   // v4: blocks, retrieved blocks per retrieved cluster (and its storage width)
  float scale;
  int32_t lev_m[MUSE_MAXLEV];
  int32_t lev_nseg[MUSE_MAXLEV];
  int32_t lev_pfirst[MUSE_MAXLEV + 1];
};

struct Geom {
  int lev, k0, kn, q0, qn;
};

__host__ __device__ inline Geom prob_geom(const Plan& pl, int p) {
  Geom g;
  int lev = 0;
  while (lev + 1 < pl.nlev && pl.lev_pfirst[lev + 1] <= p) ++lev;
  g.lev = lev;
  if (!pl.causal || pl.v4) {
    g.k0 = 0; g.kn = pl.N; g.q0 = 0; g.qn = pl.N;
    return g;
  }
  int t = p - pl.lev_pfirst[lev];
  int m = pl.lev_m[lev];
  g.k0 = t * 2 * m;
  g.kn = m;
  g.q0 = g.k0 + m;
  g.qn = min(m, pl.N - g.q0);
  return g;
}

// One side (queries or keys) of the clustering problems of a call.
struct CSet {
  const void* X;        // [heads][N][D] in the input dtype
  int32_t heads;        // B*Hq or B*Hkv
  int32_t is_q;         // 1: query geometry (q0, qn), 0: key geometry
  const int32_t* init;  // [heads][P][this set's C] or null (floor(c n / C_eff))
  int32_t* labels;      // [nlev][heads][N]
  int32_t* perm;        // [nlev][heads][N]: sorted position -> row
  int32_t* offs;        // [heads][P][C+1], relative to the problem start
  float* cent;          // [heads][P][C][D] k-means centroids
  int32_t C;            // clusters of this set (cq or ck; at most the storage count Plan::C)
};

__host__ __device__ inline void cset_rows(const Plan& pl, const CSet& s, int p, int& lev, int& r0,
                                          int& n) {
  Geom g = prob_geom(pl, p);
  lev = g.lev;
  if (s.is_q) { r0 = g.q0; n = g.qn; } else { r0 = g.k0; n = g.kn; }
}

// ---------------------------------------------------------------------------
// bf16 helpers (round to nearest even; inputs are finite)
// ---------------------------------------------------------------------------
// The value of lane l ^ 16 (or l ^ 32) of a wave, through the lane-swap
// instructions (VALU; no LDS round trip).  With the same register in both
// operands, the swap leaves the values of lanes l & ~B and l | B in its two
// results on every lane l (B = 16 or 32); the partner's is the other one.
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float lane_xor16(float x) { return __uint_as_float(lane_xor16(__float_as_uint(x))); }
__device__ __forceinline__ float lane_xor32(float x) { return __uint_as_float(lane_xor32(__float_as_uint(x))); }
__device__ __forceinline__ int lane_xor16(int x) { return (int)lane_xor16((uint32_t)x); }
__device__ __forceinline__ int lane_xor32(int x) { return (int)lane_xor32((uint32_t)x); }
// max of the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same on all four)
__device__ __forceinline__ float max4_lanes(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// fp32 -> bf16, round to nearest even (the hardware conversion; the values
// converted here are finite)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// two floats -> packed bf16 pair, a in the low half (one hardware conversion,
// the same rounding as f2bf)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// x = hi + mid + lo with each part bf16 (24 significant bits in total).
__device__ __forceinline__ void split3(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  hi = f2bf(x);
  float r = x - bf2f(hi);
  mid = f2bf(r);
  lo = f2bf(r - bf2f(mid));
}

template <int NS>
__device__ __forceinline__ void split_store(float x, uint16_t* dst, int split_stride) {
  if (NS == 1) {
    dst[0] = f2bf(x);
  } else {
    uint16_t a, b, c;
    split3(x, a, b, c);
    dst[0] = a;
    dst[split_stride] = b;
    dst[2 * split_stride] = c;
  }
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A.B with A and B given as NA / NB bf16 parts; the products kept
// are those with part-index sum < max(NA, NB) (all of them when one side
// is exact in bf16), smallest terms first.
template <int NA, int NB>
__device__ __forceinline__ f32x4 mfma_split(const u16x8* a, const u16x8* b, f32x4 acc) {
  constexpr int NM = NA > NB ? NA : NB;
#pragma unroll
  for (int sum = NM - 1; sum >= 0; --sum) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int j = sum - i;
      if (j >= 0 && j < NB) acc = mfma(as_bf(a[i]), as_bf(b[j]), acc);
    }
  }
  return acc;
}

// Load 8 consecutive input elements as NS bf16 parts.
template <typename TIn, int NS>
__device__ __forceinline__ void load8_split(const TIn* p, u16x8* out) {
  if constexpr (sizeof(TIn) == 2) {
    out[0] = *reinterpret_cast<const u16x8*>(p);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t h, m, l;
      split3(v[j], h, m, l);
      out[0][j] = h;
      if (NS > 1) { out[1][j] = m; out[2][j] = l; }
    }
  }
}

// 8 consecutive input elements as float.
template <typename TIn>
__device__ __forceinline__ void load8_f32(const TIn* p, float* v) {
  if constexpr (sizeof(TIn) == 2) {
    u16x8 h = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = bf2f(h[j]);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  }
}

template <typename TIn>
__device__ __forceinline__ float load1_f32(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) return bf2f(*reinterpret_cast<const uint16_t*>(p));
  else return *p;
}

template <typename TOut>
__device__ __forceinline__ void store1(TOut* p, float v) {
  if constexpr (sizeof(TOut) == 2) *reinterpret_cast<uint16_t*>(p) = f2bf(v);
  else *p = v;
}

// input element type tags
struct bf16_t { uint16_t v; };

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// wave-wide shuffles (64 lanes)
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

}  // namespace muse
