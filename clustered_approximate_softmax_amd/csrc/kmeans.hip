// Lloyd k-means of queries and of keys, each in its own space, per head
// and per problem (gist.science page, Technical Summary, Core Mechanisms,
// Bidirectional Semantic Clustering), plus the cluster-contiguous
// permutation of every problem.
//
// Assignment: d_c = |mu_c|^2 - 2 x.mu_c is screened with one bf16 MFMA
// pass (A = bf16 centroids, B = bf16 points).  The screening error is at
// most 2^-8 |x| |mu_c| (bf16 inputs; 2^-7 for fp32 inputs), so every
// cluster within twice that bound of the screened minimum is a candidate
// for the true nearest centroid.  A point with one candidate is decided;
// otherwise the candidates' distances sum_e (x_e - mu_ce)^2 are computed
// in fp32 and the lowest index wins ties.
//
// Update: partial sums per cluster are a one-hot x points MFMA product
// (exact products, fp32 accumulation in a fixed order), so centroids are
// deterministic.  Problems up to a size limit run all iterations inside
// one workgroup (km_local); larger ones use one launch per iteration of
// km_assign over point chunks followed by km_reduce.
#include "common.h"
#include "launch.h"

namespace muse {

constexpr int KM_NT = 256;  // threads per workgroup (4 waves)

template <typename TIn, int D>
struct KmShape {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  // bf16 inputs: centroid operand in two bf16 parts (hi, lo of -2 mu); the
  // padding slots D..D+7 of the hi rows carry the squared norm for one extra
  // k-step.  fp32 inputs: bf16 mu
  static constexpr int NP = NS == 1 ? 2 : 1;
  static constexpr int MUP = D + 8;  // padded centroid row (bf16 elements)
  static constexpr int SUB = NS == 1 ? 128 : (D == 128 ? 64 : 256);
  static constexpr int XTP = SUB + 8;  // padded transposed row
  static constexpr int G16 = SUB / 64; // 16-point groups per wave per sub-tile
};

template <typename TIn, int D, int CT>
struct alignas(16) KmSmem {
  using S = KmShape<TIn, D>;
  // fp32 centroids for the refinement step, kept in LDS when small
  static constexpr bool KEEP32 = S::NS == 3 && CT * 16 * D * 4 <= 32768;
  float mu32[KEEP32 ? CT * 16 : 1][D + 4];
  uint16_t mu_hat[S::NP][CT * 16][S::MUP];
  float mu_norm[CT * 16];
  uint16_t xt[S::NS][D][S::XTP];
  uint16_t lab[S::SUB];      // labels of the sub-tile (0xffff: no point)
  int32_t cnt[MUSE_MAXC];
  int32_t wcnt[4][MUSE_MAXC];
  float red[8];
};

// Screening operands from fp32 centroid rows (global or LDS): bf16 rows
// (two parts of -2 mu for bf16 inputs, with the squared norm in an extra
// k-step), fp32 squared norms and the largest norm.  Norms are 8-element
// partial sums combined by shuffles in a fixed order.
template <typename TIn, int D, int CT, typename SM>
__device__ void km_centroids(SM& sm, const float* src, int stride, bool write32, int Ceff, float& Rmax) {
  using S = KmShape<TIn, D>;
  constexpr int TPC = D / 8;
  const int tid = threadIdx.x;
  float mx = 0.f;
  for (int idx = tid; idx < CT * 16 * TPC; idx += KM_NT) {
    const int c = idx / TPC, e0 = (idx % TPC) * 8;
    float v[8];
    if (c < Ceff) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + (size_t)c * stride + e0);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + (size_t)c * stride + e0 + 4);
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    u16x8 h, l;
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      part = fmaf(v[j], v[j], part);
      if constexpr (S::NS == 1) {
        const float m2 = -2.f * v[j];
        h[j] = f2bf(m2);
        l[j] = f2bf(m2 - bf2f(h[j]));
      } else {
        h[j] = f2bf(v[j]);
      }
    }
    *reinterpret_cast<u16x8*>(&sm.mu_hat[0][c][e0]) = h;
    if constexpr (S::NS == 1) *reinterpret_cast<u16x8*>(&sm.mu_hat[S::NP - 1][c][e0]) = l;
    if constexpr (SM::KEEP32) {
      if (write32) {
        *reinterpret_cast<f32x4*>(&sm.mu32[c][e0]) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(&sm.mu32[c][e0 + 4]) = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
#pragma unroll
    for (int m = 1; m < TPC; m <<= 1) part += __shfl_xor(part, m, 64);
    if (idx % TPC == 0) {
      sm.mu_norm[c] = c < Ceff ? part : INFINITY;
      if (c < Ceff) mx = fmaxf(mx, part);
      if constexpr (S::NS == 1) {
        // extra k-step: slots (1, |mu|^2 hi, |mu|^2 lo, 1) pair with the point's
        // (|x|^2 hi, 1, 1, |x|^2 lo) in lane group 0 (the other groups' point
        // slots are zero); absent clusters get a huge finite norm
        const float nn = c < Ceff ? part : 1e30f;
        u16x8 e = {0, 0, 0, 0, 0, 0, 0, 0};
        e[0] = 0x3F80;
        e[1] = f2bf(nn);
        e[2] = c < Ceff ? f2bf(nn - bf2f(e[1])) : (uint16_t)0;
        e[3] = 0x3F80;
        *reinterpret_cast<u16x8*>(&sm.mu_hat[0][c][D]) = e;
      }
    }
  }
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if ((tid & 63) == 0) sm.red[tid >> 6] = mx;
  __syncthreads();
  Rmax = sqrtf(fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3])));
}

template <typename TIn, int D, int CT>
__device__ void km_load_centroids(KmSmem<TIn, D, CT>& sm, const float* cent, int Ceff, float& Rmax) {
  km_centroids<TIn, D, CT>(sm, cent, D, true, Ceff, Rmax);
}

// Points of one sub-tile held in registers (raw input elements): lane
// (col, g) of wave w holds point w*SUB/4 + 16*grp + col, dims 32k+8g..+7.
template <typename TIn, int D>
struct XRegs {
  using S = KmShape<TIn, D>;
  using V8 = typename std::conditional<sizeof(TIn) == 2, u16x8, f32x8>::type;
  V8 x[S::G16][D / 32];
};

template <typename TIn, int D>
__device__ __forceinline__ void km_fetch(XRegs<TIn, D>& xr, const TIn* Xp, int sub0, int nvalid) {
  using S = KmShape<TIn, D>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int grp = 0; grp < S::G16; ++grp) {
    const int pl = w * (S::SUB / 4) + grp * 16 + col;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      if (pl < nvalid) {
        const TIn* src = Xp + (size_t)(sub0 + pl) * D + 32 * k + 8 * g;
        if constexpr (sizeof(TIn) == 2) {
          xr.x[grp][k] = *reinterpret_cast<const u16x8*>(src);
        } else {
          f32x4 a0 = *reinterpret_cast<const f32x4*>(src), a1 = *reinterpret_cast<const f32x4*>(src + 4);
          xr.x[grp][k] = f32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
      } else {
        xr.x[grp][k] = typename XRegs<TIn, D>::V8{};
      }
    }
  }
}

// median of three signed integers (one VALU instruction)
__device__ __forceinline__ int med3i(int a, int b, int c) {
  int r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Smallest two of {m1, m2, a, b} (m1 <= m2, all distinct) into m1, m2: the
// second smallest is min(m2, med3(m1, a, b)).
__device__ __forceinline__ void top2_pair(int& m1, int& m2, int a, int b) {
  m2 = min(m2, med3i(m1, a, b));
  m1 = min(min(m1, a), b);
}

template <typename V8>
__device__ __forceinline__ float xval(const V8& v, int j) {
  if constexpr (sizeof(v[0]) == 2) return bf2f(v[j]);
  else return v[j];
}

// bf16 inputs.  Two-part screening: the point is exact in bf16 and
// -2 mu = hi + lo to 2^-16, so acc = |x|^2 + |mu|^2 - 2 x.mu (norms through
// the extra k-step) is the squared distance to about 2^-15 |x| |mu|.  Keys
// hold the distance bits with the low bits replaced by the cluster index
// (16t + i here, 4g added after the loop); the smallest two keys per point
// are tracked with min / med3 on signed integers (a distance rounded below
// zero orders first).  Points whose two best keys lie within the screening
// error of each other are decided by fp32 distances to the candidate
// clusters, lowest index on ties.
// Screening sums of 16 points (lane (col, g): point col) against the TB
// cluster tiles t0 .. t0+TB-1: every centroid fragment of the batch is read
// from LDS first, then the MFMAs run interleaved over TB independent
// accumulators (per accumulator: lo parts, hi parts, norm step, as before).
template <int D, int TB, typename SM, typename V8>
__device__ __forceinline__ void km_screen_batch(const SM& sm, const V8 (&x)[D / 32], const u16x8& bn, int t0,
                                                f32x4 (&acc)[TB]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  u16x8 flo[TB][KS], fhi[TB][KS], fnm[TB];
#pragma unroll
  for (int u = 0; u < TB; ++u) {
    const int row = 16 * (t0 + u) + col;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      flo[u][k] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[1][row][32 * k + 8 * g]);
      fhi[u][k] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[0][row][32 * k + 8 * g]);
    }
    fnm[u] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[0][row][D]);
  }
#pragma unroll
  for (int u = 0; u < TB; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int u = 0; u < TB; ++u) acc[u] = mfma(as_bf(flo[u][k]), as_bf(x[k]), acc[u]);
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int u = 0; u < TB; ++u) acc[u] = mfma(as_bf(fhi[u][k]), as_bf(x[k]), acc[u]);
#pragma unroll
  for (int u = 0; u < TB; ++u) acc[u] = mfma(as_bf(fnm[u]), as_bf(bn), acc[u]);
}

// The same screening sums for the two 16-point groups of a wave at once:
// each centroid fragment is read from LDS once and feeds both groups'
// MFMAs (every accumulator sees the same operations in the same order as
// in km_screen_batch, so the sums are identical).
template <int D, int TB, typename SM, typename V8>
__device__ __forceinline__ void km_screen_batch2(const SM& sm, const V8 (&x)[2][D / 32], const u16x8 (&bn)[2],
                                                 int t0, f32x4 (&acc)[2][TB]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  u16x8 flo[TB][KS], fhi[TB][KS], fnm[TB];
#pragma unroll
  for (int u = 0; u < TB; ++u) {
    const int row = 16 * (t0 + u) + col;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      flo[u][k] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[1][row][32 * k + 8 * g]);
      fhi[u][k] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[0][row][32 * k + 8 * g]);
    }
    fnm[u] = *reinterpret_cast<const u16x8*>(&sm.mu_hat[0][row][D]);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int u = 0; u < TB; ++u) acc[q][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int u = 0; u < TB; ++u)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q][u] = mfma(as_bf(flo[u][k]), as_bf(x[q][k]), acc[q][u]);
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int u = 0; u < TB; ++u)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q][u] = mfma(as_bf(fhi[u][k]), as_bf(x[q][k]), acc[q][u]);
#pragma unroll
  for (int u = 0; u < TB; ++u)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[q][u] = mfma(as_bf(fnm[u]), as_bf(bn[q]), acc[q][u]);
}

// Stage group grp of the wave's points (transposed, in LDS) and form its
// squared norm and the point side of the norm k-step.
template <typename TIn, int D, typename SM>
__device__ __forceinline__ void km_stage_group(SM& sm, const XRegs<TIn, D>& xr, int grp, float& xsq_out,
                                               u16x8& bn) {
  using S = KmShape<TIn, D>;
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int pl = w * (S::SUB / 4) + grp * 16 + col;
  float xsq = 0.f;
#pragma unroll
  for (int k = 0; k < KS; ++k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = xval(xr.x[grp][k], j);
      xsq = fmaf(v, v, xsq);
      sm.xt[0][32 * k + 8 * g + j][pl] = xr.x[grp][k][j];
    }
  }
  xsq += __shfl_xor(xsq, 16, 64);
  xsq += __shfl_xor(xsq, 32, 64);
  xsq_out = xsq;
  bn = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  if (g == 0) {
    const uint16_t xh = f2bf(xsq);
    bn[0] = xh;
    bn[1] = 0x3F80;
    bn[2] = 0x3F80;
    bn[3] = f2bf(xsq - bf2f(xh));
  }
}

// Decide the label of each point of group grp from its screened best and
// runner-up keys (this lane's share; merged over the wave here), refine the
// near-ties in fp32, write the label to LDS and to glab.
template <typename TIn, int D, int CT, typename SM>
__device__ __forceinline__ void km_finish_group(SM& sm, const XRegs<TIn, D>& xr, int grp, int m1, int m2,
                                                float xsq, const u16x8& bn, int sub0, int nvalid,
                                                const float* cent, int Ceff, float Rmax, int32_t* glab) {
  constexpr int TB = CT < 4 ? CT : 4;
  using S = KmShape<TIn, D>;
  constexpr int KS = D / 32;
  constexpr int IB = CT <= 8 ? 7 : 8;
  constexpr int KMASK = ~((1 << IB) - 1);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int pl = w * (S::SUB / 4) + grp * 16 + col;
  const bool valid = pl < nvalid;
  // the two-candidate shortcut below is taken from four cluster tiles up
  // (with fewer, its registers cost occupancy and the full scan is short)
  constexpr bool TWO = CT >= 4;
  m1 |= 4 * g;
  int m3 = 0;
  if constexpr (TWO) {
    m2 |= 4 * g;
    // merged over the lane groups: best m1, runner-up m2, and m3, a lower
    // bound on the third key (a group's unknown third is bounded below by
    // its runner-up); the third of two sorted triples is
    // min(a3, b3, max(a1, b2), max(a2, b1))
    m3 = m2;
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
      const int b1 = __shfl_xor(m1, m, 64), b2 = __shfl_xor(m2, m, 64), b3 = __shfl_xor(m3, m, 64);
      m3 = min(min(m3, b3), min(max(m1, b2), max(m2, b1)));
      m2 = min(max(m1, b1), min(m2, b2));
      m1 = min(m1, b1);
    }
  } else {
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
      const int b1 = __shfl_xor(m1, m, 64), b2 = __shfl_xor(m2, m, 64);
      m2 = min(max(m1, b1), min(m2, b2));
      m1 = min(m1, b1);
    }
  }
  int label = m1 & ((1 << IB) - 1);
  const float f1 = __int_as_float(m1 & KMASK), f2 = __int_as_float(m2 & KMASK);
  const float xn = sqrtf(xsq);
  // screening error (split residual, accumulation, norm split) plus key truncation
  const float trunc = IB == 7 ? 3.0517578125e-05f : 6.103515625e-05f;
  const float margin = 2.44140625e-4f * xn * Rmax + 1.220703125e-4f * (xsq + Rmax * Rmax) +
                       trunc * (fabsf(f1) + fabsf(f2));
  const bool need = valid && Ceff > 1 && (f2 - f1 <= margin);
  // The candidates (screened distance within f1 + margin) are exactly the
  // best and the runner-up when every other key is at least m3 >= 0 (keys of
  // non-negative distances order as the distances, and a key's distance bits
  // are at most its screened distance) with f3 beyond the threshold, and the
  // runner-up's screened distance (below f2 plus its truncation) is inside it.
  // (m3 = INT_MAX, a NaN pattern, means there is no third key.)
  const float thr = f1 + margin;
  const float f3 = __int_as_float(m3 & KMASK);
  const bool two = TWO && m3 >= 0 && !(f3 <= thr) && f2 + trunc * fabsf(f2) <= thr;
  if (TWO && !__any(need && !two)) {
    if (TWO && __any(need)) {
      // exact fp32 distances of the two candidates, both rows read together
      const int c1 = min(m1 & ((1 << IB) - 1), Ceff - 1), c2 = min(m2 & ((1 << IB) - 1), Ceff - 1);
      float mv1[KS][8], mv2[KS][8];
#pragma unroll
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (SM::KEEP32) {
            mv1[k][j] = sm.mu32[c1][32 * k + 8 * g + j];
            mv2[k][j] = sm.mu32[c2][32 * k + 8 * g + j];
          } else {
            mv1[k][j] = cent[(size_t)c1 * D + 32 * k + 8 * g + j];
            mv2[k][j] = cent[(size_t)c2 * D + 32 * k + 8 * g + j];
          }
        }
      float p1 = 0.f, p2 = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float d1 = xval(xr.x[grp][k], j) - mv1[k][j], d2 = xval(xr.x[grp][k], j) - mv2[k][j];
          p1 = fmaf(d1, d1, p1);
          p2 = fmaf(d2, d2, p2);
        }
      p1 += __shfl_xor(p1, 16, 64);
      p2 += __shfl_xor(p2, 16, 64);
      p1 += __shfl_xor(p1, 32, 64);
      p2 += __shfl_xor(p2, 32, 64);
      if (need) label = (p2 < p1 || (p2 == p1 && c2 < c1)) ? c2 : c1;
    }
  } else if (__any(need)) {
    // candidates within the margin; the screening MFMAs are recomputed by the
    // whole wave (an MFMA reads its operands from every lane, active or not)
    const float thr = f1 + margin;
    constexpr int NW = (CT * 16 + 63) / 64;
    unsigned long long cm[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q) cm[q] = 0ull;
    auto cands = [&](auto tbc, int t0) {
      constexpr int TBX = decltype(tbc)::value;
      f32x4 acc[TBX];
      km_screen_batch<D, TBX>(sm, xr.x[grp], bn, t0, acc);
#pragma unroll
      for (int u = 0; u < TBX; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * (t0 + u) + 4 * g + i;
          if (need && c < Ceff && acc[u][i] <= thr) cm[c >> 6] |= 1ull << (c & 63);
        }
    };
#pragma unroll
    for (int t0 = 0; t0 < CT; t0 += TB) {
      const int live = min(TB, (Ceff - 16 * t0 + 15) / 16);
      if (live > 2) cands(std::integral_constant<int, TB>{}, t0);
      else if (live == 2) cands(std::integral_constant<int, TB < 2 ? TB : 2>{}, t0);
      else if (live == 1) cands(std::integral_constant<int, 1>{}, t0);
    }
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      cm[q] |= __shfl_xor(cm[q], 16, 64);
      cm[q] |= __shfl_xor(cm[q], 32, 64);
    }
    // exact fp32 distances of the candidates (lanes of points that need no
    // refinement have an empty mask)
    float bd = INFINITY;
    int bc = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      unsigned long long mword = cm[q];
      while (mword) {
        const int c = 64 * q + __builtin_ctzll(mword);
        mword &= mword - 1;
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          float mv[8];
          if constexpr (SM::KEEP32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) mv[j] = sm.mu32[c][32 * k + 8 * g + j];
          } else {
            const float* mr = cent + (size_t)c * D + 32 * k + 8 * g;
#pragma unroll
            for (int j = 0; j < 8; ++j) mv[j] = mr[j];
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float df = xval(xr.x[grp][k], j) - mv[j];
            part = fmaf(df, df, part);
          }
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if (part < bd || (part == bd && c < bc)) { bd = part; bc = c; }
      }
    }
    if (need) label = bc;
  }
  if (g == 0) {
    sm.lab[pl] = valid ? (uint16_t)label : (uint16_t)0xffff;
    if (valid) glab[sub0 + pl] = label;
  }
}

// bf16 inputs: assignment of one sub-tile (two 16-point groups per wave).
// From four cluster tiles up (eight at D = 128), both groups are screened together so that
// every centroid fragment read from LDS feeds two MFMAs; with fewer, each
// group is screened on its own (fewer live registers, more workgroups).
template <typename TIn, int D, int CT, typename SM>
__device__ void km_assign_bf16(SM& sm, const XRegs<TIn, D>& xr, int sub0, int nvalid, const float* cent,
                               int Ceff, float Rmax, int32_t* glab) {
  constexpr int TB = CT < 4 ? CT : 4;   // cluster tiles per screening batch
  using S = KmShape<TIn, D>;
  constexpr int IB = CT <= 8 ? 7 : 8;
  constexpr int KMASK = ~((1 << IB) - 1);
  static_assert(S::G16 == 2, "two 16-point groups per wave");
  // (at D = 128 with four tiles the paired path would need more than 256 VGPRs)
  if constexpr (CT >= 4 && (D == 64 || CT >= 8)) {
    float xsq[2];
    u16x8 bn[2];
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) km_stage_group<TIn, D>(sm, xr, grp, xsq[grp], bn[grp]);
    int m1[2] = {0x7fffffff, 0x7fffffff}, m2[2] = {0x7fffffff, 0x7fffffff};
    // batches of two cluster tiles for both groups (the same four
    // accumulators in flight as four tiles of one group); a batch with one
    // live tile runs at that width (absent clusters carry a huge norm)
    auto keys = [&](auto tbc, int t0) __attribute__((always_inline)) {
      constexpr int TBX = decltype(tbc)::value;
      f32x4 acc[2][TBX];
      km_screen_batch2<D, TBX>(sm, xr.x, bn, t0, acc);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < TBX; ++u)
#pragma unroll
          for (int i = 0; i < 4; i += 2)
            top2_pair(m1[q], m2[q], (__float_as_int(acc[q][u][i]) & KMASK) | (16 * (t0 + u) + i),
                      (__float_as_int(acc[q][u][i + 1]) & KMASK) | (16 * (t0 + u) + i + 1));
    };
#pragma unroll
    for (int t0 = 0; t0 < CT; t0 += 2) {
      const int live = min(2, (Ceff - 16 * t0 + 15) / 16);
      if (live == 2) keys(std::integral_constant<int, 2>{}, t0);
      else if (live == 1) keys(std::integral_constant<int, 1>{}, t0);
    }
#pragma unroll
    for (int grp = 0; grp < 2; ++grp)
      km_finish_group<TIn, D, CT>(sm, xr, grp, m1[grp], m2[grp], xsq[grp], bn[grp], sub0, nvalid, cent, Ceff,
                                  Rmax, glab);
  } else {
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      float xsq;
      u16x8 bn;
      km_stage_group<TIn, D>(sm, xr, grp, xsq, bn);
      int m1 = 0x7fffffff, m2 = 0x7fffffff;
      // batches of up to TB cluster tiles; a batch with 1 or 2 live tiles
      // runs at that width (rows of absent clusters carry a huge norm)
      auto keys = [&](auto tbc, int t0) __attribute__((always_inline)) {
        constexpr int TBX = decltype(tbc)::value;
        f32x4 acc[TBX];
        km_screen_batch<D, TBX>(sm, xr.x[grp], bn, t0, acc);
#pragma unroll
        for (int u = 0; u < TBX; ++u)
#pragma unroll
          for (int i = 0; i < 4; i += 2)
            top2_pair(m1, m2, (__float_as_int(acc[u][i]) & KMASK) | (16 * (t0 + u) + i),
                      (__float_as_int(acc[u][i + 1]) & KMASK) | (16 * (t0 + u) + i + 1));
      };
#pragma unroll
      for (int t0 = 0; t0 < CT; t0 += TB) {
        const int live = min(TB, (Ceff - 16 * t0 + 15) / 16);
        if (live > 2) keys(std::integral_constant<int, TB>{}, t0);
        else if (live == 2) keys(std::integral_constant<int, TB < 2 ? TB : 2>{}, t0);
        else if (live == 1) keys(std::integral_constant<int, 1>{}, t0);
      }
      km_finish_group<TIn, D, CT>(sm, xr, grp, m1, m2, xsq, bn, sub0, nvalid, cent, Ceff, Rmax, glab);
    }
  }
}

// Assign the prefetched points [sub0, sub0 + nvalid) and stage them
// transposed in LDS for the update.  Writes labels to LDS and to glab.
template <typename TIn, int D, int CT, typename SM>
__device__ void km_assign_sub(SM& sm, const XRegs<TIn, D>& xr, int sub0, int nvalid,
                              const float* cent, int Ceff, float Rmax, int32_t* glab) {
  using S = KmShape<TIn, D>;
  constexpr int NS = S::NS;
  constexpr int KS = D / 32;
  if constexpr (NS == 1) {
    km_assign_bf16<TIn, D, CT>(sm, xr, sub0, nvalid, cent, Ceff, Rmax, glab);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  // screening error bound factor: bf16 centroids and bf16 points (fp32 input)
  const float efac = 0.0078125f * 1.05f;

#pragma unroll
  for (int grp = 0; grp < S::G16; ++grp) {
    const int pl = w * (S::SUB / 4) + grp * 16 + col;
    const bool valid = pl < nvalid;
    u16x8 xf[KS][NS];
    float xsq = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if constexpr (NS == 1) {
        xf[k][0] = xr.x[grp][k];
#pragma unroll
        for (int j = 0; j < 8; ++j) { const float v = xval(xr.x[grp][k], j); xsq = fmaf(v, v, xsq); }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = xr.x[grp][k][j];
          uint16_t h, m, l;
          split3(v, h, m, l);
          xf[k][0][j] = h; xf[k][NS > 1 ? 1 : 0][j] = m; xf[k][NS > 2 ? 2 : 0][j] = l;
          xsq = fmaf(v, v, xsq);
        }
      }
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.xt[sp][32 * k + 8 * g + j][pl] = xf[k][sp][j];
    }
    xsq += __shfl_xor(xsq, 16, 64);
    xsq += __shfl_xor(xsq, 32, 64);

    float dv[CT * 4];
    float best = INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      if (t * 16 < Ceff) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          u16x8 a = *reinterpret_cast<const u16x8*>(&sm.mu_hat[0][16 * t + col][32 * k + 8 * g]);
          acc = mfma(as_bf(a), as_bf(xf[k][0]), acc);
        }
        const f32x4 nrm = *reinterpret_cast<const f32x4*>(&sm.mu_norm[16 * t + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = fmaf(-2.f, acc[i], nrm[i]);
          dv[t * 4 + i] = d;
          if (d < best) { best = d; bi = 16 * t + 4 * g + i; }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[t * 4 + i] = INFINITY;
      }
    }
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
      float ob = __shfl_xor(best, m, 64);
      int oi = __shfl_xor(bi, m, 64);
      if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const float xn = sqrtf(xsq);
    const float margin = 2.f * (efac * xn * Rmax + 1.52587890625e-05f * (xsq + Rmax * Rmax));
    const float thr = best + margin;
    int cand = 0;
#pragma unroll
    for (int q = 0; q < CT * 4; ++q) cand += (dv[q] <= thr) ? 1 : 0;
    cand += __shfl_xor(cand, 16, 64);
    cand += __shfl_xor(cand, 32, 64);
    int label = bi;
    if (cand > 1) {
      // candidate clusters as a bitmask shared by the 4 lanes of this point
      constexpr int NW = (CT * 16 + 63) / 64;
      unsigned long long cm[NW];
#pragma unroll
      for (int q = 0; q < NW; ++q) cm[q] = 0ull;
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (dv[t * 4 + i] <= thr) {
            const int c = 16 * t + 4 * g + i;
            cm[c >> 6] |= 1ull << (c & 63);
          }
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        cm[q] |= __shfl_xor(cm[q], 16, 64);
        cm[q] |= __shfl_xor(cm[q], 32, 64);
      }
      float bd = INFINITY;
      int bc = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        unsigned long long mword = cm[q];
        while (mword) {
          const int c = 64 * q + __builtin_ctzll(mword);
          mword &= mword - 1;
          float part = 0.f;
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            float mv[8];
            if constexpr (SM::KEEP32) {
#pragma unroll
              for (int j = 0; j < 8; ++j) mv[j] = sm.mu32[c][32 * k + 8 * g + j];
            } else {
              const float* mr = cent + (size_t)c * D + 32 * k + 8 * g;
#pragma unroll
              for (int j = 0; j < 8; ++j) mv[j] = mr[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float df = xval(xr.x[grp][k], j) - mv[j];
              part = fmaf(df, df, part);
            }
          }
          part += __shfl_xor(part, 16, 64);
          part += __shfl_xor(part, 32, 64);
          if (part < bd || (part == bd && c < bc)) { bd = part; bc = c; }
        }
      }
      label = bc;
    }
    if (g == 0) {
      sm.lab[pl] = valid ? (uint16_t)label : (uint16_t)0xffff;
      if (valid) glab[sub0 + pl] = label;
    }
  }
}

// bf16 one-hot of 8 labels held two to a register: 1.0 where a label equals
// the cluster (both halves of clp), else 0.  Per half: x = l ^ c is zero
// exactly on a match; min(x, 1) is 0 or 1; 0x3F80 - 0x3F80 min(x, 1) (modulo
// 2^16) is 1.0 or 0.  Three packed 16-bit integer operations per two labels.
template <typename V>
__device__ __forceinline__ u16x8 onehot8(const V& lp, uint32_t clp) {
  // (each constant is given in both halves of a register: an inline constant
  // would supply only the low half)
  const uint32_t one1 = 0x00010001u, neg = 0xC080C080u, one = 0x3F803F80u;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m, o;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(m) : "v"((uint32_t)lp[q] ^ clp), "v"(one1));
    asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(o) : "v"(m), "v"(neg), "v"(one));
    r[q] = o;
  }
  return __builtin_bit_cast(u16x8, r);
}

// One-hot update: acc += onehot(labels) . X.  Wave w owns the cluster tiles
// ct = w, w+4, ... with every dim tile (one-hot built once per 32 points
// and cluster tile); with 2 cluster tiles it owns tile w & 1, dim tiles
// w/2, w/2 + 2, ...; with one, dim tiles dt = w, w+4, ... of tile 0.
template <typename TIn, int D, int CT>
struct KmAcc {
  static constexpr int DT = D / 16;
  static constexpr int U = CT >= 4 ? (CT / 4) * DT : CT == 2 ? DT / 2 : DT / 4;
  f32x4 a[U];
};

template <typename TIn, int D, int CT>
__device__ __forceinline__ void km_tile_of(int w, int u, int& ct, int& dt) {
  constexpr int DT = D / 16;
  if constexpr (CT >= 4) {
    ct = w + 4 * (u / DT);
    dt = u % DT;
  } else if constexpr (CT == 2) {
    ct = w & 1;
    dt = (w >> 1) + 2 * u;
  } else {
    ct = 0;
    dt = w + 4 * u;
  }
}

template <typename TIn, int D, int CT, typename SM>
__device__ void km_update_sub(SM& sm, KmAcc<TIn, D, CT>& acc, int Ceff) {
  using S = KmShape<TIn, D>;
  constexpr int NS = S::NS;
  constexpr int DT = D / 16;
  constexpr int NCT = CT >= 4 ? CT / 4 : 1;                          // cluster tiles per wave
  constexpr int NDT = CT >= 4 ? DT : CT == 2 ? DT / 2 : DT / 4;      // dim tiles per wave
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
#pragma unroll 2
  for (int ks = 0; ks < S::SUB / 32; ++ks) {
    // labels of points 32ks + 8g .. +7, two to a register
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 lp = *reinterpret_cast<const u32x4*>(&sm.lab[32 * ks + 8 * g]);
    u16x8 b[NDT][NS];
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
      const int dt = CT >= 4 ? d : CT == 2 ? (w >> 1) + 2 * d : w + 4 * d;
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        b[d][sp] = *reinterpret_cast<const u16x8*>(&sm.xt[sp][16 * dt + col][32 * ks + 8 * g]);
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int ct = CT >= 4 ? w + 4 * c : CT == 2 ? (w & 1) : 0;
      if (ct * 16 >= Ceff) continue;
      const u16x8 a = onehot8(lp, (uint32_t)(16 * ct + col) * 0x10001u);
#pragma unroll
      for (int d = 0; d < NDT; ++d) acc.a[c * NDT + d] = mfma_split<1, NS>(&a, b[d], acc.a[c * NDT + d]);
    }
  }
}

// ---------------------------------------------------------------------------
// Stable counting sort of a problem's labels into perm / offs.
// ---------------------------------------------------------------------------
template <typename SM>
__device__ void stable_perm(SM& sm, const int32_t* lab, int n, int C, int row0, int32_t* perm,
                            int32_t* offs) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int c = tid; c < MUSE_MAXC; c += KM_NT) sm.cnt[c] = 0;
  __syncthreads();
  // labels outside [0, C) (caller-provided assignments) are clamped
  for (int j = tid; j < n; j += KM_NT) atomicAdd(&sm.cnt[min(max(lab[j], 0), C - 1)], 1);
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of C <= 256 counts by one wave, 4 per lane
    int v[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = lane * 4 + q;
      v[q] = c < C ? sm.cnt[c] : 0;
      s += v[q];
    }
    int inc = s;
    for (int m = 1; m < 64; m <<= 1) {
      int o = __shfl_up(inc, m, 64);
      if (lane >= m) inc += o;
    }
    int run = inc - s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c = lane * 4 + q;
      if (c < C) { sm.cnt[c] = run; offs[c] = run; }
      run += v[q];
    }
    if (lane == 63) offs[C] = inc;
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = 0; b0 < n; b0 += KM_NT) {
    for (int c = tid; c < 4 * MUSE_MAXC; c += KM_NT) (&sm.wcnt[0][0])[c] = 0;
    __syncthreads();
    const int j = b0 + tid;
    const bool valid = j < n;
    const int L = valid ? min(max(lab[j], 0), C - 1) : 0;
    unsigned long long mt = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      unsigned long long bb = __ballot((L >> bit) & 1);
      mt &= ((L >> bit) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(mt & lt);
    if (valid && rank == 0) sm.wcnt[w][L] = __popcll(mt);
    __syncthreads();
    if (valid) {
      int pre = sm.cnt[L];
      for (int q = 0; q < w; ++q) pre += sm.wcnt[q][L];
      perm[pre + rank] = row0 + j;
    }
    __syncthreads();
    for (int c = tid; c < C; c += KM_NT)
      sm.cnt[c] += sm.wcnt[0][c] + sm.wcnt[1][c] + sm.wcnt[2][c] + sm.wcnt[3][c];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
struct CProb {
  const CSet* s;
  int head, p, lev, r0, n, Ceff;
};

__device__ __forceinline__ size_t cp_index(const Plan& pl, int head, int p) {
  return (size_t)head * pl.P + p;
}

template <typename TIn>
__global__ void __launch_bounds__(KM_NT) km_init_kernel(Plan pl, CSet s0, CSet s1, int D) {
  // one thread per (set, head, problem, cluster, 8-wide chunk of the row)
  const int tpc = D / 8;
  long long id = (long long)blockIdx.x * KM_NT + threadIdx.x;
  const int C = pl.C;
  const long long per_set0 = (long long)s0.heads * pl.P * C * tpc;
  const long long total = per_set0 + (long long)s1.heads * pl.P * C * tpc;
  if (id >= total) return;
  const bool first = id < per_set0;
  const CSet& s = first ? s0 : s1;
  if (!first) id -= per_set0;
  const int e0 = (int)(id % tpc) * 8;
  id /= tpc;
  const int c = (int)(id % C);
  id /= C;
  const int p = (int)(id % pl.P);
  const int head = (int)(id / pl.P);
  int lev, r0, n;
  cset_rows(pl, s, p, lev, r0, n);
  const int Ceff = min(s.C, n);
  float* dst = s.cent + (cp_index(pl, head, p) * C + c) * D + e0;
  float v[8];
  if (c < Ceff) {
    const int32_t* init = s.init ? s.init + cp_index(pl, head, p) * s.C : nullptr;
    int r = init ? init[c] : (int)(((long long)c * n) / Ceff);
    r = min(max(r, 0), n - 1);
    load8_f32<TIn>(reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0 + r) * D + e0, v);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
  }
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// All iterations for one problem in one workgroup; ends with the permutation.
template <typename TIn, int D, int CT>
__global__ void __launch_bounds__(KM_NT) km_local_kernel(Plan pl, CSet s0, CSet s1, int plocal) {
  using S = KmShape<TIn, D>;
  extern __shared__ __align__(16) unsigned char smraw[];
  KmSmem<TIn, D, CT>& sm = *reinterpret_cast<KmSmem<TIn, D, CT>*>(smraw);
  // largest problems first across both sets: p descends, and for each p
  // every head of both sets
  const int nh = s0.heads + s1.heads;
  const int hh = (int)blockIdx.x % nh;
  const int p = plocal - 1 - (int)blockIdx.x / nh;
  const CSet& s = hh < s0.heads ? s0 : s1;
  const int head = hh < s0.heads ? hh : hh - s0.heads;
  int lev, r0, n;
  cset_rows(pl, s, p, lev, r0, n);
  const int C = pl.C, Ceff = min(s.C, n);
  const TIn* Xp = reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0) * D;
  float* cent = s.cent + cp_index(pl, head, p) * C * D;
  int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  constexpr int U = KmAcc<TIn, D, CT>::U;

  for (int it = 0; it < pl.iters; ++it) {
    XRegs<TIn, D> xr;
    km_fetch<TIn, D>(xr, Xp, 0, min(S::SUB, n));
    float Rmax;
    km_load_centroids<TIn, D, CT>(sm, cent, Ceff, Rmax);
    for (int c = tid; c < MUSE_MAXC; c += KM_NT) sm.cnt[c] = 0;
    KmAcc<TIn, D, CT> acc;
#pragma unroll
    for (int u = 0; u < U; ++u) acc.a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int sub0 = 0; sub0 < n; sub0 += S::SUB) {
      const int nv = min(S::SUB, n - sub0);
      km_assign_sub<TIn, D, CT>(sm, xr, sub0, nv, cent, Ceff, Rmax, glab);
      if (sub0 + S::SUB < n) km_fetch<TIn, D>(xr, Xp, sub0 + S::SUB, min(S::SUB, n - sub0 - S::SUB));
      __syncthreads();
      for (int q = tid; q < nv; q += KM_NT) atomicAdd(&sm.cnt[sm.lab[q]], 1);
      km_update_sub<TIn, D, CT>(sm, acc, Ceff);
      __syncthreads();
    }
    // new centroids: mean of members, empty clusters keep theirs
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int ct, dt;
      km_tile_of<TIn, D, CT>(w, u, ct, dt);
      if (ct >= CT || ct * 16 >= Ceff) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * ct + 4 * g + i;
        const int k = sm.cnt[c];
        if (c < Ceff && k > 0) cent[(size_t)c * D + 16 * dt + col] = acc.a[u][i] / (float)k;
      }
    }
    __syncthreads();
  }
  int32_t* perm = s.perm + ((size_t)lev * s.heads + head) * pl.N + r0;
  int32_t* offs = s.offs + cp_index(pl, head, p) * (C + 1);
  stable_perm(sm, glab, n, Ceff, r0, perm, offs);
  for (int c = Ceff + 1 + tid; c <= C; c += KM_NT) offs[c] = n;
}

// One Lloyd iteration over point chunks of the large problems.
template <typename TIn, int D, int CT>
__global__ void __launch_bounds__(KM_NT) km_assign_kernel(Plan pl, CSet s0, CSet s1, KmLarge lg,
                                                          float* part, int32_t* pcnt) {
  using S = KmShape<TIn, D>;
  extern __shared__ __align__(16) unsigned char smraw[];
  KmSmem<TIn, D, CT>& sm = *reinterpret_cast<KmSmem<TIn, D, CT>*>(smraw);
  int li = 0;
  while (li + 1 < lg.nl && lg.wfirst[li + 1] <= (int)blockIdx.x) ++li;
  const int lev = lg.lev[li], nch = lg.nch[li], nseg = pl.lev_nseg[lev];
  // the chunks of one problem share an XCD (dispatch is round-robin over 8)
  const int wl = blockIdx.x - lg.wfirst[li];
  const int xcd = wl % 8, loc = wl / 8;
  const int prob = (loc / nch) * 8 + xcd;
  if (prob >= (s0.heads + s1.heads) * nseg) return;
  const int chunk = lg.cfirst[li] + prob * nch + loc % nch;
  int rem = chunk - lg.cfirst[li];
  const int per_head = nseg * nch;
  const bool first = rem < s0.heads * per_head;
  const CSet& s = first ? s0 : s1;
  if (!first) rem -= s0.heads * per_head;
  const int head = rem / per_head;
  const int t = (rem % per_head) / nch, ci = rem % nch;
  const int p = pl.lev_pfirst[lev] + t;
  int lv, r0, n;
  cset_rows(pl, s, p, lv, r0, n);
  const int C = pl.C, Ceff = min(s.C, n);
  const int c0 = ci * lg.ch, c1 = min(n, c0 + lg.ch);
  const TIn* Xp = reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0) * D;
  const float* cent = s.cent + cp_index(pl, head, p) * C * D;
  int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  constexpr int U = KmAcc<TIn, D, CT>::U;

  XRegs<TIn, D> xr;
  km_fetch<TIn, D>(xr, Xp, c0, min(S::SUB, c1 - c0));
  float Rmax;
  km_load_centroids<TIn, D, CT>(sm, cent, Ceff, Rmax);
  for (int c = tid; c < MUSE_MAXC; c += KM_NT) sm.cnt[c] = 0;
  KmAcc<TIn, D, CT> acc;
#pragma unroll
  for (int u = 0; u < U; ++u) acc.a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int sub0 = c0; sub0 < c1; sub0 += S::SUB) {
    const int nv = min(S::SUB, c1 - sub0);
    km_assign_sub<TIn, D, CT>(sm, xr, sub0, nv, cent, Ceff, Rmax, glab);
    if (sub0 + S::SUB < c1) km_fetch<TIn, D>(xr, Xp, sub0 + S::SUB, min(S::SUB, c1 - sub0 - S::SUB));
    __syncthreads();
    for (int q = tid; q < nv; q += KM_NT) atomicAdd(&sm.cnt[sm.lab[q]], 1);
    km_update_sub<TIn, D, CT>(sm, acc, Ceff);
    __syncthreads();
  }
  float* pp = part + (size_t)chunk * C * D;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int ct, dt;
    km_tile_of<TIn, D, CT>(w, u, ct, dt);
    if (ct >= CT || ct * 16 >= Ceff) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ct + 4 * g + i;
      if (c < Ceff) pp[(size_t)c * D + 16 * dt + col] = acc.a[u][i];
    }
  }
  for (int c = tid; c < C; c += KM_NT) pcnt[(size_t)chunk * C + c] = sm.cnt[c];
}

// Centroids of the large problems from the chunk partials: one thread per
// (cluster, dim), chunks summed in a fixed order.
__global__ void __launch_bounds__(256) km_reduce_kernel(Plan pl, CSet s0, CSet s1, KmLarge lg,
                                                        const float* part, const int32_t* pcnt, int D) {
  const int cpb = 256 / D;                       // clusters per workgroup
  const int ncb = (pl.C + cpb - 1) / cpb;
  int li = 0;
  while (li + 1 < lg.nl && lg.rfirst[li + 1] <= (int)blockIdx.x) ++li;
  const int wl = blockIdx.x - lg.rfirst[li];
  const int xcd = wl % 8, loc = wl / 8;
  const int lev = lg.lev[li], nch = lg.nch[li], nseg = pl.lev_nseg[lev];
  const int prob = (loc / ncb) * 8 + xcd;
  const int cb = loc % ncb;
  if (prob >= (s0.heads + s1.heads) * nseg) return;
  int rem = prob;
  const bool first = rem < s0.heads * nseg;
  const CSet& s = first ? s0 : s1;
  const int cbase_set = first ? 0 : s0.heads * nseg * nch;
  if (!first) rem -= s0.heads * nseg;
  const int head = rem / nseg, t = rem % nseg;
  const int p = pl.lev_pfirst[lev] + t;
  int lv, r0, n;
  cset_rows(pl, s, p, lv, r0, n);
  const int C = pl.C, Ceff = min(s.C, n);
  const int c = cb * cpb + threadIdx.x / D, e = threadIdx.x % D;
  if (c >= Ceff) return;
  const int nchp = (n + lg.ch - 1) / lg.ch;
  const size_t chunk0 = (size_t)lg.cfirst[li] + cbase_set + ((size_t)head * nseg + t) * nch;
  // batches of 8 independent loads, summed in a fixed order
  float sum = 0.f;
  int k = 0;
  for (int q0 = 0; q0 < nchp; q0 += 8) {
    float v[8];
    int n8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool ok = q0 + q < nchp;
      const size_t b = (chunk0 + q0 + q) * C + c;
      v[q] = ok ? part[b * D + e] : 0.f;
      n8[q] = ok ? pcnt[b] : 0;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) { sum += v[q]; k += n8[q]; }
  }
  if (k > 0) s.cent[(cp_index(pl, head, p) * C + c) * D + e] = sum / (float)k;
}

// Permutation of the large problems after their last iteration, one
// workgroup per chunk: the cluster counts of every chunk (the last
// iteration's chunk histograms) give each chunk's output base per cluster;
// ranks inside the chunk come from wave ballots, so the order is stable.
__global__ void __launch_bounds__(KM_NT) km_perm_chunk_kernel(Plan pl, CSet s0, CSet s1, KmLarge lg,
                                                              const int32_t* pcnt) {
  __shared__ struct {
    int32_t base[MUSE_MAXC];
    int32_t tot[MUSE_MAXC];
    int32_t wcnt[4][MUSE_MAXC];
  } sm;
  int li = 0;
  while (li + 1 < lg.nl && lg.wfirst[li + 1] <= (int)blockIdx.x) ++li;
  const int lev = lg.lev[li], nch = lg.nch[li], nseg = pl.lev_nseg[lev];
  const int wl = blockIdx.x - lg.wfirst[li];
  const int xcd = wl % 8, loc = wl / 8;
  const int prob = (loc / nch) * 8 + xcd;
  if (prob >= (s0.heads + s1.heads) * nseg) return;
  const int ci = loc % nch;
  const int chunk0 = lg.cfirst[li] + prob * nch;     // first chunk of this problem
  int rem = prob;
  const bool first = rem < s0.heads * nseg;
  const CSet& s = first ? s0 : s1;
  if (!first) rem -= s0.heads * nseg;
  const int head = rem / nseg, t = rem % nseg;
  const int p = pl.lev_pfirst[lev] + t;
  int lv, r0, n;
  cset_rows(pl, s, p, lv, r0, n);
  const int C = pl.C, Ceff = min(s.C, n);
  const int nchp = (n + lg.ch - 1) / lg.ch;
  const int c0 = ci * lg.ch, c1 = min(n, c0 + lg.ch);
  if (c0 >= c1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // totals and this chunk's base per cluster
  for (int c = tid; c < MUSE_MAXC; c += KM_NT) {
    int tot = 0, before = 0;
    if (c < Ceff) {
      for (int q = 0; q < nchp; ++q) {
        const int k = pcnt[(size_t)(chunk0 + q) * C + c];
        tot += k;
        if (q < ci) before += k;
      }
    }
    sm.tot[c] = tot;
    sm.base[c] = before;
  }
  __syncthreads();
  int32_t* offs = s.offs + cp_index(pl, head, p) * (C + 1);
  if (tid < 64) {
    // exclusive scan of the totals (4 per lane)
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lane * 4 + q;
      v[q] = c < Ceff ? sm.tot[c] : 0;
      sum += v[q];
    }
    int inc = sum;
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(inc, m, 64);
      if (lane >= m) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lane * 4 + q;
      if (c < Ceff) {
        sm.base[c] += run;
        if (ci == 0) offs[c] = run;
      }
      run += v[q];
    }
  }
  if (ci == 0)
    for (int c = Ceff + tid; c <= C; c += KM_NT) offs[c] = n;
  __syncthreads();
  const int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  int32_t* perm = s.perm + ((size_t)lev * s.heads + head) * pl.N + r0;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = c0; b0 < c1; b0 += KM_NT) {
    for (int c = tid; c < 4 * MUSE_MAXC; c += KM_NT) (&sm.wcnt[0][0])[c] = 0;
    __syncthreads();
    const int j = b0 + tid;
    const bool valid = j < c1;
    const int L = valid ? min(max(glab[j], 0), Ceff - 1) : 0;
    unsigned long long mt = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      unsigned long long bb = __ballot((L >> bit) & 1);
      mt &= ((L >> bit) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(mt & lt);
    if (valid && rank == 0) sm.wcnt[w][L] = __popcll(mt);
    __syncthreads();
    if (valid) {
      int pre = sm.base[L];
      for (int q = 0; q < w; ++q) pre += sm.wcnt[q][L];
      perm[pre + rank] = r0 + j;
    }
    __syncthreads();
    for (int c = tid; c < Ceff; c += KM_NT)
      sm.base[c] += sm.wcnt[0][c] + sm.wcnt[1][c] + sm.wcnt[2][c] + sm.wcnt[3][c];
    __syncthreads();
  }
}

// Permutation of a set of problems from given labels (one workgroup each).
__global__ void __launch_bounds__(KM_NT) km_perm_kernel(Plan pl, CSet s0, CSet s1, int plocal) {
  __shared__ struct {
    int32_t cnt[MUSE_MAXC];
    int32_t wcnt[4][MUSE_MAXC];
  } sm;
  const int nl = pl.P - plocal;
  int id = blockIdx.x;
  const CSet& s = (id < s0.heads * nl) ? s0 : s1;
  if (id >= s0.heads * nl) id -= s0.heads * nl;
  const int head = id / nl, p = plocal + id % nl;
  int lev, r0, n;
  cset_rows(pl, s, p, lev, r0, n);
  const int C = pl.C, Ceff = min(s.C, n);
  const int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  int32_t* perm = s.perm + ((size_t)lev * s.heads + head) * pl.N + r0;
  int32_t* offs = s.offs + cp_index(pl, head, p) * (C + 1);
  stable_perm(sm, glab, n, Ceff, r0, perm, offs);
  for (int c = Ceff + 1 + threadIdx.x; c <= C; c += KM_NT) offs[c] = n;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename TIn, int D, int CT>
static hipError_t km_run_t(const Plan& pl, const CSet& s0, const CSet& s1, int plocal,
                           const KmLarge& lg, float* part, int32_t* pcnt, hipStream_t st) {
  const int nsets_heads = s0.heads + s1.heads;
  const size_t smem = sizeof(KmSmem<TIn, D, CT>);
  if (nsets_heads == 0) return hipSuccess;
  if (!pl.warm) {   // a warm start keeps the centroids the state already holds
    const long long thr = (long long)nsets_heads * pl.P * pl.C * (D / 8);
    MUSE_KT_PRE(st);
    km_init_kernel<TIn><<<(unsigned)((thr + KM_NT - 1) / KM_NT), KM_NT, 0, st>>>(pl, s0, s1, D);
    MUSE_KT_POST("km_init", st);
  }
  if (plocal > 0) {
    auto k = km_local_kernel<TIn, D, CT>;
    set_smem_once((const void*)k, smem);
    MUSE_KT_PRE(st);
    k<<<nsets_heads * plocal, KM_NT, smem, st>>>(pl, s0, s1, plocal);
    MUSE_KT_POST("km_local", st);
  }
  if (lg.nl > 0) {
    auto ka = km_assign_kernel<TIn, D, CT>;
    set_smem_once((const void*)ka, smem);
    for (int it = 0; it < pl.iters; ++it) {
      MUSE_KT_PRE(st);
      ka<<<lg.wfirst[lg.nl], KM_NT, smem, st>>>(pl, s0, s1, lg, part, pcnt);
      MUSE_KT_POST("km_assign", st);
      MUSE_KT_PRE(st);
      km_reduce_kernel<<<lg.rfirst[lg.nl], 256, 0, st>>>(pl, s0, s1, lg, part, pcnt, D);
      MUSE_KT_POST("km_reduce", st);
    }
    MUSE_KT_PRE(st);
    km_perm_chunk_kernel<<<lg.wfirst[lg.nl], KM_NT, 0, st>>>(pl, s0, s1, lg, pcnt);
    MUSE_KT_POST("km_perm", st);
  }
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t km_run_d(const Plan& pl, const CSet& s0, const CSet& s1, int plocal,
                           const KmLarge& lg, float* part, int32_t* pcnt, hipStream_t st) {
  if (pl.C <= 16) return km_run_t<TIn, D, 1>(pl, s0, s1, plocal, lg, part, pcnt, st);
  if (pl.C <= 32) return km_run_t<TIn, D, 2>(pl, s0, s1, plocal, lg, part, pcnt, st);
  if (pl.C <= 64) return km_run_t<TIn, D, 4>(pl, s0, s1, plocal, lg, part, pcnt, st);
  if (pl.C <= 128) return km_run_t<TIn, D, 8>(pl, s0, s1, plocal, lg, part, pcnt, st);
  return km_run_t<TIn, D, 16>(pl, s0, s1, plocal, lg, part, pcnt, st);
}

hipError_t launch_kmeans(const Plan& pl, int dtype, const CSet& s0, const CSet& s1, int plocal,
                         const KmLarge& lg, float* part, int32_t* pcnt, hipStream_t st) {
  if (dtype == 1) {
    if (pl.D == 64) return km_run_d<uint16_t, 64>(pl, s0, s1, plocal, lg, part, pcnt, st);
    return km_run_d<uint16_t, 128>(pl, s0, s1, plocal, lg, part, pcnt, st);
  }
  if (pl.D == 64) return km_run_d<float, 64>(pl, s0, s1, plocal, lg, part, pcnt, st);
  return km_run_d<float, 128>(pl, s0, s1, plocal, lg, part, pcnt, st);
}

hipError_t launch_perm_only(const Plan& pl, const CSet& s0, hipStream_t st) {
  CSet s1{nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0};
  if (s0.heads * pl.P == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  km_perm_kernel<<<s0.heads * pl.P, KM_NT, 0, st>>>(pl, s0, s1, 0);
  MUSE_KT_POST("km_perm", st);
  return hipGetLastError();
}

size_t kmeans_smem_bytes(int dtype, int D, int C) {
  auto pick = [&](auto tin, auto dd) -> size_t {
    using T = decltype(tin);
    constexpr int DD = decltype(dd)::value;
    if (C <= 16) return sizeof(KmSmem<T, DD, 1>);
    if (C <= 32) return sizeof(KmSmem<T, DD, 2>);
    if (C <= 64) return sizeof(KmSmem<T, DD, 4>);
    if (C <= 128) return sizeof(KmSmem<T, DD, 8>);
    return sizeof(KmSmem<T, DD, 16>);
  };
  if (dtype == 1)
    return D == 64 ? pick(uint16_t{}, std::integral_constant<int, 64>{})
                   : pick(uint16_t{}, std::integral_constant<int, 128>{});
  return D == 64 ? pick(float{}, std::integral_constant<int, 64>{})
                 : pick(float{}, std::integral_constant<int, 128>{});
}

int kmeans_sub(int dtype, int D) { return dtype == 1 ? 128 : (D == 128 ? 64 : 256); }

}  // namespace muse
