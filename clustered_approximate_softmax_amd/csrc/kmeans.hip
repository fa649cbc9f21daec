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
  static constexpr int MUP = D + 8;  // padded centroid row (bf16 elements)
  static constexpr int SUB = (NS == 3 && D == 128) ? 64 : 256;
  static constexpr int XTP = SUB + 8;  // padded transposed row
  static constexpr int G16 = SUB / 64; // 16-point groups per wave per sub-tile
};

template <typename TIn, int D, int CT>
struct alignas(16) KmSmem {
  using S = KmShape<TIn, D>;
  uint16_t mu_hat[CT * 16][S::MUP];
  float mu_norm[CT * 16];
  uint16_t xt[S::NS][D][S::XTP];
  int32_t lab[S::SUB];
  int32_t cnt[MUSE_MAXC];
  int32_t wcnt[4][MUSE_MAXC];
  float red[8];
};

// Load the problem's current fp32 centroids into bf16 rows + squared norms.
template <typename TIn, int D, int CT>
__device__ void km_load_centroids(KmSmem<TIn, D, CT>& sm, const float* cent, int Ceff, float& Rmax) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < CT * 16 * (D / 8); idx += KM_NT) {
    int c = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
    u16x8 h;
    if (c < Ceff) {
      const float* src = cent + (size_t)c * D + e0;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = f2bf(src[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = 0;
    }
    *reinterpret_cast<u16x8*>(&sm.mu_hat[c][e0]) = h;
  }
  float mx = 0.f;
  for (int c = tid; c < CT * 16; c += KM_NT) {
    float s = INFINITY;
    if (c < Ceff) {
      const float* src = cent + (size_t)c * D;
      s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(src[e], src[e], s);
      mx = fmaxf(mx, s);
    }
    sm.mu_norm[c] = s;
  }
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if ((tid & 63) == 0) sm.red[tid >> 6] = mx;
  __syncthreads();
  Rmax = sqrtf(fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3])));
}

// Assign the points [sub0, sub0 + nvalid) of a problem (rows relative to
// Xp) and stage them transposed in LDS for the update.  Writes labels to
// LDS and to glab (problem-local index).
template <typename TIn, int D, int CT>
__device__ void km_assign_sub(KmSmem<TIn, D, CT>& sm, const TIn* Xp, int sub0, int nvalid,
                              const float* cent, int Ceff, float Rmax, int32_t* glab) {
  using S = KmShape<TIn, D>;
  constexpr int NS = S::NS;
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  // screening error bound factor: bf16 centroids (and bf16 points for fp32 input)
  const float efac = (NS == 1 ? 0.00390625f : 0.0078125f) * 1.05f;

#pragma unroll 1
  for (int grp = 0; grp < S::G16; ++grp) {
    const int pl = w * (S::SUB / 4) + grp * 16 + col;
    const bool valid = pl < nvalid;
    u16x8 xf[KS][NS];
    float xsq = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (valid) {
        const TIn* src = Xp + (size_t)(sub0 + pl) * D + 32 * k + 8 * g;
        load8_split<TIn, NS>(src, xf[k]);
        float v[8];
        load8_f32<TIn>(src, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) xsq = fmaf(v[j], v[j], xsq);
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) xf[k][s][j] = 0;
      }
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.xt[s][32 * k + 8 * g + j][pl] = xf[k][s][j];
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
          u16x8 a = *reinterpret_cast<const u16x8*>(&sm.mu_hat[16 * t + col][32 * k + 8 * g]);
          acc = mfma(as_bf(a), as_bf(xf[k][0]), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * t + 4 * g + i;
          const float d = sm.mu_norm[c] - 2.f * acc[i];
          dv[t * 4 + i] = d;
          if (d < best) { best = d; bi = c; }
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
      float bd = INFINITY;
      int bc = 0x7fffffff;
      if (valid) {
        const TIn* xr = Xp + (size_t)(sub0 + pl) * D;
#pragma unroll
        for (int t = 0; t < CT; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (dv[t * 4 + i] <= thr) {
              const int c = 16 * t + 4 * g + i;
              const float* mr = cent + (size_t)c * D;
              float d = 0.f;
              for (int e = 0; e < D; e += 8) {
                float xv[8];
                load8_f32<TIn>(xr + e, xv);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                  float df = xv[j] - mr[e + j];
                  d = fmaf(df, df, d);
                }
              }
              if (d < bd || (d == bd && c < bc)) { bd = d; bc = c; }
            }
          }
        }
      }
#pragma unroll
      for (int m = 16; m <= 32; m <<= 1) {
        float ob = __shfl_xor(bd, m, 64);
        int oi = __shfl_xor(bc, m, 64);
        if (ob < bd || (ob == bd && oi < bc)) { bd = ob; bc = oi; }
      }
      label = bc;
    }
    if (g == 0) {
      sm.lab[pl] = valid ? label : -1;
      if (valid) glab[sub0 + pl] = label;
    }
  }
}

// One-hot update: acc[u] += onehot(labels) . X for this wave's tiles.
// Wave w owns tiles tau = ct * (D/16) + dt with tau % 4 == w.
template <typename TIn, int D, int CT>
struct KmAcc {
  static constexpr int U = CT * (D / 16) / 4 > 0 ? CT * (D / 16) / 4 : 1;
  f32x4 a[U];
};

template <typename TIn, int D, int CT>
__device__ __forceinline__ void km_tile_of(int w, int u, int& ct, int& dt) {
  int tau = w + 4 * u;
  ct = tau / (D / 16);
  dt = tau % (D / 16);
}

template <typename TIn, int D, int CT>
__device__ void km_update_sub(KmSmem<TIn, D, CT>& sm, KmAcc<TIn, D, CT>& acc, int Ceff) {
  using S = KmShape<TIn, D>;
  constexpr int NS = S::NS;
  constexpr int U = KmAcc<TIn, D, CT>::U;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
#pragma unroll 1
  for (int ks = 0; ks < S::SUB / 32; ++ks) {
    int labs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) labs[j] = sm.lab[32 * ks + 8 * g + j];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int ct, dt;
      km_tile_of<TIn, D, CT>(w, u, ct, dt);
      if (ct >= CT || ct * 16 >= Ceff) continue;
      u16x8 a;
      const int cl = 16 * ct + col;
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (labs[j] == cl) ? (uint16_t)0x3F80 : (uint16_t)0;
      u16x8 b[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        b[s] = *reinterpret_cast<const u16x8*>(&sm.xt[s][16 * dt + col][32 * ks + 8 * g]);
      acc.a[u] = mfma_split<1, NS>(&a, b, acc.a[u]);
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
  for (int j = tid; j < n; j += KM_NT) atomicAdd(&sm.cnt[lab[j]], 1);
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
    const int L = valid ? lab[j] : 0;
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
  // one workgroup per (set, head, p)
  int id = blockIdx.x;
  const int per = pl.P;
  const CSet& s = (id < s0.heads * per) ? s0 : s1;
  if (id >= s0.heads * per) id -= s0.heads * per;
  const int head = id / per, p = id % per;
  int lev, r0, n;
  cset_rows(pl, s, p, lev, r0, n);
  const int C = pl.C, Ceff = min(C, n);
  const TIn* X = reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0) * D;
  float* cent = s.cent + cp_index(pl, head, p) * C * D;
  const int32_t* init = s.init ? s.init + cp_index(pl, head, p) * C : nullptr;
  for (int idx = threadIdx.x; idx < C * D; idx += KM_NT) {
    int c = idx / D, e = idx % D;
    float v = 0.f;
    if (c < Ceff) {
      int r = init ? init[c] : (int)(((long long)c * n) / Ceff);
      r = min(max(r, 0), n - 1);
      v = load1_f32<TIn>(X + (size_t)r * D + e);
    }
    cent[idx] = v;
  }
}

// All iterations for one problem in one workgroup; ends with the permutation.
template <typename TIn, int D, int CT>
__global__ void __launch_bounds__(KM_NT) km_local_kernel(Plan pl, CSet s0, CSet s1, int plocal) {
  using S = KmShape<TIn, D>;
  extern __shared__ __align__(16) unsigned char smraw[];
  KmSmem<TIn, D, CT>& sm = *reinterpret_cast<KmSmem<TIn, D, CT>*>(smraw);
  int id = blockIdx.x;
  // largest problems first: p descends within each set
  const CSet& s = (id < s0.heads * plocal) ? s0 : s1;
  if (id >= s0.heads * plocal) id -= s0.heads * plocal;
  const int head = id % s.heads;
  const int p = plocal - 1 - id / s.heads;
  int lev, r0, n;
  cset_rows(pl, s, p, lev, r0, n);
  const int C = pl.C, Ceff = min(C, n);
  const TIn* Xp = reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0) * D;
  float* cent = s.cent + cp_index(pl, head, p) * C * D;
  int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  constexpr int U = KmAcc<TIn, D, CT>::U;

  for (int it = 0; it < pl.iters; ++it) {
    float Rmax;
    km_load_centroids<TIn, D, CT>(sm, cent, Ceff, Rmax);
    for (int c = tid; c < MUSE_MAXC; c += KM_NT) sm.cnt[c] = 0;
    KmAcc<TIn, D, CT> acc;
#pragma unroll
    for (int u = 0; u < U; ++u) acc.a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int sub0 = 0; sub0 < n; sub0 += S::SUB) {
      const int nv = min(S::SUB, n - sub0);
      km_assign_sub<TIn, D, CT>(sm, Xp, sub0, nv, cent, Ceff, Rmax, glab);
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
  const int chunk = blockIdx.x;
  int li = 0;
  while (li + 1 < lg.nl && lg.cfirst[li + 1] <= chunk) ++li;
  const int lev = lg.lev[li], nch = lg.nch[li], nseg = pl.lev_nseg[lev];
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
  const int C = pl.C, Ceff = min(C, n);
  const int c0 = ci * lg.ch, c1 = min(n, c0 + lg.ch);
  const TIn* Xp = reinterpret_cast<const TIn*>(s.X) + ((size_t)head * pl.N + r0) * D;
  const float* cent = s.cent + cp_index(pl, head, p) * C * D;
  int32_t* glab = s.labels + ((size_t)lev * s.heads + head) * pl.N + r0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  constexpr int U = KmAcc<TIn, D, CT>::U;

  float Rmax;
  km_load_centroids<TIn, D, CT>(sm, cent, Ceff, Rmax);
  for (int c = tid; c < MUSE_MAXC; c += KM_NT) sm.cnt[c] = 0;
  KmAcc<TIn, D, CT> acc;
#pragma unroll
  for (int u = 0; u < U; ++u) acc.a[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int sub0 = c0; sub0 < c1; sub0 += S::SUB) {
    const int nv = min(S::SUB, c1 - sub0);
    km_assign_sub<TIn, D, CT>(sm, Xp, sub0, nv, cent, Ceff, Rmax, glab);
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

// Centroids of the large problems from the chunk partials.
__global__ void km_reduce_kernel(Plan pl, CSet s0, CSet s1, KmLarge lg, const float* part,
                                 const int32_t* pcnt, int D) {
  // one workgroup per (level entry, set, head, t); threads over (c, e)
  int id = blockIdx.x;
  int li = 0;
  while (li + 1 < lg.nl && lg.pfirst[li + 1] <= id) ++li;
  const int lev = lg.lev[li], nch = lg.nch[li], nseg = pl.lev_nseg[lev];
  int rem = id - lg.pfirst[li];
  const bool first = rem < s0.heads * nseg;
  const CSet& s = first ? s0 : s1;
  const int cbase_set = first ? 0 : s0.heads * nseg * nch;
  if (!first) rem -= s0.heads * nseg;
  const int head = rem / nseg, t = rem % nseg;
  const int p = pl.lev_pfirst[lev] + t;
  int lv, r0, n;
  cset_rows(pl, s, p, lv, r0, n);
  const int C = pl.C, Ceff = min(C, n);
  const int nchp = (n + lg.ch - 1) / lg.ch;
  const size_t chunk0 = (size_t)lg.cfirst[li] + cbase_set + ((size_t)head * nseg + t) * nch;
  float* cent = s.cent + cp_index(pl, head, p) * C * D;
  for (int idx = threadIdx.x; idx < Ceff * D; idx += blockDim.x) {
    const int c = idx / D;
    float sum = 0.f;
    int k = 0;
    for (int q = 0; q < nchp; ++q) {
      sum += part[(chunk0 + q) * C * D + idx];
      k += pcnt[(chunk0 + q) * C + c];
    }
    if (k > 0) cent[idx] = sum / (float)k;
  }
}

// Permutation of the large problems after their last iteration.
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
  const int C = pl.C, Ceff = min(C, n);
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
  MUSE_KT_PRE(st);
  km_init_kernel<TIn><<<nsets_heads * pl.P, KM_NT, 0, st>>>(pl, s0, s1, D);
  MUSE_KT_POST("km_init", st);
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
      ka<<<lg.cfirst[lg.nl], KM_NT, smem, st>>>(pl, s0, s1, lg, part, pcnt);
      MUSE_KT_POST("km_assign", st);
      MUSE_KT_PRE(st);
      km_reduce_kernel<<<lg.pfirst[lg.nl], 256, 0, st>>>(pl, s0, s1, lg, part, pcnt, D);
      MUSE_KT_POST("km_reduce", st);
    }
    MUSE_KT_PRE(st);
    km_perm_kernel<<<nsets_heads * (pl.P - plocal), KM_NT, 0, st>>>(pl, s0, s1, plocal);
    MUSE_KT_POST("km_perm", st);
  }
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t km_run_d(const Plan& pl, const CSet& s0, const CSet& s1, int plocal,
                           const KmLarge& lg, float* part, int32_t* pcnt, hipStream_t st) {
  if (pl.C <= 16) return km_run_t<TIn, D, 1>(pl, s0, s1, plocal, lg, part, pcnt, st);
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
  CSet s1{nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
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

int kmeans_sub(int dtype, int D) { return (dtype == 0 && D == 128) ? 64 : 256; }

}  // namespace muse
