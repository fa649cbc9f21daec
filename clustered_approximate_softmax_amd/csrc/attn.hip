// Stage two of the two-stage attention and the exact parts of the causal
// hierarchy (gist.science page, Technical Summary, Core Mechanisms:
// Decomposition, Hierarchical Two-Stage Attention, Retrieval-Augmented
// Approximation; newx.sg page, Abstract: exact local blocks).
//
// For a query i of query cluster I the softmax runs over two kinds of
// items: every key j of a retrieved cluster (logit s q_i.k_j, weight 1,
// value v_j) and every other non-empty key cluster c (logit s q_i.mu_c,
// weight n_c, value T_Ic / n_c).  Both kinds are fed through the same tile
// loop: a tile is 32 items staged in LDS as rows (for S^T = K Q^T) and as a
// transposed value block (for O^T = V^T P^T), plus a log-weight per item;
// one online softmax covers all tiles.  The local causal block uses the same
// loop over contiguous keys with the causal mask.
#include "common.h"
#include "launch.h"

namespace muse {

enum { MODE_ACAUSAL = 0, MODE_LEVEL = 1, MODE_LOCAL = 2 };
constexpr int AT_KT = 32;

template <typename TIn, int D, int WAVES>
struct alignas(16) AtSmem {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  uint16_t ks[NS][AT_KT][D + 8];
  uint16_t vt[NS][D][AT_KT + 8];
  float bias[AT_KT];
  int32_t krow[AT_KT];
  int32_t qrow[16 * WAVES];
  float far_bias[MUSE_MAXC];
  float far_ninv[MUSE_MAXC];
  int32_t rc[MUSE_MAXC];
  int32_t rcum[MUSE_MAXC + 1];
  int32_t tpre[MUSE_MAXC + 1];
  int32_t sel[4];
};

// Stage rows (K and V) of a tile given per-item row indices (-1: masked).
template <typename TIn, int D, int WAVES>
__device__ __forceinline__ void stage_rows(AtSmem<TIn, D, WAVES>& sm, const TIn* K, const TIn* V) {
  constexpr int NS = AtSmem<TIn, D, WAVES>::NS;
  constexpr int NT = 64 * WAVES;
  constexpr int TPK = D / 8;
  for (int idx = threadIdx.x; idx < AT_KT * TPK; idx += NT) {
    const int it = idx / TPK, e0 = (idx % TPK) * 8;
    const int row = sm.krow[it];
    u16x8 kk[NS], vv[NS];
    if (row >= 0) {
      load8_split<TIn, NS>(K + (size_t)row * D + e0, kk);
      load8_split<TIn, NS>(V + (size_t)row * D + e0, vv);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) { kk[s][j] = 0; vv[s][j] = 0; }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      *reinterpret_cast<u16x8*>(&sm.ks[s][it][e0]) = kk[s];
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.vt[s][e0 + j][it] = vv[s][j];
    }
  }
}

template <int NS, int D>
struct AtState {
  static constexpr int DT = D / 16;
  float m, lpart;
  f32x4 o[DT];
};

// Consume the staged tile: logits, online softmax, O^T += V^T P^T.
template <typename TIn, int D, int WAVES, bool CAUSAL>
__device__ __forceinline__ void consume_tile(AtSmem<TIn, D, WAVES>& sm,
                                             const u16x8 (&qf)[D / 32][AtSmem<TIn, D, WAVES>::NS],
                                             AtState<AtSmem<TIn, D, WAVES>::NS, D>& st, float s,
                                             int qrow) {
  constexpr int NS = AtSmem<TIn, D, WAVES>::NS;
  constexpr int KS = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  f32x4 sc[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    sc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u16x8 a[NS];
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        a[sp] = *reinterpret_cast<const u16x8*>(&sm.ks[sp][16 * rt + col][32 * k + 8 * g]);
      sc[rt] = mfma_split<NS, NS>(a, qf[k], sc[rt]);
    }
  }
  float x[8];
  float mloc = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int it = 16 * rt + 4 * g + i;
      float v = s * sc[rt][i] + sm.bias[it];
      if (CAUSAL && sm.krow[it] > qrow) v = -INFINITY;
      x[rt * 4 + i] = v;
      mloc = fmaxf(mloc, v);
    }
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  const float mnew = fmaxf(st.m, mloc);
  const float alpha = __expf(st.m - mnew);
  float psum = 0.f;
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __expf(x[j] - mnew);
    psum += p[j];
  }
  st.lpart = st.lpart * alpha + psum;
  st.m = mnew;
  u16x8 pb[NS];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (NS == 1) {
      pb[0][j] = f2bf(p[j]);
    } else {
      uint16_t h, mm, l;
      split3(p[j], h, mm, l);
      pb[0][j] = h; pb[1 % NS][j] = mm; pb[2 % NS][j] = l;
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st.o[dt] *= alpha;
    u16x8 a[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const uint16_t* r = &sm.vt[sp][16 * dt + col][0];
      u16x4 lo = *reinterpret_cast<const u16x4*>(r + 4 * g);
      u16x4 hi = *reinterpret_cast<const u16x4*>(r + 16 + 4 * g);
      a[sp] = u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    st.o[dt] = mfma_split<NS, NS>(a, pb, st.o[dt]);
  }
}

template <typename TIn, typename TOut, int D, int WAVES, int MODE>
__global__ void __launch_bounds__(64 * WAVES) attn_kernel(Plan pl, AttnBufs b, int lev) {
  constexpr int NS = AtSmem<TIn, D, WAVES>::NS;
  constexpr int NT = 64 * WAVES, QT = 16 * WAVES;
  constexpr int KS = D / 32, DT = D / 16;
  __shared__ AtSmem<TIn, D, WAVES> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const float s = pl.scale;
  const int C = pl.C;

  int bh, kvh, ap = 0, I = 0, tile, kp = 0, k0 = 0, Ck = 0, Cq = 0, q0 = 0;
  int qlo = 0, qhi = 0;       // query rows (LOCAL) or positions within cluster I
  if (MODE == MODE_LOCAL) {
    const int nblk = (pl.N + pl.blk - 1) / pl.blk;
    const int tpb = (pl.blk + QT - 1) / QT;
    int id = blockIdx.x;
    tile = id % tpb; id /= tpb;
    const int blk = id % nblk;
    bh = id / nblk;
    const int b0 = blk * pl.blk;
    qlo = b0 + tile * QT;
    qhi = min(min(b0 + pl.blk, pl.N), qlo + QT);
    if (qlo >= qhi) return;
    k0 = b0;
  } else {
    const int nseg = pl.lev_nseg[lev];
    const int m = pl.lev_m[lev];
    const int spp = (m + QT - 1) / QT + C;
    int id = blockIdx.x;
    const int slot = id % spp; id /= spp;
    const int t = id % nseg;
    bh = id / nseg;
    const int p = pl.lev_pfirst[lev] + t;
    ap = bh * pl.P + p;
    const Geom gm = prob_geom(pl, p);
    Cq = min(C, gm.qn);
    Ck = min(C, gm.kn);
    k0 = gm.k0;
    q0 = gm.q0;
    const int32_t* qoffs = b.qs.offs + (size_t)ap * (C + 1);
    // tiles per query cluster and their prefix (one wave scans 4 per lane)
    if (tid < 64) {
      int v[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid * 4 + q;
        v[q] = c < Cq ? (qoffs[c + 1] - qoffs[c] + QT - 1) / QT : 0;
        sum += v[q];
      }
      int inc = sum;
      for (int mm = 1; mm < 64; mm <<= 1) {
        const int o = __shfl_up(inc, mm, 64);
        if (tid >= mm) inc += o;
      }
      int run = inc - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid * 4 + q;
        if (c < Cq && v[q] > 0 && slot >= run && slot < run + v[q]) {
          sm.sel[0] = c;
          sm.sel[1] = slot - run;
        }
        run += v[q];
      }
      if (tid == 63) sm.sel[2] = inc;
    }
    __syncthreads();
    if (slot >= sm.sel[2]) return;
    I = sm.sel[0];
    tile = sm.sel[1];
    qlo = qoffs[I] + tile * QT;
    qhi = min(qoffs[I + 1], qlo + QT);
    const int bq = bh / pl.Hq, hq = bh % pl.Hq;
    kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
    kp = kvh * pl.P + p;
  }
  if (MODE == MODE_LOCAL) {
    const int bq = bh / pl.Hq, hq = bh % pl.Hq;
    kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  }
  const TIn* Qh = reinterpret_cast<const TIn*>(b.Q) + (size_t)bh * pl.N * D;
  const TIn* Kh = reinterpret_cast<const TIn*>(b.K) + (size_t)kvh * pl.N * D;
  const TIn* Vh = reinterpret_cast<const TIn*>(b.V) + (size_t)kvh * pl.N * D;

  // query rows of this workgroup
  if (tid < QT) {
    int r = -1;
    if (MODE == MODE_LOCAL) {
      if (qlo + tid < qhi) r = qlo + tid;
    } else {
      if (qlo + tid < qhi) {
        const int32_t* qperm = b.qs.perm + ((size_t)lev * pl.B * pl.Hq + bh) * pl.N + q0;
        r = qperm[qlo + tid];
      }
    }
    sm.qrow[tid] = r;
  }
  int nret = 0;
  if (MODE != MODE_LOCAL) {
    // retrieval list, cumulative sizes; far-field log-weights and 1/n
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    const int32_t* Rr = b.R + ((size_t)ap * C + I) * pl.k1w;
    for (int c = tid; c < MUSE_MAXC; c += NT) {
      float bias = -INFINITY, ninv = 0.f;
      if (c < Ck) {
        const int nc = koffs[c + 1] - koffs[c];
        if (nc > 0) { bias = logf((float)nc); ninv = 1.f / (float)nc; }
      }
      sm.far_bias[c] = bias;
      sm.far_ninv[c] = ninv;
    }
    __syncthreads();
    if (tid < 64) {
      int v[4], cc[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = tid * 4 + q;
        cc[q] = r < pl.k1w ? Rr[r] : -1;
        v[q] = cc[q] >= 0 ? koffs[cc[q] + 1] - koffs[cc[q]] : 0;
        sum += v[q];
      }
      int inc = sum;
      for (int mm = 1; mm < 64; mm <<= 1) {
        const int o = __shfl_up(inc, mm, 64);
        if (tid >= mm) inc += o;
      }
      int run = inc - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = tid * 4 + q;
        if (r < MUSE_MAXC) {
          sm.rc[r] = cc[q];
          sm.rcum[r] = run;
        }
        run += v[q];
      }
      if (tid == 63) sm.rcum[MUSE_MAXC] = inc;
    }
    __syncthreads();
    // retrieved clusters leave the far field
    for (int r = tid; r < pl.k1w; r += NT)
      if (sm.rc[r] >= 0) sm.far_bias[sm.rc[r]] = -INFINITY;
    nret = sm.rcum[MUSE_MAXC];
  }
  __syncthreads();

  // query fragments (B operand of S^T = K Q^T)
  const int myq = sm.qrow[w * 16 + col];
  u16x8 qf[KS][NS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if (myq >= 0) {
      load8_split<TIn, NS>(Qh + (size_t)myq * D + 32 * k + 8 * g, qf[k]);
    } else {
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[k][sp][j] = 0;
    }
  }
  AtState<NS, D> st;
  st.m = -1e30f;
  st.lpart = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (MODE != MODE_LOCAL) {
    // ---- far field: 32 key clusters per tile ----
    const float* mu = b.kst.mu + (size_t)kp * C * D;
    const float* T = b.T + ((size_t)ap * C + I) * D * b.Cp32;
    for (int c0 = 0; c0 < Ck; c0 += AT_KT) {
      for (int idx = tid; idx < AT_KT * (D / 8); idx += NT) {
        const int it = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
        const int c = c0 + it;
        float v[8];
        if (c < Ck) {
          const float* src = mu + (size_t)c * D + e0;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = src[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) split_store<NS>(v[j], &sm.ks[0][it][e0 + j], AT_KT * (D + 8));
      }
      for (int idx = tid; idx < D * (AT_KT / 8); idx += NT) {
        const int d = idx / (AT_KT / 8), cb = (idx % (AT_KT / 8)) * 8;
        const float* src = T + (size_t)d * b.Cp32 + c0 + cb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + cb + j;
          const float ni = (c < Ck) ? sm.far_ninv[c] : 0.f;
          const float v = (c < Ck && sm.far_bias[c] > -INFINITY) ? src[j] * ni : 0.f;
          split_store<NS>(v, &sm.vt[0][d][cb + j], D * (AT_KT + 8));
        }
      }
      if (tid < AT_KT) {
        const int c = c0 + tid;
        sm.bias[tid] = c < Ck ? sm.far_bias[c] : -INFINITY;
      }
      __syncthreads();
      consume_tile<TIn, D, WAVES, false>(sm, qf, st, s, myq);
      __syncthreads();
    }
    // ---- exact attention over the retrieved clusters' keys ----
    const int32_t* kperm = b.ks.perm + ((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + k0;
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    for (int v0 = 0; v0 < nret; v0 += AT_KT) {
      if (tid < AT_KT) {
        const int v = v0 + tid;
        int row = -1;
        if (v < nret) {
          int r = 0;
          while (sm.rcum[r + 1] <= v) ++r;
          row = kperm[koffs[sm.rc[r]] + (v - sm.rcum[r])];
        }
        sm.krow[tid] = row;
        sm.bias[tid] = row >= 0 ? 0.f : -INFINITY;
      }
      __syncthreads();
      stage_rows<TIn, D, WAVES>(sm, Kh, Vh);
      __syncthreads();
      consume_tile<TIn, D, WAVES, false>(sm, qf, st, s, myq);
      __syncthreads();
    }
  } else {
    // ---- local causal block: keys [k0, last query row] ----
    const int klast = qhi - 1;
    for (int j0 = k0; j0 <= klast; j0 += AT_KT) {
      if (tid < AT_KT) {
        const int j = j0 + tid;
        sm.krow[tid] = j <= klast ? j : -1;
        sm.bias[tid] = j <= klast ? 0.f : -INFINITY;
      }
      __syncthreads();
      stage_rows<TIn, D, WAVES>(sm, Kh, Vh);
      __syncthreads();
      consume_tile<TIn, D, WAVES, true>(sm, qf, st, s, myq < 0 ? 0x7fffffff : myq);
      __syncthreads();
    }
  }

  // ---- finish: normalise, write or merge ----
  float l = st.lpart;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (myq < 0) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? st.m + logf(l) : -INFINITY;
  if (MODE == MODE_ACAUSAL) {
    TOut* O = reinterpret_cast<TOut*>(b.O) + ((size_t)bh * pl.N + myq) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) store1<TOut>(O + 16 * dt + 4 * g + i, st.o[dt][i] * inv);
    if (g == 0) b.lse[(size_t)bh * pl.N + myq] = lse;
  } else {
    float* oa = b.oacc + ((size_t)bh * pl.N + myq) * D;
    float* la = b.lacc + (size_t)bh * pl.N + myq;
    if (MODE == MODE_LOCAL) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = st.o[dt] * inv;
      if (g == 0) *la = lse;
    } else {
      if (!(l > 0.f)) return;
      const float lold = *la;
      const float L = fmaxf(lold, lse);
      const float wo = __expf(lold - L), wn = __expf(lse - L);
      const float tot = wo + wn;
      const float fo = wo / tot, fn = wn * inv / tot;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        f32x4 prev = *reinterpret_cast<const f32x4*>(oa + 16 * dt + 4 * g);
        *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = prev * fo + st.o[dt] * fn;
      }
      if (g == 0) *la = L + logf(tot);
    }
  }
}

template <typename TOut>
__global__ void finalize_kernel(const float* oacc, const float* lacc, TOut* O, float* lse,
                                long long rows, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n = rows * D;
  if (i < n) store1<TOut>(O + i, oacc[i]);
  if (i < rows) lse[i] = lacc[i];
}

// ---------------------------------------------------------------------------
template <typename TIn, int D, int WAVES>
static hipError_t attn_level(const Plan& pl, const AttnBufs& b, int lev, hipStream_t st) {
  constexpr int QT = 16 * WAVES;
  const int spp = (pl.lev_m[lev] + QT - 1) / QT + pl.C;
  const long long grid = (long long)pl.B * pl.Hq * pl.lev_nseg[lev] * spp;
  if (grid == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  if (pl.causal)
    attn_kernel<TIn, TIn, D, WAVES, MODE_LEVEL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, lev);
  else
    attn_kernel<TIn, TIn, D, WAVES, MODE_ACAUSAL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, lev);
  MUSE_KT_POST(pl.causal ? "attn_level" : "attn_far_retrieve", st);
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t attn_all(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (pl.causal) {
    constexpr int WAVES = 4, QT = 64;
    const int nblk = (pl.N + pl.blk - 1) / pl.blk;
    const long long grid = (long long)pl.B * pl.Hq * nblk * ((pl.blk + QT - 1) / QT);
    MUSE_KT_PRE(st);
    attn_kernel<TIn, TIn, D, WAVES, MODE_LOCAL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, 0);
    MUSE_KT_POST("attn_local", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int lev = 0; lev < pl.nlev; ++lev) {
    // small query clusters: one wave per workgroup; large: four
    const int avg = pl.lev_m[lev] / (pl.C > 0 ? pl.C : 1);
    e = avg >= 48 ? attn_level<TIn, D, 4>(pl, b, lev, st) : attn_level<TIn, D, 1>(pl, b, lev, st);
    if (e != hipSuccess) return e;
  }
  if (pl.causal) {
    const long long rows = (long long)pl.B * pl.Hq * pl.N;
    const long long n = rows * pl.D;
    MUSE_KT_PRE(st);
    finalize_kernel<TIn><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        b.oacc, b.lacc, reinterpret_cast<TIn*>(b.O), b.lse, rows, pl.D);
    MUSE_KT_POST("finalize", st);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attn(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st) {
  if (dtype == 1) return pl.D == 64 ? attn_all<uint16_t, 64>(pl, b, st) : attn_all<uint16_t, 128>(pl, b, st);
  return pl.D == 64 ? attn_all<float, 64>(pl, b, st) : attn_all<float, 128>(pl, b, st);
}

}  // namespace muse
