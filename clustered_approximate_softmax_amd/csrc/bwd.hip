// Backward of the MuSe forward with the cluster assignments, retrieval sets
// and counts held fixed (the differentiable path of the two-stage attention:
// gist.science page, Technical Summary, Core Mechanisms; newx.sg page,
// Abstract: monopole + dipole summaries, causal hierarchy).
//
// A far-field item (cluster c seen from query cluster I) behaves exactly
// like a key with row mu_c, value T_Ic / n_c and log-weight ln n_c, so the
// softmax-backward formulas give, per query i and item x with
// p = exp(logit - lse_i) and dl = p (dO_i . value_x - Delta_i):
//   dq_i += s sum_x dl k_x;  "dk_x" = s sum_i dl q_i;  "dv_x" = sum_i p dO_i.
// For a far item, "dk" is the gradient of mu_c through its logits and
// "dv" / n_c is dT_Ic.  The summaries are then differentiated through
// T_Ic = S_c + s M_c nu_I, S_c = sum v_j, M_c = sum v_j (k_j - mu_c)^T,
// mu_c = mean k_j and nu_I = mean q_i.
//
// Kernels, per causal level in order (every output row is owned by one
// workgroup per launch, so there are no atomics and the result does not
// depend on scheduling):
//   bwd_q       query-centric: dq_i over far, retrieved and local items
//   bwd_kv      item-centric: dk, dv of retrieved keys (gathered over every
//               query cluster of the query-head group that retrieved them)
//               and of local causal blocks
//   bwd_far     dT / mu-gradient partials of the far items, one workgroup
//               per block of clusters looping over several query clusters
//   reduce_k    dmu_c (far logits) per key cluster from the far pass's
//               per-block partials (and dS_c without the dipole term)
//   gemm dM     dM_c = s sum_I dT_Ic nu_I^T         (split-bf16 MFMA),
//               and dS_c = sum_I dT_Ic from the same pass over dT
//   gemm dnu    dnu_I = s sum_c M_c^T dT_Ic          (split-bf16 MFMA)
//   spread_q    dq_i += dnu_I / m_I
//   bcast_k     dk_j += dM_c^T (v_j - S_c/n_c) + dmu_c / n_c,
//               dv_j += dS_c + dM_c (k_j - mu_c)
#include "common.h"
#include "launch.h"

namespace muse {

constexpr float B_LOG2E = 1.4426950408889634f;
constexpr int QB = 32;   // queries per tile in the item-centric kernel

template <typename TIn>
struct BwdTraits {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;   // bf16 parts per operand
  static constexpr int BT = sizeof(TIn) == 2 ? 64 : 32; // items per query-centric tile
};


// 8 floats (contraction slots in order) -> NS bf16 parts
template <int NS>
__device__ __forceinline__ void pack8(const float* x, u16x8* out) {
  if constexpr (NS == 1) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 w = {pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]), pk_bf16(x[6], x[7])};
    out[0] = __builtin_bit_cast(u16x8, w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t h, m, l;
      split3(x[j], h, m, l);
      out[0][j] = h;
      out[1][j] = m;
      if (NS > 2) out[2][j] = l;
    }
  }
}

template <int NS>
__device__ __forceinline__ void zero8(u16x8* out) {
#pragma unroll
  for (int sp = 0; sp < NS; ++sp)
#pragma unroll
    for (int j = 0; j < 8; ++j) out[sp][j] = 0;
}

// position of item r (0..31 of a 32-item block) in contraction-slot order
__device__ __forceinline__ int slot_of(int r) {
  return r < 16 ? 8 * (r / 4) + (r % 4) : 8 * ((r - 16) / 4) + 4 + (r % 4);
}

// wave-0 scan over per-cluster tile counts: the (cluster, tile) of `slot`.
// sel[0] = cluster, sel[1] = the tile's first row (offs[cluster] + tile * tile
// size), sel[2] = total tiles, sel[3] = the cluster's end (offs[cluster + 1]).
__device__ __forceinline__ void find_slot(const int32_t* offs, int Cn, int tile, int slot, int* sel) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    // every offset is read unconditionally (clusters past Cn read cluster
    // Cn - 1), so the reads are one round trip
    int lo[4], hi[4], v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = max(min(tid * 4 + q, Cn - 1), 0);
      lo[q] = offs[c];
      hi[q] = offs[c + 1];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = tid * 4 + q < Cn ? (hi[q] - lo[q] + tile - 1) / tile : 0;
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
      if (v[q] > 0 && slot >= run && slot < run + v[q]) {
        sel[0] = tid * 4 + q;
        sel[1] = lo[q] + (slot - run) * tile;
        sel[3] = hi[q];
      }
      run += v[q];
    }
    if (tid == 63) sel[2] = inc;
  }
}

struct BwdArgs {
  Plan pl;
  AttnBufs a;
  const void* dO;
  const float* lse;
  float* delta;   // [B*Hq][N]
  float* dq;      // [B*Hq][N][D]   fp32 accumulators
  float* dk;      // [B*Hkv][N][D]
  float* dv;
  // per-level buffers; lp = bh * nseg + t, kl = kvh * nseg + t
  void* dT;       // [lp][C][D][C]   (I, d, c): sum_i p dO_i / n_c over far items, input dtype
  float* G;       // [lp][nib][C][D] (block of query clusters, c, e): s sum_{I in block} sum_i dl q_i over far items
  float* dnu;     // [lp][C][D]
  float* dS;      // [kl][C][D]
  float* dmu;     // [kl][C][D]
  float* dM;      // [kl][D][C][D]   (d, c, e)
};

// ===========================================================================
// Delta_i = dO_i . O_i ; zero fill ; fp32 -> output dtype
// ===========================================================================
// D / 8 consecutive lanes per row, 8 elements each (coalesced rows), summed
// across the row's lanes by shuffles in a fixed order
template <typename TIn, int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const TIn* O, const TIn* dO, float* delta, long long rows) {
  constexpr int TPR = D / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long r = gid / TPR;
  const int e = (int)(gid % TPR) * 8;
  float s = 0.f;
  if (r < rows) {
    float a[8], b[8];
    load8_f32<TIn>(O + r * D + e, a);
    load8_f32<TIn>(dO + r * D + e, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(a[j], b[j], s);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (r < rows && e == 0) delta[r] = s;
}

__global__ void bwd_zero_kernel(float* p, long long n) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 3 < n) *reinterpret_cast<f32x4*>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  else for (long long k = i; k < n; ++k) p[k] = 0.f;
}

// fp32 accumulators to the output dtype, 8 elements per thread (n8 = n / 8)
template <typename TOut>
__global__ void __launch_bounds__(256) bwd_out_kernel(const float* src, TOut* dst, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + 8 * i + 4);
  if constexpr (sizeof(TOut) == 2) {
    *reinterpret_cast<u16x8*>(dst + 8 * i) =
        u16x8{f2bf(a[0]), f2bf(a[1]), f2bf(a[2]), f2bf(a[3]), f2bf(b[0]), f2bf(b[1]), f2bf(b[2]), f2bf(b[3])};
  } else {
    *reinterpret_cast<f32x4*>(dst + 8 * i) = a;
    *reinterpret_cast<f32x4*>(dst + 8 * i + 4) = b;
  }
}

// ===========================================================================
// Query-centric kernel: 64 queries (4 waves x 16) against tiles of BT items.
// S^T = K Q^T and dP^T = V dO^T (items as rows), dS^T = P^T (dP^T - Delta),
// dQ^T += K^T dS^T.
// ===========================================================================
enum { BQ_PROBLEM = 0, BQ_LOCAL = 1 };

template <typename TIn, int D>
struct alignas(16) BqSmem {
  static constexpr int NS = BwdTraits<TIn>::NS, BT = BwdTraits<TIn>::BT;
  uint16_t ks[NS][BT][D + 8];    // K rows
  uint16_t vs[NS][BT][D + 8];    // V rows
  uint16_t kt[NS][D][BT + 8];    // K^T in contraction-slot order
  float bias[BT];
  int32_t irow[BT];              // item -> source row, -1 if none
  int32_t qrow[64];
  float far_bias[MUSE_MAXC];
  int32_t rbeg[MUSE_MAXC];
  int32_t rcum[MUSE_MAXC + 1];
  int32_t sel[4];
};

// Stage BT items: rows of K and V, and K^T.  Far items: rows of mu_c and
// columns of T / n_c (stored (d, c)).
template <typename TIn, int D, int NT>
__device__ __forceinline__ void bq_stage(BqSmem<TIn, D>& sm, bool far, const TIn* Kb, const TIn* Vb,
                                         const TIn* mu, const TIn* T, int Cp, int c0, int Ck) {
  using SM = BqSmem<TIn, D>;
  constexpr int NS = SM::NS, BT = SM::BT;
  if constexpr (NS == 1) {
    // bf16: raw 16-byte row chunks; K^T as 4-item runs in slot order
    for (int idx = threadIdx.x; idx < (BT / 4) * (D / 8); idx += NT) {
      const int kb = idx % (BT / 4), e0 = (idx / (BT / 4)) * 8;
      // every read in range (absent items read row / cluster 0, or the last
      // cluster) and issued in one group; absent items are zeroed after
      u16x8 kr[4], vr[4];
      bool ok[4];
      if (far) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = c0 + 4 * kb + r;
          ok[r] = c < Ck;
          kr[r] = *reinterpret_cast<const u16x8*>(mu + (size_t)max(min(c, Ck - 1), 0) * D + e0);
        }
        // T / n_c is stored (d, c): four consecutive clusters per dim
        u16x4 t4[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t4[j] = *reinterpret_cast<const u16x4*>(T + (size_t)(e0 + j) * Cp + c0 + 4 * kb);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) vr[r][j] = t4[j][r];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = sm.irow[4 * kb + r];
          ok[r] = row >= 0;
          kr[r] = *reinterpret_cast<const u16x8*>(Kb + (size_t)max(row, 0) * D + e0);
          vr[r] = *reinterpret_cast<const u16x8*>(Vb + (size_t)max(row, 0) * D + e0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (!ok[r]) vr[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!ok[r]) kr[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      const int pos = 32 * ((4 * kb) / 32) + slot_of((4 * kb) % 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u16x8*>(&sm.ks[0][4 * kb + r][e0]) = kr[r];
        *reinterpret_cast<u16x8*>(&sm.vs[0][4 * kb + r][e0]) = vr[r];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u16x4*>(&sm.kt[0][e0 + j][pos]) = u16x4{kr[0][j], kr[1][j], kr[2][j], kr[3][j]};
    }
    return;
  }
  for (int idx = threadIdx.x; idx < (BT / 4) * (D / 8); idx += NT) {
    const int kb = idx % (BT / 4), e0 = (idx / (BT / 4)) * 8;
    float kv[4][8], vv[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int it = 4 * kb + r;
      const TIn* kp = nullptr;
      const TIn* vp = nullptr;
      if (far) {
        if (c0 + it < Ck) kp = mu + (size_t)(c0 + it) * D + e0;
      } else {
        const int row = sm.irow[it];
        if (row >= 0) { kp = Kb + (size_t)row * D + e0; vp = Vb + (size_t)row * D + e0; }
      }
      if (kp) {
        load8_f32<TIn>(kp, kv[r]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[r][j] = 0.f;
      }
      if (!far) {
        if (vp) {
          load8_f32<TIn>(vp, vv[r]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) vv[r][j] = 0.f;
        }
      }
    }
    if (far) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const TIn* tp = T + (size_t)(e0 + j) * Cp + c0 + 4 * kb;
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r][j] = load1_f32<TIn>(tp + r);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int it = 4 * kb + r;
      const int pos = 32 * (it / 32) + slot_of(it % 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        split_store<NS>(kv[r][j], &sm.ks[0][it][e0 + j], BT * (D + 8));
        split_store<NS>(vv[r][j], &sm.vs[0][it][e0 + j], BT * (D + 8));
        split_store<NS>(kv[r][j], &sm.kt[0][e0 + j][pos], D * (BT + 8));
      }
    }
  }
}

// WAVES waves of 16 queries each (one wave for small query clusters)
template <typename TIn, int D, int MODE, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) bwd_q_kernel(BwdArgs A, int lev) {
  using SM = BqSmem<TIn, D>;
  constexpr int NS = SM::NS, BT = SM::BT, KS = D / 32, DT = D / 16, RT = BT / 16, PS = BT / 32;
  constexpr int NT = 64 * WAVES, QT = 16 * WAVES;
  extern __shared__ __align__(16) unsigned char bq_raw[];
  SM& sm = *reinterpret_cast<SM*>(bq_raw);
  const Plan& pl = A.pl;
  const AttnBufs& b = A.a;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
  const float s = pl.scale, s2 = pl.scale * B_LOG2E;
  const int C = pl.C;
  int bh, ap = 0, I = 0, Ck = 0, q0 = 0, k0 = 0, qlo, qhi;
  if (MODE == BQ_LOCAL) {
    const int nblk = (pl.N + pl.blk - 1) / pl.blk, tpb = (pl.blk + QT - 1) / QT;
    int id = blockIdx.x;
    const int tile = id % tpb; id /= tpb;
    const int blk = id % nblk;
    bh = id / nblk;
    k0 = blk * pl.blk;
    qlo = k0 + tile * QT;
    qhi = min(min(k0 + pl.blk, pl.N), qlo + QT);
    if (qlo >= qhi) return;
  } else {
    const int nseg = pl.lev_nseg[lev], m = pl.lev_m[lev];
    const int spp = (m + QT - 1) / QT + C;
    int id = blockIdx.x;
    const int slot = id % spp; id /= spp;
    const int t = id % nseg;
    bh = id / nseg;
    const int p = pl.lev_pfirst[lev] + t;
    ap = bh * pl.P + p;
    const Geom gm = prob_geom(pl, p);
    const int Cq = min(C, gm.qn);
    Ck = min(C, gm.kn);
    k0 = gm.k0;
    q0 = gm.q0;
    const int32_t* qoffs = b.qs.offs + (size_t)ap * (C + 1);
    find_slot(qoffs, Cq, QT, slot, sm.sel);
    __syncthreads();
    if (slot >= sm.sel[2]) return;
    I = __builtin_amdgcn_readfirstlane(sm.sel[0]);
    qlo = __builtin_amdgcn_readfirstlane(sm.sel[1]);
    qhi = min(__builtin_amdgcn_readfirstlane(sm.sel[3]), qlo + QT);
  }
  const int kvh = (bh / pl.Hq) * pl.Hkv + ((bh % pl.Hq) * pl.Hkv) / pl.Hq;
  const int kp = kvh * pl.P + (ap % pl.P);
  // query rows (one per thread of wave 0), far-item counts and the retrieved
  // list: every read in range and issued before any is used
  int qrow_t = -1;
  if (MODE == BQ_LOCAL) {
    qrow_t = qlo + tid < qhi ? qlo + tid : -1;
  } else {
    const int v = b.qs.perm[((size_t)lev * pl.B * pl.Hq + bh) * pl.N + q0 + min(qlo + tid, qhi - 1)];
    qrow_t = qlo + tid < qhi ? v : -1;
  }
  int nfar = 0, nret = 0;
  if (MODE != BQ_LOCAL) {
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    const int32_t* Rr = b.R + ((size_t)ap * C + I) * pl.k1w;
    constexpr int FBN = (MUSE_MAXC + NT - 1) / NT;
    int kn0[FBN], kn1[FBN];
#pragma unroll
    for (int i = 0; i < FBN; ++i) {
      const int c = tid + i * NT;
      kn0[i] = koffs[min(c, Ck)];
      kn1[i] = koffs[min(c + 1, Ck)];
    }
    int cc[4];
    if (tid < 64) {
      int v[4], bg[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = tid * 4 + q;
        const int rv = Rr[min(r, pl.k1w - 1)];
        cc[q] = r < pl.k1w ? rv : -1;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ci = min(max(cc[q], 0), C - 1);
        const int a = koffs[ci], e = koffs[ci + 1];
        bg[q] = cc[q] >= 0 ? a : 0;
        v[q] = cc[q] >= 0 ? e - a : 0;
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
        sm.rbeg[r] = bg[q];
        sm.rcum[r] = run;
        run += v[q];
      }
      if (tid == 63) sm.rcum[MUSE_MAXC] = inc;
    }
#pragma unroll
    for (int i = 0; i < FBN; ++i) {
      const int c = tid + i * NT;
      const int nc = kn1[i] - kn0[i];
      if (c < MUSE_MAXC) sm.far_bias[c] = c < Ck && nc > 0 ? __log2f((float)nc) : -INFINITY;
    }
    if (tid < 64) sm.qrow[tid] = qrow_t;
    __syncthreads();
    // retrieved clusters leave the far field
    if (tid < 64) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (cc[q] >= 0) sm.far_bias[cc[q]] = -INFINITY;
    }
    nret = sm.rcum[MUSE_MAXC];
    nfar = (Ck + BT - 1) / BT;
  } else {
    nret = qhi - k0;
    if (tid < 64) sm.qrow[tid] = qrow_t;
  }
  __syncthreads();
  const TIn* Qh = reinterpret_cast<const TIn*>(b.Q) + (size_t)bh * pl.N * D;
  const TIn* dOh = reinterpret_cast<const TIn*>(A.dO) + (size_t)bh * pl.N * D;
  const int myq = sm.qrow[w * 16 + col];
  // the query rows are a prefix of the tile: a wave past it stages items with
  // the others but has nothing to contract (local-block tiles are full)
  const bool wlive = MODE == BQ_LOCAL || 16 * w < qhi - qlo;
  u16x8 qf[KS][NS], df[KS][NS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    if (myq >= 0) {
      load8_split<TIn, NS>(Qh + (size_t)myq * D + 32 * k + 8 * g, qf[k]);
      load8_split<TIn, NS>(dOh + (size_t)myq * D + 32 * k + 8 * g, df[k]);
    } else {
      zero8<NS>(qf[k]);
      zero8<NS>(df[k]);
    }
  }
  const float lse2 = myq >= 0 ? A.lse[(size_t)bh * pl.N + myq] * B_LOG2E : 0.f;
  const float dlt = myq >= 0 ? A.delta[(size_t)bh * pl.N + myq] : 0.f;
  f32x4 dqt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const TIn* Kb;
  const TIn* Vb;
  const TIn* mu = nullptr;
  const TIn* T = nullptr;
  if (MODE == BQ_LOCAL) {
    Kb = reinterpret_cast<const TIn*>(b.K) + (size_t)kvh * pl.N * D;
    Vb = reinterpret_cast<const TIn*>(b.V) + (size_t)kvh * pl.N * D;
  } else {
    const size_t kb = (((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + k0) * D;
    Kb = reinterpret_cast<const TIn*>(b.kst.Kp) + kb;
    Vb = reinterpret_cast<const TIn*>(b.kst.Vp) + kb;
    mu = reinterpret_cast<const TIn*>(b.kst.mu_in) + (size_t)kp * C * D;
    T = reinterpret_cast<const TIn*>(b.T) + ((size_t)ap * C + I) * D * b.Cp32;
  }
  const int nex = (nret + BT - 1) / BT;
  for (int t = 0; t < nfar + nex; ++t) {
    const bool far = t < nfar;
    const int base = (far ? t : t - nfar) * BT;
    if (tid < BT) {
      const int it = base + tid;
      int row = -1;
      float bias = -INFINITY;
      if (far) {
        bias = it < Ck ? sm.far_bias[it] : -INFINITY;
      } else if (MODE == BQ_LOCAL) {
        if (it < nret) { row = k0 + it; bias = 0.f; }
      } else if (it < nret) {
        int r = 0;
        while (sm.rcum[r + 1] <= it) ++r;
        row = sm.rbeg[r] + (it - sm.rcum[r]);
        bias = 0.f;
      }
      sm.irow[tid] = row;
      sm.bias[tid] = bias;
    }
    __syncthreads();
    bq_stage<TIn, D, NT>(sm, far, Kb, Vb, mu, T, b.Cp32, base, Ck);
    __syncthreads();
    if (!wlive) {
      __syncthreads();
      continue;
    }
    float ds[RT * 4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u16x8 ak[NS], av[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
          ak[sp] = *reinterpret_cast<const u16x8*>(&sm.ks[sp][16 * rt + col][32 * k + 8 * g]);
          av[sp] = *reinterpret_cast<const u16x8*>(&sm.vs[sp][16 * rt + col][32 * k + 8 * g]);
        }
        sc = mfma_split<NS, NS>(ak, qf[k], sc);
        dp = mfma_split<NS, NS>(av, df[k], dp);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int it = 16 * rt + 4 * g + i;
        float x = fmaf(s2, sc[i], sm.bias[it]);
        // local block: key row k0 + base + it is visible to query myq when <= myq
        if (MODE == BQ_LOCAL && k0 + base + it > myq) x = -INFINITY;
        const float p = myq >= 0 ? __builtin_amdgcn_exp2f(x - lse2) : 0.f;
        ds[rt * 4 + i] = p * (dp[i] - dlt);
      }
    }
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      u16x8 db[NS];
      pack8<NS>(&ds[ps * 8], db);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u16x8 a[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
          a[sp] = *reinterpret_cast<const u16x8*>(&sm.kt[sp][16 * dt + col][32 * ps + 8 * g]);
        dqt[dt] = mfma_split<NS, NS>(a, db, dqt[dt]);
      }
    }
    __syncthreads();
  }
  if (myq < 0) return;
  float* dq = A.dq + ((size_t)bh * pl.N + myq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const f32x4 prev = *reinterpret_cast<const f32x4*>(dq + 16 * dt + 4 * g);
    *reinterpret_cast<f32x4*>(dq + 16 * dt + 4 * g) = prev + dqt[dt] * s;
  }
}

// ===========================================================================
// Item-centric kernel: a workgroup owns 64 items (4 waves x 16) and streams
// the queries that see them in tiles of QB.  S = Q K^T, dP = dO V^T (queries
// as rows), dS = P (dP - Delta), dV^T += dO^T P, dK^T += Q^T dS.
// ===========================================================================
// far items have a kernel of their own; BK_STREAM is BK_EXACT with the
// retrieving query clusters' queries as one stream (levels of small query
// clusters, where one stream per query cluster would leave most of each
// query tile empty)
enum { BK_EXACT = 0, BK_STREAM = 1, BK_LOCAL = 2 };

template <typename TIn, int D>
struct alignas(16) BkSmem {
  static constexpr int NS = BwdTraits<TIn>::NS;
  uint16_t qs[NS][QB][D + 8];     // Q rows
  uint16_t os[NS][QB][D + 8];     // dO rows
  uint16_t qt[NS][D][QB + 8];     // Q^T, slot order
  uint16_t ot[NS][D][QB + 8];     // dO^T, slot order
  float lse2[QB];
  float dlt[QB];
  int32_t qrow[QB];
  int32_t list[256];              // (query head, query cluster) pairs retrieving the cluster
  int32_t cum[257];               // their first position in the combined query stream
  int32_t hq0[256];               // their first q_perm position
  int32_t hbh[256];               // their query head
  int32_t wc[4];
  int32_t sel[4];
};

// fp32 inputs: rows sm.qrow[0 .. QB) of Qh / dOh (-1 for none) into LDS as
// split-bf16 parts, rows and slot-order transposes (bf16 inputs stage through
// the software-pipelined path of bk_query_range)
template <typename TIn, int D, int NT>
__device__ __forceinline__ void bk_stage_queries(BkSmem<TIn, D>& sm, const TIn* Qh, const TIn* dOh,
                                                 const float* lse, const float* delta) {
  constexpr int NS = BkSmem<TIn, D>::NS;
  static_assert(NS > 1, "bf16 inputs take the pipelined staging");
  for (int idx = threadIdx.x; idx < QB * (D / 8); idx += NT) {
    const int q = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
    const int row = sm.qrow[q];
    float qv[8], ov[8];
    if (row >= 0) {
      load8_f32<TIn>(Qh + (size_t)row * D + e0, qv);
      load8_f32<TIn>(dOh + (size_t)row * D + e0, ov);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) { qv[j] = 0.f; ov[j] = 0.f; }
    }
    const int pos = slot_of(q);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      split_store<NS>(qv[j], &sm.qs[0][q][e0 + j], QB * (D + 8));
      split_store<NS>(ov[j], &sm.os[0][q][e0 + j], QB * (D + 8));
      split_store<NS>(qv[j], &sm.qt[0][e0 + j][pos], D * (QB + 8));
      split_store<NS>(ov[j], &sm.ot[0][e0 + j][pos], D * (QB + 8));
    }
  }
  if (threadIdx.x < QB) {
    const int row = sm.qrow[threadIdx.x];
    sm.lse2[threadIdx.x] = row >= 0 ? lse[row] * B_LOG2E : 0.f;
    sm.dlt[threadIdx.x] = row >= 0 ? delta[row] : 0.f;
  }
}

// One query tile against this wave's 16 items (the lane's column).
template <typename TIn, int D, bool CAUSAL>
__device__ __forceinline__ void bk_consume(const BkSmem<TIn, D>& sm,
                                           const u16x8 (&kf)[D / 32][BwdTraits<TIn>::NS],
                                           const u16x8 (&vf)[D / 32][BwdTraits<TIn>::NS], float ibias,
                                           int irow, float s2, f32x4 (&dvt)[D / 16], f32x4 (&dkt)[D / 16]) {
  constexpr int NS = BwdTraits<TIn>::NS, KS = D / 32, DT = D / 16;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  float p[8], dsv[8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u16x8 aq[NS], ad[NS];
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) {
        aq[sp] = *reinterpret_cast<const u16x8*>(&sm.qs[sp][16 * rt + col][32 * k + 8 * g]);
        ad[sp] = *reinterpret_cast<const u16x8*>(&sm.os[sp][16 * rt + col][32 * k + 8 * g]);
      }
      sc = mfma_split<NS, NS>(aq, kf[k], sc);
      dp = mfma_split<NS, NS>(ad, vf[k], dp);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 16 * rt + 4 * g + i;
      const int qr = sm.qrow[q];
      float x = fmaf(s2, sc[i], ibias);
      if (qr < 0 || (CAUSAL && irow > qr)) x = -INFINITY;
      const float pv = __builtin_amdgcn_exp2f(x - sm.lse2[q]);
      p[rt * 4 + i] = pv;
      dsv[rt * 4 + i] = pv * (dp[i] - sm.dlt[q]);
    }
  }
  u16x8 pb[NS], db[NS];
  pack8<NS>(p, pb);
  pack8<NS>(dsv, db);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    u16x8 a[NS], c[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      a[sp] = *reinterpret_cast<const u16x8*>(&sm.ot[sp][16 * dt + col][8 * g]);
      c[sp] = *reinterpret_cast<const u16x8*>(&sm.qt[sp][16 * dt + col][8 * g]);
    }
    dvt[dt] = mfma_split<NS, NS>(a, pb, dvt[dt]);
    dkt[dt] = mfma_split<NS, NS>(c, db, dkt[dt]);
  }
}

// Where a stream position's row index lies: the row is base + *p.
struct RowLoc {
  const int32_t* p;
  int base;
};

// A stream of n queries: query q < n is row base + *p of Qh / dOh / lse /
// delta, {p, base} = row_of(q).  A wave with no valid item (wlive false, the
// small key clusters of the levels that stream) stages its share of every
// tile but skips the contraction.  bf16: software-pipelined.  While tile t is contracted,
// the Q / dO rows and the lse / Delta of tile t+1 are in flight, and the row
// indices of tile t+2 (so that no load waits on another inside an
// iteration).
template <typename TIn, int D, bool CAUSAL, int NT, class RowAt>
__device__ __forceinline__ void bk_query_stream(BkSmem<TIn, D>& sm, const TIn* Qh, const TIn* dOh, const float* lse,
                                                const float* delta, int n, RowAt row_of,
                                                const u16x8 (&kf)[D / 32][BwdTraits<TIn>::NS],
                                                const u16x8 (&vf)[D / 32][BwdTraits<TIn>::NS], float ibias,
                                                int irow, float s2, f32x4 (&dvt)[D / 16], f32x4 (&dkt)[D / 16],
                                                bool wlive) {
  const int qa = 0, qb = n;
  if constexpr (BkSmem<TIn, D>::NS == 1) {
    // staging layout: thread -> 4 queries (block qb4) x 8 dims (e0); the first QB
    // threads also own one query's row index, lse and Delta
    constexpr int NSTG = (QB / 4) * (D / 8);
    static_assert(NSTG <= NT && QB <= NT, "one staging item per thread");
    const int tid = threadIdx.x;
    const bool stg = tid < NSTG;
    const int qb4 = tid % (QB / 4), e0 = (tid / (QB / 4)) * 8;
    const int ntile = (qb - qa + QB - 1) / QB;
    if (n <= 0) return;
    int r1[4], s1 = -1;
    u16x8 qd[4], od[4];
    float l1 = 0.f, d1 = 0.f;
    // the five row indices a thread needs are located first (LDS only), then
    // read together (positions past the stream read its last row's index);
    // the read values stay pending until take_rows needs them
    int v2[5], b2[5];
    bool f2[5];
    auto load_rows = [&](int q0) __attribute__((always_inline)) {
      RowLoc lc[5];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lc[r] = row_of(min(q0 + 4 * qb4 + r, qb - 1));
        f2[r] = stg && q0 + 4 * qb4 + r < qb;
      }
      lc[4] = row_of(min(q0 + tid, qb - 1));
      f2[4] = tid < QB && q0 + tid < qb;
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        b2[u] = lc[u].base;
        v2[u] = *lc[u].p;
      }
    };
    auto take_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) r1[r] = f2[r] ? b2[r] + v2[r] : -1;
      s1 = f2[4] ? b2[4] + v2[4] : -1;
    };
    auto load_data = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        qd[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        od[r] = qd[r];
        if (r1[r] >= 0) {
          qd[r] = *reinterpret_cast<const u16x8*>(Qh + (size_t)r1[r] * D + e0);
          od[r] = *reinterpret_cast<const u16x8*>(dOh + (size_t)r1[r] * D + e0);
        }
      }
      // raw values (row 0's for lanes without a row), scaled and masked when
      // staged, so that nothing here waits for them
      l1 = lse[max(s1, 0)];
      d1 = delta[max(s1, 0)];
    };
    load_rows(qa);
    take_rows();
    load_data();
    if (ntile > 1) load_rows(qa + QB);
    for (int t = 0; t < ntile; ++t) {
      // tile t into LDS
      if (stg) {
        const int pos = slot_of(4 * qb4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<u16x8*>(&sm.qs[0][4 * qb4 + r][e0]) = qd[r];
          *reinterpret_cast<u16x8*>(&sm.os[0][4 * qb4 + r][e0]) = od[r];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          *reinterpret_cast<u16x4*>(&sm.qt[0][e0 + j][pos]) = u16x4{qd[0][j], qd[1][j], qd[2][j], qd[3][j]};
          *reinterpret_cast<u16x4*>(&sm.ot[0][e0 + j][pos]) = u16x4{od[0][j], od[1][j], od[2][j], od[3][j]};
        }
      }
      if (tid < QB) {
        sm.qrow[tid] = s1;
        sm.lse2[tid] = s1 >= 0 ? l1 * B_LOG2E : 0.f;
        sm.dlt[tid] = s1 >= 0 ? d1 : 0.f;
      }
      __syncthreads();
      // tile t+1's rows and scalars, tile t+2's row indices: in flight during the contraction
      if (t + 1 < ntile) {
        take_rows();
        load_data();
        if (t + 2 < ntile) load_rows(qa + (t + 2) * QB);
      }
      if (wlive) bk_consume<TIn, D, CAUSAL>(sm, kf, vf, ibias, irow, s2, dvt, dkt);
      __syncthreads();
    }
  } else {
    for (int q0 = qa; q0 < qb; q0 += QB) {
      if (threadIdx.x < QB) {
        const int q = q0 + threadIdx.x;
        int r = -1;
        if (q < qb) {
          const RowLoc lc = row_of(q);
          r = lc.base + *lc.p;
        }
        sm.qrow[threadIdx.x] = r;
      }
      __syncthreads();
      bk_stage_queries<TIn, D, NT>(sm, Qh, dOh, lse, delta);
      __syncthreads();
      if (wlive) bk_consume<TIn, D, CAUSAL>(sm, kf, vf, ibias, irow, s2, dvt, dkt);
      __syncthreads();
    }
  }
}

// Queries rows[qa .. qb) of head bh (rows == nullptr: rows qa .. qb themselves).
// bf16: software-pipelined.  While tile t is contracted, the Q / dO rows and
// the lse / Delta of tile t+1 are in flight, and the row indices of tile t+2
// (so that no load waits on another inside an iteration).
template <typename TIn, int D, bool CAUSAL, int NT>
__device__ __forceinline__ void bk_query_range(BkSmem<TIn, D>& sm, const BwdArgs& A, int bh, const int32_t* rows,
                                               int qa, int qb, const u16x8 (&kf)[D / 32][BwdTraits<TIn>::NS],
                                               const u16x8 (&vf)[D / 32][BwdTraits<TIn>::NS], float ibias,
                                               int irow, float s2, f32x4 (&dvt)[D / 16], f32x4 (&dkt)[D / 16]) {
  const Plan& pl = A.pl;
  const TIn* Qh = reinterpret_cast<const TIn*>(A.a.Q) + (size_t)bh * pl.N * D;
  const TIn* dOh = reinterpret_cast<const TIn*>(A.dO) + (size_t)bh * pl.N * D;
  const float* lse = A.lse + (size_t)bh * pl.N;
  const float* delta = A.delta + (size_t)bh * pl.N;
  if constexpr (BkSmem<TIn, D>::NS == 1) {
    // staging layout: thread -> 4 queries (block qb4) x 8 dims (e0); the first QB
    // threads also own one query's row index, lse and Delta
    constexpr int NSTG = (QB / 4) * (D / 8);
    static_assert(NSTG <= NT && QB <= NT, "one staging item per thread");
    const int tid = threadIdx.x;
    const bool stg = tid < NSTG;
    const int qb4 = tid % (QB / 4), e0 = (tid / (QB / 4)) * 8;
    const int ntile = (qb - qa + QB - 1) / QB;
    if (qb <= qa) return;
    int r1[4], s1 = -1;
    u16x8 qd[4], od[4];
    float l1 = 0.f, d1 = 0.f;
    // row indices read together (positions past the range read its last one);
    // the read values stay pending until take_rows needs them
    int v2[5];
    bool f2[5];
    auto load_rows = [&](int q0) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = min(q0 + 4 * qb4 + r, qb - 1);
        v2[r] = rows ? rows[q] : q;
        f2[r] = stg && q0 + 4 * qb4 + r < qb;
      }
      const int q = min(q0 + tid, qb - 1);
      v2[4] = rows ? rows[q] : q;
      f2[4] = tid < QB && q0 + tid < qb;
    };
    auto take_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) r1[r] = f2[r] ? v2[r] : -1;
      s1 = f2[4] ? v2[4] : -1;
    };
    auto load_data = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        qd[r] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        od[r] = qd[r];
        if (r1[r] >= 0) {
          qd[r] = *reinterpret_cast<const u16x8*>(Qh + (size_t)r1[r] * D + e0);
          od[r] = *reinterpret_cast<const u16x8*>(dOh + (size_t)r1[r] * D + e0);
        }
      }
      if constexpr (CAUSAL) {
        // local block: scaled and masked here (measured faster in this
        // instantiation, where the deferred form split the row reads above
        // into several waited groups)
        l1 = s1 >= 0 ? lse[s1] * B_LOG2E : 0.f;
        d1 = s1 >= 0 ? delta[s1] : 0.f;
      } else {
        // raw values (row 0's for lanes without a row), scaled and masked
        // when staged, so that nothing here waits for them
        l1 = lse[max(s1, 0)];
        d1 = delta[max(s1, 0)];
      }
    };
    load_rows(qa);
    take_rows();
    load_data();
    if (ntile > 1) load_rows(qa + QB);
    for (int t = 0; t < ntile; ++t) {
      // tile t into LDS
      if (stg) {
        const int pos = slot_of(4 * qb4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<u16x8*>(&sm.qs[0][4 * qb4 + r][e0]) = qd[r];
          *reinterpret_cast<u16x8*>(&sm.os[0][4 * qb4 + r][e0]) = od[r];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          *reinterpret_cast<u16x4*>(&sm.qt[0][e0 + j][pos]) = u16x4{qd[0][j], qd[1][j], qd[2][j], qd[3][j]};
          *reinterpret_cast<u16x4*>(&sm.ot[0][e0 + j][pos]) = u16x4{od[0][j], od[1][j], od[2][j], od[3][j]};
        }
      }
      if (tid < QB) {
        sm.qrow[tid] = s1;
        sm.lse2[tid] = CAUSAL ? l1 : s1 >= 0 ? l1 * B_LOG2E : 0.f;
        sm.dlt[tid] = CAUSAL ? d1 : s1 >= 0 ? d1 : 0.f;
      }
      __syncthreads();
      // tile t+1's rows and scalars, tile t+2's row indices: in flight during the contraction
      if (t + 1 < ntile) {
        take_rows();
        load_data();
        if (t + 2 < ntile) load_rows(qa + (t + 2) * QB);
      }
      bk_consume<TIn, D, CAUSAL>(sm, kf, vf, ibias, irow, s2, dvt, dkt);
      __syncthreads();
    }
  } else {
    for (int q0 = qa; q0 < qb; q0 += QB) {
      if (threadIdx.x < QB) {
        const int q = q0 + threadIdx.x;
        sm.qrow[threadIdx.x] = q < qb ? (rows ? rows[q] : q) : -1;
      }
      __syncthreads();
      bk_stage_queries<TIn, D, NT>(sm, Qh, dOh, lse, delta);
      __syncthreads();
      bk_consume<TIn, D, CAUSAL>(sm, kf, vf, ibias, irow, s2, dvt, dkt);
      __syncthreads();
    }
  }
}

// WAVES waves of 16 items each (one wave for small key clusters)
template <typename TIn, int D, int KIND, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) bwd_kv_kernel(BwdArgs A, int lev) {
  using SM = BkSmem<TIn, D>;
  constexpr int NS = SM::NS, KS = D / 32, DT = D / 16;
  constexpr int NT = 64 * WAVES, IT = 16 * WAVES;
  extern __shared__ __align__(16) unsigned char bk_raw[];
  SM& sm = *reinterpret_cast<SM*>(bk_raw);
  const Plan& pl = A.pl;
  const AttnBufs& b = A.a;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
  const float s = pl.scale, s2 = pl.scale * B_LOG2E;
  const int C = pl.C, Gq = pl.Hq / pl.Hkv;
  int bq = 0, kvh = 0, p = 0, t = 0, nseg = 1, kp = 0, Ck = 0, c = 0, ibeg = 0, iend = 0;
  int blk1 = 0;
  Geom gm{};
  if (KIND == BK_LOCAL) {
    const int nblk = (pl.N + pl.blk - 1) / pl.blk, tpb = (pl.blk + IT - 1) / IT;
    int id = blockIdx.x;
    const int tile = id % tpb; id /= tpb;
    const int blk = id % nblk;
    kvh = id / nblk;
    bq = kvh / pl.Hkv;
    const int blk0 = blk * pl.blk;
    blk1 = min(blk0 + pl.blk, pl.N);
    ibeg = blk0 + tile * IT;
    iend = min(blk1, ibeg + IT);
    if (ibeg >= iend) return;
  } else {
    nseg = pl.lev_nseg[lev];
    const int m = pl.lev_m[lev];
    const int spp = (m + IT - 1) / IT + C;
    int id = blockIdx.x;
    const int slot = id % spp; id /= spp;
    t = id % nseg;
    kvh = id / nseg;
    bq = kvh / pl.Hkv;
    p = pl.lev_pfirst[lev] + t;
    kp = kvh * pl.P + p;
    gm = prob_geom(pl, p);
    Ck = min(C, gm.kn);
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    find_slot(koffs, Ck, IT, slot, sm.sel);
    __syncthreads();
    if (slot >= sm.sel[2]) return;
    c = __builtin_amdgcn_readfirstlane(sm.sel[0]);
    ibeg = __builtin_amdgcn_readfirstlane(sm.sel[1]);
    iend = min(__builtin_amdgcn_readfirstlane(sm.sel[3]), ibeg + IT);
  }

  // ---- this lane's item (wave w owns items 16w .. 16w+15) ----
  const int item = ibeg + 16 * w + col;
  const bool ivalid = item < iend;
  u16x8 kf[KS][NS], vf[KS][NS];
  float ibias = -INFINITY;
  int irow = -1;
  {
    const TIn* kp_ = nullptr;
    const TIn* vp_ = nullptr;
    if (KIND == BK_LOCAL) {
      if (ivalid) {
        kp_ = reinterpret_cast<const TIn*>(b.K) + ((size_t)kvh * pl.N + item) * D;
        vp_ = reinterpret_cast<const TIn*>(b.V) + ((size_t)kvh * pl.N + item) * D;
        irow = item;
        ibias = 0.f;
      }
    } else {
      if (ivalid) {
        const size_t kb = (((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + gm.k0 + item) * D;
        kp_ = reinterpret_cast<const TIn*>(b.kst.Kp) + kb;
        vp_ = reinterpret_cast<const TIn*>(b.kst.Vp) + kb;
        irow = b.ks.perm[((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + gm.k0 + item];
        ibias = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (kp_) load8_split<TIn, NS>(kp_ + 32 * k + 8 * g, kf[k]);
      else zero8<NS>(kf[k]);
      if (vp_) load8_split<TIn, NS>(vp_ + 32 * k + 8 * g, vf[k]);
      else zero8<NS>(vf[k]);
    }
  }
  f32x4 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dkt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- the queries that see these items ----
  if (KIND != BK_LOCAL) {
    // (query head of the group, query cluster) pairs whose retrieval set holds c,
    // scanned in a fixed order, at most 256 per round
    const int Cq = min(C, gm.qn);
    const int total = Gq * Cq;
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < total; base += NT) {
      const int e = base + tid;
      bool hit = false;
      {
        // every read in range (pairs past the total read the last pair, entries
        // past k1 the last entry), eight in flight at a time
        const int ec = min(e, total - 1);
        const int hl = ec / Cq, Iq = ec % Cq;
        const int bhx = bq * pl.Hq + (kvh % pl.Hkv) * Gq + hl;
        const int32_t* Rr = b.R + (((size_t)bhx * pl.P + p) * C + Iq) * pl.k1w;
        for (int r0 = 0; r0 < pl.k1w; r0 += 8) {
          int rv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) rv[u] = Rr[min(r0 + u, pl.k1w - 1)];
#pragma unroll
          for (int u = 0; u < 8; ++u) hit |= rv[u] == c;
        }
        hit = hit && e < total;
      }
      const unsigned long long bal = __ballot(hit);
      if (lane == 0) sm.wc[w] = __popcll(bal);
      __syncthreads();
      int off = 0;
      for (int q = 0; q < w; ++q) off += sm.wc[q];
      if (hit) sm.list[off + __popcll(bal & lt)] = e;
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < WAVES; ++q) cnt += sm.wc[q];
      __syncthreads();
      // the listed pairs' queries as one stream (small clusters then share
      // query tiles): pair li holds stream positions [cum[li], cum[li+1]),
      // its queries at q_perm positions hq0[li] + 0, 1, ... of head hbh[li]
      if (tid < 64) {
        int v[4], pos[4], hb[4], sum = 0;
        // unlisted slots read pair 0's offsets (in range) and count nothing
        int o1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int li = tid * 4 + q;
          const int ent = li < cnt ? sm.list[li] : 0;
          const int hl = ent / Cq, Iq = ent % Cq;
          hb[q] = bq * pl.Hq + (kvh % pl.Hkv) * Gq + hl;
          const int32_t* qoffs = b.qs.offs + ((size_t)hb[q] * pl.P + p) * (C + 1);
          pos[q] = qoffs[Iq];
          o1[q] = qoffs[Iq + 1];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = tid * 4 + q < cnt ? o1[q] - pos[q] : 0;
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
          const int li = tid * 4 + q;
          if (li < cnt) {
            sm.cum[li] = run;
            sm.hq0[li] = pos[q];
            sm.hbh[li] = hb[q];
          }
          run += v[q];
        }
        if (tid == 63) sm.cum[cnt] = inc;
      }
      __syncthreads();
      const int total = sm.cum[cnt];
      const int32_t* permb = b.qs.perm + (size_t)lev * pl.B * pl.Hq * pl.N + gm.q0;
      if constexpr (KIND == BK_STREAM) {
        int hc = 0;   // this thread's cursor: successive lookups move it a few pairs at most
        auto row_of = [&](int v) __attribute__((always_inline)) -> RowLoc {
          // the pair holding stream position v: the last li with cum[li] <= v;
          // its row is base + *p
          while (hc > 0 && sm.cum[hc] > v) --hc;
          while (hc + 1 < cnt && sm.cum[hc + 1] <= v) ++hc;
          const int bhx = sm.hbh[hc];
          return RowLoc{permb + (size_t)bhx * pl.N + sm.hq0[hc] + (v - sm.cum[hc]), bhx * pl.N};
        };
        bk_query_stream<TIn, D, false, NT>(sm, reinterpret_cast<const TIn*>(A.a.Q),
                                           reinterpret_cast<const TIn*>(A.dO), A.lse, A.delta, total, row_of, kf,
                                           vf, ibias, irow, s2, dvt, dkt, 16 * w < iend - ibeg);
      } else {
        // one stream per pair (row indices read straight from q_perm)
        for (int li = 0; li < cnt; ++li) {
          const int bhx = sm.hbh[li], q0 = sm.hq0[li];
          bk_query_range<TIn, D, false, NT>(sm, A, bhx, permb + (size_t)bhx * pl.N, q0,
                                            q0 + sm.cum[li + 1] - sm.cum[li], kf, vf, ibias, irow, s2, dvt, dkt);
        }
      }
      __syncthreads();
    }
  } else {
    // local causal block: the queries from the tile's first row to the block end, every head of the group
    for (int hl = 0; hl < Gq; ++hl) {
      const int bhx = bq * pl.Hq + (kvh % pl.Hkv) * Gq + hl;
      bk_query_range<TIn, D, true, NT>(sm, A, bhx, nullptr, ibeg, blk1, kf, vf, ibias, irow, s2, dvt, dkt);
    }
  }
  if (!ivalid) return;
  // ---- outputs: lane holds dims d = 16dt + 4g + i of its item ----
  {
    float* dk = A.dk + ((size_t)kvh * pl.N + irow) * D;
    float* dv = A.dv + ((size_t)kvh * pl.N + irow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 pk = *reinterpret_cast<const f32x4*>(dk + 16 * dt + 4 * g);
      const f32x4 pv = *reinterpret_cast<const f32x4*>(dv + 16 * dt + 4 * g);
      *reinterpret_cast<f32x4*>(dk + 16 * dt + 4 * g) = pk + dkt[dt] * s;
      *reinterpret_cast<f32x4*>(dv + 16 * dt + 4 * g) = pv + dvt[dt];
    }
  }
}

// Far items: key clusters cb*IT .. cb*IT+IT-1 (row mu_c, value T_Ic / n_c,
// log-weight log n_c, none for retrieved or empty clusters) seen from the
// query clusters I0 .. I0+ig-1 of one (query head, segment).  The clusters'
// centroid rows are loaded once; per query cluster the retrieval bias and
// the value column change, and the cluster's queries stream through LDS.
// Writes dT_Ic (d, c) per query cluster and, for the whole block of query
// clusters, G = s sum_I sum_{i in I} dl_ic q_i (c, e): the mu-gradient is only
// ever needed summed over query clusters.
template <typename TIn, int D, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, sizeof(TIn) == 2 ? 2 : 1) bwd_far_kernel(BwdArgs A, int lev, int ig) {
  using SM = BkSmem<TIn, D>;
  constexpr int NS = SM::NS, KS = D / 32, DT = D / 16;
  constexpr int NT = 64 * WAVES, IT = 16 * WAVES;
  extern __shared__ __align__(16) unsigned char bf_raw[];
  SM& sm = *reinterpret_cast<SM*>(bf_raw);
  // value columns of the block for one query cluster (bf16), item-major
  __shared__ __align__(16) uint16_t tcol[NS == 1 ? IT : 1][D + 8];
  const Plan& pl = A.pl;
  const AttnBufs& b = A.a;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const float s = pl.scale, s2 = pl.scale * B_LOG2E;
  const int C = pl.C, nseg = pl.lev_nseg[lev];
  const int nct = (C + IT - 1) / IT, nib = (C + ig - 1) / ig;
  int id = blockIdx.x;
  const int cb = id % nct; id /= nct;
  const int ib = id % nib; id /= nib;
  const int t = id % nseg, bh = id / nseg;
  const int bq = bh / pl.Hq;
  const int kvh = bq * pl.Hkv + ((bh % pl.Hq) * pl.Hkv) / pl.Hq;
  const int p = pl.lev_pfirst[lev] + t;
  const size_t ap = (size_t)bh * pl.P + p, kp = (size_t)kvh * pl.P + p;
  const Geom gm = prob_geom(pl, p);
  const int Ck = min(C, gm.kn), Cq = min(C, gm.qn);
  const int I0 = ib * ig, I1 = min(Cq, I0 + ig);
  if (I0 >= I1) return;
  // this lane's item (wave w owns items 16w .. 16w+15 of the block)
  const int item = cb * IT + 16 * w + col;
  const bool ivalid = item < C;
  const bool real = item < Ck;
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const int nc = real ? koffs[item + 1] - koffs[item] : 0;
  const float inv = nc > 0 ? 1.f / (float)nc : 0.f;
  const float lw = nc > 0 ? __log2f((float)nc) : -INFINITY;
  u16x8 kf[KS][NS], vf[KS][NS];
  {
    const TIn* kr = reinterpret_cast<const TIn*>(b.kst.mu_in) + (kp * C + item) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (real) load8_split<TIn, NS>(kr + 32 * k + 8 * g, kf[k]);
      else zero8<NS>(kf[k]);
    }
  }
  const int32_t* qoffs = b.qs.offs + ap * (C + 1);
  const int32_t* qperm = b.qs.perm + ((size_t)lev * pl.B * pl.Hq + bh) * pl.N + gm.q0;
  const size_t lp = (size_t)bh * nseg + t;
  f32x4 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma nounroll
  for (int I = I0; I < I1; ++I) {
    // retrieved clusters leave the far field of I
    bool ret = false;
    const int32_t* Rr = b.R + (ap * C + I) * pl.k1w;
    for (int r = 0; r < pl.k1w; ++r) ret |= (Rr[r] == item);
    const float ibias = ret ? -INFINITY : lw;
    // value: column `item` of T_I / n_c, stored (d, c)
    const TIn* T = reinterpret_cast<const TIn*>(b.T) + (ap * C + I) * D * b.Cp32;
    if constexpr (NS == 1) {
      // the block's D x IT values: 16-byte row loads, transposed into LDS
      // (item rows), then 16-byte fragment reads (columns C .. Cp-1 of T are zero)
      const uint16_t* T16 = reinterpret_cast<const uint16_t*>(T) + cb * IT;
      for (int idx = threadIdx.x; idx < D * (IT / 8); idx += NT) {
        const int d = idx / (IT / 8), i0 = (idx % (IT / 8)) * 8;
        const u16x8 v = *reinterpret_cast<const u16x8*>(T16 + (size_t)d * b.Cp32 + i0);
#pragma unroll
        for (int q = 0; q < 8; ++q) tcol[i0 + q][d] = v[q];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KS; ++k) vf[k][0] = *reinterpret_cast<const u16x8*>(&tcol[16 * w + col][32 * k + 8 * g]);
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        float v8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v8[j] = real ? load1_f32<TIn>(T + (size_t)(32 * k + 8 * g + j) * b.Cp32 + item) : 0.f;
        pack8<NS>(v8, vf[k]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dvt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bk_query_range<TIn, D, false, NT>(sm, A, bh, qperm, qoffs[I], qoffs[I + 1], kf, vf, ibias, -1, s2, dvt, dkt);
    if (ivalid) {
      TIn* dT = reinterpret_cast<TIn*>(A.dT) + (lp * C + I) * (size_t)D * C;   // (d, c)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) store1<TIn>(dT + (size_t)(16 * dt + 4 * g + i) * C + item, dvt[dt][i] * inv);
    }
  }
  if (ivalid) {
    float* G = A.G + ((lp * nib + ib) * C + item) * (size_t)D;    // (c, e)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(G + 16 * dt + 4 * g) = dkt[dt] * s;
  }
}

// ===========================================================================
// Batched fp32 contraction on split-bf16 MFMA: C[m][n] = sum_k A[m][k] B[k][n]
// per batch, for the whole n range (N = D) and 128 rows of m per workgroup,
// k in steps of 32, so that the large operand is read once.  Each thread
// loads 16 consecutive floats of A (along k, or along m) and N/8 of B (along
// n) per step; the next step's loads are in flight while the current step
// is contracted.  The problem type supplies the batch view and the row
// loads (zeros outside the operand); per output element the k order is
// ascending in steps of 32, the same for every tiling.
// ===========================================================================
template <int NS>
__device__ __forceinline__ void split_parts(float x, uint16_t* dst, int stride) {
  if constexpr (NS == 1) {
    dst[0] = f2bf(x);
  } else {
    uint16_t h, m, l;
    split3(x, h, m, l);
    dst[0] = h;
    dst[stride] = m;
    if (NS > 2) dst[2 * stride] = l;
  }
}

__device__ __forceinline__ void load4x(const float* p, int n4, float* out) {
  for (int q = 0; q < n4; ++q) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p + 4 * q);
    out[4 * q] = x[0]; out[4 * q + 1] = x[1]; out[4 * q + 2] = x[2]; out[4 * q + 3] = x[3];
  }
}

// 16 consecutive elements of dT (fp32, or bf16 for bf16 inputs) as floats
template <typename DT>
__device__ __forceinline__ void load16(const DT* p, float* out) {
  if constexpr (sizeof(DT) == 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u16x8 x = *reinterpret_cast<const u16x8*>(p + 8 * q);
#pragma unroll
      for (int j = 0; j < 8; ++j) out[8 * q + j] = bf2f(x[j]);
    }
  } else {
    load4x(p, 4, out);
  }
}

constexpr int BG_TM = 128, BG_KT = 32;

template <class P, int NS, int N>
__global__ void __launch_bounds__(256) bwd_gemm_kernel(P prob) {
  static_assert(N == 64 || N == 128, "N is the head dim");
  constexpr int TM = BG_TM, KT = BG_KT, BF = KT * N / 256;   // B floats per thread
  __shared__ __align__(16) uint16_t As[NS][TM][KT + 8];
  __shared__ __align__(16) uint16_t Bs[NS][N][KT + 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
  int id = blockIdx.x;
  const int tm = id % prob.mtiles;
  id /= prob.mtiles;
  typename P::View v;
  prob.view(id, v);
  const int m0 = tm * TM;
  if (m0 >= v.M) return;
  float ra[16], rb[BF];
  auto load = [&](int k0) __attribute__((always_inline)) {
    if constexpr (P::A_KC) prob.a16(v, m0 + tid / 2, k0 + (tid % 2) * 16, ra);   // row m, 16 k
    else prob.a16(v, m0 + (tid % 8) * 16, k0 + tid / 8, ra);                    // 16 m, column k
    prob.bn(v, k0 + tid / 8, (tid % 8) * BF, rb);
  };
  auto stage = [&]() __attribute__((always_inline)) {
    if constexpr (P::A_KC) {
      const int m = tid / 2, kk = (tid % 2) * 16;
#pragma unroll
      for (int j = 0; j < 16; ++j) split_parts<NS>(ra[j], &As[0][m][kk + j], TM * (KT + 8));
    } else {
      const int mm = (tid % 8) * 16, kk = tid / 8;
#pragma unroll
      for (int j = 0; j < 16; ++j) split_parts<NS>(ra[j], &As[0][mm + j][kk], TM * (KT + 8));
    }
    const int kk = tid / 8, nn = (tid % 8) * BF;
#pragma unroll
    for (int j = 0; j < BF; ++j) split_parts<NS>(rb[j], &Bs[0][nn + j][kk], N * (KT + 8));
  };
  // wave w owns rows 32w .. 32w+31 (two row tiles) and every column tile
  f32x4 acc[2][N / 16];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < N / 16; ++q) acc[r][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row sums of A (problems with ROWSUM): this thread's 16 rows over its k
  float rsum[P::ROWSUM ? 16 : 1];
#pragma unroll
  for (int j = 0; j < (P::ROWSUM ? 16 : 1); ++j) rsum[j] = 0.f;
  load(v.K0);
  for (int k0 = v.K0; k0 < v.K; k0 += KT) {
    if constexpr (P::ROWSUM) {
#pragma unroll
      for (int j = 0; j < 16; ++j) rsum[j] += ra[j];
    }
    stage();
    __syncthreads();
    if (k0 + KT < v.K) load(k0 + KT);
    u16x8 a[2][NS];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        a[r][sp] = *reinterpret_cast<const u16x8*>(&As[sp][32 * w + 16 * r + col][8 * g]);
#pragma unroll
    for (int q = 0; q < N / 16; ++q) {
      u16x8 bb[NS];
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) bb[sp] = *reinterpret_cast<const u16x8*>(&Bs[sp][16 * q + col][8 * g]);
#pragma unroll
      for (int r = 0; r < 2; ++r) acc[r][q] = mfma_split<NS, NS>(a[r], bb, acc[r][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < N / 16; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 32 * w + 16 * r + 4 * g + i, n = 16 * q + col;
        if (m < v.M) prob.c(v, m, n, acc[r][q][i]);
      }
  if constexpr (P::ROWSUM) {
    // the 32 threads of a row range (k = tid / 8 mod 32) combine through LDS
    static_assert(!P::A_KC && 32 * TM * 4 <= (int)sizeof(As), "row sums reuse the A stage");
    float* red = reinterpret_cast<float*>(&As[0][0][0]);
    const int mm = (tid % 8) * 16, kq = tid / 8;
#pragma unroll
    for (int j = 0; j < 16; ++j) red[kq * TM + mm + j] = rsum[j];
    __syncthreads();
    if (tid < TM && m0 + tid < v.M) {
      float sum = 0.f;
      for (int q = 0; q < 32; ++q) sum += red[q * TM + tid];
      prob.rowsum(v, m0 + tid, sum);
    }
  }
}

// dnu_I[e] = s sum_{d,c} dT_I[d][c] M[d][c][e]; batch = lp = bh * nseg + t.
// With ksplit > 1 each workgroup contracts one of ksplit ranges of k = (d, c)
// and writes its partial to slab ks of dnu ([ks][lp][I][e]); bwd_dnu_sum then
// adds the slabs into slab 0 in order.
template <typename DT>
struct GemmDnu {
  static constexpr bool A_KC = true, ROWSUM = false;
  Plan pl;
  int lev, mtiles, ksplit;
  const DT* dT;
  const float* Mst;
  float* dnu;
  struct View { int M, K0, K; const DT* A; const float* B; float* C; };
  __device__ void view(int id, View& v) const {
    const int ks = id % ksplit, batch = id / ksplit;
    const int nseg = pl.lev_nseg[lev];
    const int t = batch % nseg, bh = batch / nseg;
    const int p = pl.lev_pfirst[lev] + t;
    const Geom gm = prob_geom(pl, p);
    const int kvh = (bh / pl.Hq) * pl.Hkv + ((bh % pl.Hq) * pl.Hkv) / pl.Hq;
    const size_t kp = (size_t)kvh * pl.P + p;
    v.M = min(pl.C, gm.qn);
    const int kc = pl.D * pl.C / ksplit;   // a multiple of 32
    v.K0 = ks * kc;
    v.K = v.K0 + kc;
    v.A = dT + (size_t)batch * pl.C * pl.D * pl.C;
    v.B = Mst + kp * pl.D * pl.C * pl.D;
    v.C = dnu + ((size_t)ks * pl.B * pl.Hq * nseg + batch) * pl.C * pl.D;
  }
  // A row m, k .. k+15 (K is a multiple of 64)
  __device__ void a16(const View& v, int m, int k, float* out) const {
    if (m < v.M && k < v.K) load16<DT>(v.A + (size_t)m * pl.D * pl.C + k, out);   // rows of D * C
    else for (int j = 0; j < 16; ++j) out[j] = 0.f;
  }
  template <int BF>
  __device__ void bn(const View& v, int k, int n, float (&out)[BF]) const {
    if (k < v.K) load4x(v.B + (size_t)k * pl.D + n, BF / 4, out);
    else for (int j = 0; j < BF; ++j) out[j] = 0.f;
  }
  __device__ void c(const View& v, int m, int n, float x) const { v.C[(size_t)m * pl.D + n] = pl.scale * x; }
};

// dM[d][c][e] = s sum_{h,I} dT_{h,I}[d][c] nu_{h,I}[e]; batch = kl = kvh * nseg + t
template <typename DT>
struct GemmDm {
  // also the row sums of dT over (h, I): dS_c[d] for m = (d, c)
  static constexpr bool A_KC = false, ROWSUM = true;
  Plan pl;
  int lev, mtiles;
  const DT* dT;
  const float* nu;   // query centroids [B*Hq][P][C][D]
  float* dM;
  float* dS;         // [kl][C][D]
  struct View { int M, K0, K, Cq, t, p, bh0, kl; float* C; };
  __device__ void view(int batch, View& v) const {
    const int nseg = pl.lev_nseg[lev];
    const int t = batch % nseg, kvh = batch / nseg;
    const int p = pl.lev_pfirst[lev] + t;
    const Geom gm = prob_geom(pl, p);
    const int Gq = pl.Hq / pl.Hkv;
    v.Cq = min(pl.C, gm.qn);
    v.M = pl.D * pl.C;
    v.K0 = 0;
    v.K = Gq * pl.C;
    v.t = t;
    v.p = p;
    v.bh0 = (kvh / pl.Hkv) * pl.Hq + (kvh % pl.Hkv) * Gq;
    v.kl = batch;
    v.C = dM + (size_t)batch * pl.D * pl.C * pl.D;
  }
  // A rows m .. m+15 of column k = (query head h, query cluster I) (M is a multiple of 64)
  __device__ void a16(const View& v, int m, int k, float* out) const {
    const int h = k / pl.C, I = k % pl.C;
    if (k < v.K && I < v.Cq && m < v.M) {
      const size_t lp = (size_t)(v.bh0 + h) * pl.lev_nseg[lev] + v.t;
      load16<DT>(dT + (lp * pl.C + I) * (size_t)pl.D * pl.C + m, out);
    } else {
      for (int j = 0; j < 16; ++j) out[j] = 0.f;
    }
  }
  template <int BF>
  __device__ void bn(const View& v, int k, int n, float (&out)[BF]) const {
    const int h = k / pl.C, I = k % pl.C;
    if (k < v.K && I < v.Cq) {
      const size_t ap = (size_t)(v.bh0 + h) * pl.P + v.p;
      load4x(nu + (ap * pl.C + I) * pl.D + n, BF / 4, out);
    } else {
      for (int j = 0; j < BF; ++j) out[j] = 0.f;
    }
  }
  __device__ void c(const View& v, int m, int n, float x) const { v.C[(size_t)m * pl.D + n] = pl.scale * x; }
  __device__ void rowsum(const View& v, int m, float x) const {
    const int d = m / pl.C, c = m % pl.C;
    dS[((size_t)v.kl * pl.C + c) * pl.D + d] = x;
  }
};

// ===========================================================================
// dmu_c[e] = sum_{h, blocks} G[c][e] and, when no dM contraction runs (no
// dipole term), dS_c[d] = sum_{h,I} dT_{h,I}[d][c]
// one thread per (kl, index in C*D)
// ===========================================================================
template <typename TIn>
__global__ void __launch_bounds__(256) bwd_reduce_k_kernel(BwdArgs A, int lev, int ig, int with_ds) {
  const Plan& pl = A.pl;
  const int C = pl.C, D = pl.D, Gq = pl.Hq / pl.Hkv;
  const int nseg = pl.lev_nseg[lev];
  const int per = (C * D + 255) / 256;
  const int kl = blockIdx.x / per;
  const int idx = (blockIdx.x % per) * 256 + threadIdx.x;
  if (idx >= C * D) return;
  const int t = kl % nseg, kvh = kl / nseg;
  const int p = pl.lev_pfirst[lev] + t;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn);
  const int bh0 = (kvh / pl.Hkv) * pl.Hq + (kvh % pl.Hkv) * Gq;
  // G holds one partial per block of ig query clusters (blocks that exist)
  const int nib = (C + ig - 1) / ig, nibq = (Cq + ig - 1) / ig;
  float sS = 0.f, sMu = 0.f;
  for (int h = 0; h < Gq; ++h) {
    const size_t lp = (size_t)(bh0 + h) * nseg + t;
    if (with_ds)
      for (int I = 0; I < Cq; ++I)
        sS += load1_f32<TIn>(reinterpret_cast<const TIn*>(A.dT) + (lp * C + I) * (size_t)D * C + idx);
    for (int q = 0; q < nibq; ++q) sMu += A.G[(lp * nib + q) * (size_t)C * D + idx];
  }
  const int d = idx / C, c = idx % C;   // the dT index is (d, c)
  if (with_ds) A.dS[((size_t)kl * C + c) * D + d] = sS;
  A.dmu[(size_t)kl * C * D + idx] = sMu;
}

// dnu partial slabs (split contraction) summed into slab 0 in order; one
// thread per 4 values of a slab
__global__ void __launch_bounds__(256) bwd_dnu_sum_kernel(float* dnu, long long n4, long long slab, int ksplit) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(dnu + 4 * i);
  for (int q = 1; q < ksplit; ++q) v += *reinterpret_cast<const f32x4*>(dnu + q * slab + 4 * i);
  *reinterpret_cast<f32x4*>(dnu + 4 * i) = v;
}

// dq_i += dnu_I / m_I for every query of the level; one thread per (row, 4 dims)
__global__ void __launch_bounds__(256) bwd_spread_q_kernel(BwdArgs A, int lev) {
  const Plan& pl = A.pl;
  const AttnBufs& b = A.a;
  const int D = pl.D, C = pl.C;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = D / 4;
  const long long rowid = gid / per;
  if (rowid >= (long long)pl.B * pl.Hq * pl.N) return;
  const int e0 = (int)(gid % per) * 4;
  const int bh = (int)(rowid / pl.N), r = (int)(rowid % pl.N);
  const int nseg = pl.lev_nseg[lev], m = pl.lev_m[lev];
  int t = 0;
  if (pl.causal) {
    t = r / (2 * m);
    if (t >= nseg || r < 2 * m * t + m) return;
  }
  const int p = pl.lev_pfirst[lev] + t;
  const size_t ap = (size_t)bh * pl.P + p;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn);
  const int I = min(max(b.qs.labels[((size_t)lev * pl.B * pl.Hq + bh) * pl.N + r], 0), Cq - 1);
  const int32_t* qoffs = b.qs.offs + ap * (C + 1);
  const int mI = qoffs[I + 1] - qoffs[I];
  if (mI <= 0) return;
  const float inv = 1.f / (float)mI;
  const size_t lp = (size_t)bh * nseg + t;
  const f32x4 g4 = *reinterpret_cast<const f32x4*>(A.dnu + (lp * C + I) * D + e0);
  float* dq = A.dq + ((size_t)bh * pl.N + r) * D + e0;
  *reinterpret_cast<f32x4*>(dq) = *reinterpret_cast<const f32x4*>(dq) + g4 * inv;
}

// dk_j += dM_c^T (v_j - S_c/n_c) + dmu_c / n_c ; dv_j += dS_c + dM_c (k_j - mu_c)
// one workgroup per (kl, cluster, 64 keys)
template <typename TIn, int D>
struct alignas(16) BcSmem {
  float dM[D][D + 1];     // (value dim d, key dim e)
  float vc[64][D + 4];    // v_j - S_c / n_c
  float kc[64][D + 4];    // k_j - mu_c
  float aux[2][D];        // dS_c, dmu_c / n_c
  int32_t rows[64];
  int32_t sel[4];
};

template <typename TIn, int D, int NT>
__global__ void __launch_bounds__(NT) bwd_bcast_k_kernel(BwdArgs A, int lev) {
  using SM = BcSmem<TIn, D>;
  extern __shared__ __align__(16) unsigned char bc_raw[];
  SM& sm = *reinterpret_cast<SM*>(bc_raw);
  const Plan& pl = A.pl;
  const AttnBufs& b = A.a;
  const int C = pl.C;
  const int nseg = pl.lev_nseg[lev], m = pl.lev_m[lev];
  const int spp = (m + 63) / 64 + C;
  int id = blockIdx.x;
  const int slot = id % spp; id /= spp;
  const int t = id % nseg;
  const int kvh = id / nseg;
  const int p = pl.lev_pfirst[lev] + t;
  const size_t kp = (size_t)kvh * pl.P + p;
  const size_t kl = (size_t)kvh * nseg + t;
  const Geom gm = prob_geom(pl, p);
  const int Ck = min(C, gm.kn);
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const int tid = threadIdx.x;
  find_slot(koffs, Ck, 64, slot, sm.sel);
  __syncthreads();
  if (slot >= sm.sel[2]) return;
  const int c = __builtin_amdgcn_readfirstlane(sm.sel[0]);
  const int beg = __builtin_amdgcn_readfirstlane(sm.sel[1]), end = __builtin_amdgcn_readfirstlane(sm.sel[3]);
  const int cnt = min(end, beg + 64) - beg;
  const float inv = 1.f / (float)(end - koffs[c]);
  const bool dip = pl.dipole != 0;
  if (dip) {
    // D x D floats as 16-byte loads, all of a thread's in flight at once
    constexpr int NL = D * D / 4 / NT;
    f32x4 mv[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = (u * NT + tid) * 4, d = idx / D, e = idx % D;
      mv[u] = *reinterpret_cast<const f32x4*>(&A.dM[((kl * D + d) * C + c) * D + e]);
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = (u * NT + tid) * 4, d = idx / D, e = idx % D;
#pragma unroll
      for (int q = 0; q < 4; ++q) sm.dM[d][e + q] = mv[u][q];
    }
  }
  for (int e = tid; e < D; e += NT) {
    sm.aux[0][e] = A.dS[(kl * C + c) * D + e];
    sm.aux[1][e] = A.dmu[(kl * C + c) * D + e] * inv;
  }
  const size_t rb = ((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + gm.k0 + beg;
  const TIn* Kp = reinterpret_cast<const TIn*>(b.kst.Kp) + rb * D;
  const TIn* Vp = reinterpret_cast<const TIn*>(b.kst.Vp) + rb * D;
  const float* Sc = b.kst.S + (kp * C + c) * D;
  const float* muc = b.kst.mu + (kp * C + c) * D;
  for (int idx = tid; idx < 64 * (D / 8); idx += NT) {
    const int j = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
    float kv[8], vv[8];
    if (j < cnt) {
      load8_f32<TIn>(Kp + (size_t)j * D + e0, kv);
      load8_f32<TIn>(Vp + (size_t)j * D + e0, vv);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) { kv[q] = 0.f; vv[q] = 0.f; }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      sm.kc[j][e0 + q] = kv[q] - muc[e0 + q];
      sm.vc[j][e0 + q] = vv[q] - Sc[e0 + q] * inv;
    }
  }
  if (tid < 64) sm.rows[tid] = tid < cnt ? b.ks.perm[rb + tid] : -1;
  __syncthreads();
  // thread -> output dim e, keys j = grp, grp + NG, ...
  constexpr int NG = NT / D, NJ = 64 / NG;
  const int e = tid % D, grp = tid / D;
  float gk[NJ], gv[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) { gk[q] = sm.aux[1][e]; gv[q] = sm.aux[0][e]; }
  // keys of this thread's group that exist (the rest of the 64 slots are skipped)
  const int nqv = cnt > grp ? (cnt - grp + NG - 1) / NG : 0;
  if (dip && nqv > 0) {
    for (int d = 0; d < D; d += 4) {
      float mc[4], mr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { mc[u] = sm.dM[d + u][e]; mr[u] = sm.dM[e][d + u]; }
#pragma unroll
      for (int q = 0; q < NJ; ++q) {
        if (q >= nqv) break;
        const int j = grp + NG * q;
        const f32x4 vj = *reinterpret_cast<const f32x4*>(&sm.vc[j][d]);
        const f32x4 kj = *reinterpret_cast<const f32x4*>(&sm.kc[j][d]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          gk[q] = fmaf(mc[u], vj[u], gk[q]);
          gv[q] = fmaf(mr[u], kj[u], gv[q]);
        }
      }
    }
  }
  // read every key's running gradients first (keys past cnt read key cnt - 1,
  // cnt >= 1), then add and write
  float ok[NJ], ov[NJ];
  size_t oo[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    const int j = min(grp + NG * q, cnt - 1);
    oo[q] = ((size_t)kvh * pl.N + sm.rows[j]) * D + e;
    ok[q] = A.dk[oo[q]];
    ov[q] = A.dv[oo[q]];
  }
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    if (grp + NG * q >= cnt) continue;
    A.dk[oo[q]] = ok[q] + gk[q];
    A.dv[oo[q]] = ov[q] + gv[q];
  }
}

// ===========================================================================
template <typename TIn, int D>
static hipError_t bwd_all(const BwdArgs& A, void* dQo, void* dKo, void* dVo, hipStream_t st) {
  const Plan& pl = A.pl;
  constexpr int NSG = sizeof(TIn) == 2 ? 2 : 3;   // parts for the cluster-level contractions
  hipError_t e;
  const long long nq = (long long)pl.B * pl.Hq * pl.N, nk = (long long)pl.B * pl.Hkv * pl.N;
  const size_t bq_smem = sizeof(BqSmem<TIn, D>), bk_smem = sizeof(BkSmem<TIn, D>);
  const size_t bc_smem = sizeof(BcSmem<TIn, D>);
  set_smem_once((const void*)bwd_q_kernel<TIn, D, BQ_LOCAL, 4>, bq_smem);
  set_smem_once((const void*)bwd_q_kernel<TIn, D, BQ_PROBLEM, 4>, bq_smem);
  set_smem_once((const void*)bwd_kv_kernel<TIn, D, BK_LOCAL, 4>, bk_smem);
  set_smem_once((const void*)bwd_kv_kernel<TIn, D, BK_EXACT, 4>, bk_smem);
  set_smem_once((const void*)bwd_kv_kernel<TIn, D, BK_STREAM, 4>, bk_smem);
  set_smem_once((const void*)bwd_far_kernel<TIn, D, 4>, bk_smem);
  set_smem_once((const void*)bwd_bcast_k_kernel<TIn, D, 1024>, bc_smem);
  MUSE_KT_PRE(st);
  bwd_zero_kernel<<<(unsigned)((nq * D / 4 + 255) / 256), 256, 0, st>>>(A.dq, nq * D);
  bwd_zero_kernel<<<(unsigned)((nk * D / 4 + 255) / 256), 256, 0, st>>>(A.dk, nk * D);
  bwd_zero_kernel<<<(unsigned)((nk * D / 4 + 255) / 256), 256, 0, st>>>(A.dv, nk * D);
  bwd_delta_kernel<TIn, D><<<(unsigned)((nq * (D / 8) + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const TIn*>(A.a.O), reinterpret_cast<const TIn*>(A.dO), A.delta, nq);
  MUSE_KT_POST("bwd_prep", st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (pl.causal) {
    const long long nblk = (pl.N + pl.blk - 1) / pl.blk, tpb = (pl.blk + 63) / 64;
    MUSE_KT_PRE(st);
    bwd_q_kernel<TIn, D, BQ_LOCAL, 4><<<(unsigned)(pl.B * pl.Hq * nblk * tpb), 256, bq_smem, st>>>(A, 0);
    MUSE_KT_POST("bwd_q_local", st);
    MUSE_KT_PRE(st);
    bwd_kv_kernel<TIn, D, BK_LOCAL, 4><<<(unsigned)(pl.B * pl.Hkv * nblk * tpb), 256, bk_smem, st>>>(A, 0);
    MUSE_KT_POST("bwd_kv_local", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int C = pl.C;
  int msegs = 0;   // the most segments of any level: the per-level buffers hold that many
  for (int l = 0; l < pl.nlev; ++l) msegs = std::max(msegs, pl.lev_nseg[l]);
  for (int lev = 0; lev < pl.nlev; ++lev) {
    const long long nseg = pl.lev_nseg[lev];
    if (nseg == 0) continue;
    const long long m = pl.lev_m[lev];
    const long long spp = (m + 63) / 64 + C;
    static const char* const qn[8] = {"bwd_q_L0", "bwd_q_L1", "bwd_q_L2", "bwd_q_L3", "bwd_q_L4", "bwd_q_L5",
                                      "bwd_q_L6", "bwd_q_L7+"};
    static const char* const kn[8] = {"bwd_kv_L0", "bwd_kv_L1", "bwd_kv_L2", "bwd_kv_L3", "bwd_kv_L4",
                                      "bwd_kv_L5", "bwd_kv_L6", "bwd_kv_L7+"};
    MUSE_KT_PRE(st);
    bwd_q_kernel<TIn, D, BQ_PROBLEM, 4><<<(unsigned)(pl.B * pl.Hq * nseg * spp), 256, bq_smem, st>>>(A, lev);
    MUSE_KT_POST(qn[lev < 7 ? lev : 7], st);
    MUSE_KT_PRE(st);
    // query clusters of fewer than a query tile's rows on average: one query stream per key cluster
    if (m < (long long)QB * C)
      bwd_kv_kernel<TIn, D, BK_STREAM, 4><<<(unsigned)(pl.B * pl.Hkv * nseg * spp), 256, bk_smem, st>>>(A, lev);
    else
      bwd_kv_kernel<TIn, D, BK_EXACT, 4><<<(unsigned)(pl.B * pl.Hkv * nseg * spp), 256, bk_smem, st>>>(A, lev);
    MUSE_KT_POST(kn[lev < 7 ? lev : 7], st);
    MUSE_KT_PRE(st);
    // query clusters per far workgroup: enough workgroups (about 4096) to fill the chip
    const long long pairs = (long long)pl.B * pl.Hq * nseg * ((C + 63) / 64) * C;
    const int ig = (int)std::min<long long>(C, std::max<long long>(1, pairs / 4096));
    bwd_far_kernel<TIn, D, 4><<<(unsigned)(pl.B * pl.Hq * nseg * ((C + 63) / 64) * ((C + ig - 1) / ig)), 256,
                                bk_smem, st>>>(A, lev, ig);
    MUSE_KT_POST("bwd_far", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    MUSE_KT_PRE(st);
    // dS_c comes from the dM contraction when there is one (it reads every dT anyway)
    bwd_reduce_k_kernel<TIn><<<(unsigned)(pl.B * pl.Hkv * nseg * ((C * D + 255) / 256)), 256, 0, st>>>(A, lev, ig,
                                                                                                  pl.dipole ? 0 : 1);
    MUSE_KT_POST("bwd_reduce_k", st);
    if (pl.dipole) {
      GemmDm<TIn> gdm{pl, lev, (D * C + BG_TM - 1) / BG_TM, reinterpret_cast<const TIn*>(A.dT), A.a.qs.cent, A.dM,
                      A.dS};
      MUSE_KT_PRE(st);
      bwd_gemm_kernel<GemmDm<TIn>, NSG, D><<<(unsigned)(pl.B * pl.Hkv * nseg * gdm.mtiles), 256, 0, st>>>(gdm);
      MUSE_KT_POST("bwd_dM", st);
      // split k = (d, c) while the level has few (head, segment) batches: partial
      // slabs fit the buffer (sized for the most segments) and ranges stay whole k steps
      const long long nbat = (long long)pl.B * pl.Hq * nseg * ((C + BG_TM - 1) / BG_TM);
      int ksplit = 1;
      while (nseg * ksplit * 2 <= msegs && nbat * ksplit * 2 <= 1024 && (D * C) % (BG_KT * ksplit * 2) == 0)
        ksplit *= 2;
      GemmDnu<TIn> gdn{pl, lev, (C + BG_TM - 1) / BG_TM, ksplit, reinterpret_cast<const TIn*>(A.dT), A.a.kst.M,
                       A.dnu};
      MUSE_KT_PRE(st);
      bwd_gemm_kernel<GemmDnu<TIn>, NSG, D><<<(unsigned)(nbat * ksplit), 256, 0, st>>>(gdn);
      if (ksplit > 1) {
        const long long slab = (long long)pl.B * pl.Hq * nseg * C * D;
        bwd_dnu_sum_kernel<<<(unsigned)((slab / 4 + 255) / 256), 256, 0, st>>>(A.dnu, slab / 4, slab, ksplit);
      }
      MUSE_KT_POST("bwd_dnu", st);
      MUSE_KT_PRE(st);
      bwd_spread_q_kernel<<<(unsigned)((nq * (D / 4) + 255) / 256), 256, 0, st>>>(A, lev);
      MUSE_KT_POST("bwd_spread_q", st);
    }
    MUSE_KT_PRE(st);
    // 1024 threads: a workgroup holds a cluster's dM (up to 66 KB) and key
    // rows in LDS, so one fits per CU; its 16 waves hide each other's LDS latency
    bwd_bcast_k_kernel<TIn, D, 1024><<<(unsigned)(pl.B * pl.Hkv * nseg * spp), 1024, bc_smem, st>>>(A, lev);
    MUSE_KT_POST("bwd_bcast_k", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  MUSE_KT_PRE(st);
  // rows of D elements: counts of 8-element groups
  bwd_out_kernel<TIn><<<(unsigned)((nq * D / 8 + 255) / 256), 256, 0, st>>>(A.dq, reinterpret_cast<TIn*>(dQo),
                                                                           nq * D / 8);
  bwd_out_kernel<TIn><<<(unsigned)((nk * D / 8 + 255) / 256), 256, 0, st>>>(A.dk, reinterpret_cast<TIn*>(dKo),
                                                                           nk * D / 8);
  bwd_out_kernel<TIn><<<(unsigned)((nk * D / 8 + 255) / 256), 256, 0, st>>>(A.dv, reinterpret_cast<TIn*>(dVo),
                                                                           nk * D / 8);
  MUSE_KT_POST("bwd_out", st);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdLaunch& L, hipStream_t st) {
  BwdArgs A;
  A.pl = L.pl;
  A.a = L.a;
  A.dO = L.dO;
  A.lse = L.lse;
  A.delta = L.delta;
  A.dq = L.dq;
  A.dk = L.dk;
  A.dv = L.dv;
  A.dT = L.dT;
  A.G = L.G;
  A.dnu = L.dnu;
  A.dS = L.dS;
  A.dmu = L.dmu;
  A.dM = L.dM;
  if (L.dtype == 1)
    return L.pl.D == 64 ? bwd_all<uint16_t, 64>(A, L.dQ, L.dK, L.dV, st)
                        : bwd_all<uint16_t, 128>(A, L.dQ, L.dK, L.dV, st);
  return L.pl.D == 64 ? bwd_all<float, 64>(A, L.dQ, L.dK, L.dV, st)
                      : bwd_all<float, 128>(A, L.dQ, L.dK, L.dV, st);
}

}  // namespace muse
