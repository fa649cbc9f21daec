// Stage one of the two-stage attention (gist.science page, Technical
// Summary, Core Mechanisms: Hierarchical Two-Stage Attention, Exponential
// Tilting, Retrieval-Augmented Approximation):
//   * score of key cluster c for query cluster I: the log of its monopole
//     tilted mass, sigma_Ic = s nu_I.mu_c + ln n_c;
//   * retrieval set R_I: the top-k1 non-empty key clusters by sigma (ties
//     to the lower index), stored in ascending cluster order;
//   * tilted summaries T_Ic = S_c + s M_c nu_I (dipole evaluated at the
//     query-cluster centroid; newx.sg page, Abstract).
#include "common.h"
#include "launch.h"
#include "vt.h"

namespace muse {

// One wave per (attention problem, query cluster); wave-level only (no
// workgroup barriers), so any workgroup can run it.
__device__ __forceinline__ void score_topk_wave(const Plan& pl, const AttnBufs& b, int wave) {
  const int lane = threadIdx.x & 63;
  const int C = pl.C, D = pl.D;
  const int nprob = pl.B * pl.Hq * pl.P;
  if (wave >= nprob * C) return;
  const int ap = wave / C, I = wave % C;
  const int bh = ap / pl.P, p = ap % pl.P;
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kv = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  const size_t kp = (size_t)kv * pl.P + p;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn), Ck = min(C, gm.kn);
  int32_t* R = b.R + ((size_t)ap * C + I) * pl.k1w;
  const int32_t* qoffs = b.qs.offs + (size_t)ap * (C + 1);
  const int mI = I < Cq ? qoffs[I + 1] - qoffs[I] : 0;
  if (mI == 0) {
    for (int q = lane; q < pl.k1w; q += 64) R[q] = -1;
    return;
  }
  const float s = pl.scale;
  const float* nu = b.qs.cent + ((size_t)ap * C + I) * D;
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  float sig[4];
  bool sel[4];
  int nvalid = 0;
  int ncs[4];
  float dots[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = lane + 64 * r;
    ncs[r] = c < Ck ? koffs[c + 1] - koffs[c] : 0;
  }
  // nu_I is read by every lane (same addresses), mu_c by its own lane
  for (int e = 0; e < D; e += 4) {
    const f32x4 nv = *reinterpret_cast<const f32x4*>(nu + e);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (ncs[r] > 0) {
        const f32x4 mv = *reinterpret_cast<const f32x4*>(b.kst.mu + (kp * C + lane + 64 * r) * D + e);
        dots[r] = fmaf(nv[0], mv[0], fmaf(nv[1], mv[1], fmaf(nv[2], mv[2], fmaf(nv[3], mv[3], dots[r]))));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sig[r] = -INFINITY;
    sel[r] = false;
    if (ncs[r] > 0) {
      sig[r] = s * dots[r] + logf((float)ncs[r]);
      nvalid++;
    }
  }
  for (int m = 32; m >= 1; m >>= 1) nvalid += __shfl_xor(nvalid, m, 64);
  const int k1 = min(pl.topk, nvalid);
  for (int round = 0; round < k1; ++round) {
    float bv = -INFINITY;
    int bc = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = lane + 64 * r;
      if (!sel[r] && sig[r] > -INFINITY && (sig[r] > bv || (sig[r] == bv && c < bc))) {
        bv = sig[r];
        bc = c;
      }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      float ov = __shfl_xor(bv, m, 64);
      int oc = __shfl_xor(bc, m, 64);
      if (ov > bv || (ov == bv && oc < bc)) { bv = ov; bc = oc; }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lane + 64 * r == bc) sel[r] = true;
  }
  // ascending order: position = number of selected clusters with lower index
  int base = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    unsigned long long bal = __ballot(sel[r]);
    const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (sel[r]) R[base + __popcll(bal & lt)] = lane + 64 * r;
    base += __popcll(bal);
  }
  for (int q = base + lane; q < pl.k1w; q += 64) R[q] = -1;
}

__global__ void __launch_bounds__(256) score_topk_kernel(Plan pl, AttnBufs b) {
  score_topk_wave(pl, b, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// Same scores and sets for top-k1 <= KMAX: one workgroup per attention
// problem and one thread per query cluster.  The key centroids are staged in
// LDS once (fp32) and read by every thread as broadcasts; each thread forms
// its scores in the same order of operations as above and keeps its KMAX
// best in registers (clusters visited in ascending order, a later cluster
// displaces only a strictly smaller score, so ties keep the lower index).
template <int D, int KMAX>
__global__ void __launch_bounds__(256) score_topk_rows_kernel(Plan pl, AttnBufs b) {
  extern __shared__ __align__(16) float mus[];   // [C][D] centroids of the key problem
  const int C = pl.C;
  const int ap = blockIdx.x;
  const int bh = ap / pl.P, p = ap % pl.P;
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kv = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  const size_t kp = (size_t)kv * pl.P + p;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn), Ck = min(C, gm.kn);
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const float* mu = b.kst.mu + kp * (size_t)C * D;
  for (int idx = threadIdx.x; idx < Ck * (D / 4); idx += blockDim.x)
    reinterpret_cast<f32x4*>(mus)[idx] = reinterpret_cast<const f32x4*>(mu)[idx];
  __syncthreads();
  for (int I = threadIdx.x; I < C; I += blockDim.x) {
    int32_t* R = b.R + ((size_t)ap * C + I) * pl.k1w;
    const int32_t* qoffs = b.qs.offs + (size_t)ap * (C + 1);
    const int mI = I < Cq ? qoffs[I + 1] - qoffs[I] : 0;
    if (mI == 0 || pl.topk <= 0) {
      for (int q = 0; q < pl.k1w; ++q) R[q] = -1;
      continue;
    }
    const float s = pl.scale;
    const float* nu = b.qs.cent + ((size_t)ap * C + I) * D;
    f32x4 nv[D / 4];
#pragma unroll
    for (int e = 0; e < D / 4; ++e) nv[e] = reinterpret_cast<const f32x4*>(nu)[e];
    float bv[KMAX];
    int bc[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { bv[j] = -INFINITY; bc[j] = -1; }
    const int k1 = min(pl.topk, KMAX);
    for (int c = 0; c < Ck; ++c) {
      const int nc = koffs[c + 1] - koffs[c];
      if (nc <= 0) continue;
      float dot = 0.f;
      const f32x4* mr = reinterpret_cast<const f32x4*>(mus + (size_t)c * D);
#pragma unroll
      for (int e = 0; e < D / 4; ++e) {
        const f32x4 mv = mr[e];
        dot = fmaf(nv[e][0], mv[0], fmaf(nv[e][1], mv[1], fmaf(nv[e][2], mv[2], fmaf(nv[e][3], mv[3], dot))));
      }
      const float x = s * dot + logf((float)nc);
      // insert into the descending list (slots >= k1 stay empty)
      if (x > bv[k1 - 1]) {
#pragma unroll
        for (int j = KMAX - 1; j > 0; --j) {
          const bool up = x > bv[j - 1];          // x goes above slot j-1: shift it down
          const bool here = !up && x > bv[j];     // x lands in slot j
          if (j < k1) {
            bv[j] = up ? bv[j - 1] : here ? x : bv[j];
            bc[j] = up ? bc[j - 1] : here ? c : bc[j];
          }
        }
        if (x > bv[0]) { bv[0] = x; bc[0] = c; }
      }
    }
    // ascending cluster order
#pragma unroll
    for (int i = 1; i < KMAX; ++i)
#pragma unroll
      for (int j = KMAX - 1; j >= i; --j) {
        const int lo = bc[j - 1], hi = bc[j];
        const bool sw = (unsigned)lo > (unsigned)hi;   // -1 (empty) sorts last
        bc[j - 1] = sw ? hi : lo;
        bc[j] = sw ? lo : hi;
      }
    for (int q = 0; q < pl.k1w; ++q) R[q] = q < KMAX ? bc[q] : -1;
  }
}

template <int D>
static hipError_t score_rows(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  const long long nprob = (long long)pl.B * pl.Hq * pl.P;
  const size_t smem = (size_t)pl.C * D * sizeof(float);
  const int nt = pl.C <= 64 ? 64 : pl.C <= 128 ? 128 : 256;
  if (pl.topk <= 8) {
    set_smem_once((const void*)score_topk_rows_kernel<D, 8>, (size_t)MUSE_MAXC * D * sizeof(float));
    score_topk_rows_kernel<D, 8><<<(unsigned)nprob, nt, smem, st>>>(pl, b);
  } else {
    set_smem_once((const void*)score_topk_rows_kernel<D, 16>, (size_t)MUSE_MAXC * D * sizeof(float));
    score_topk_rows_kernel<D, 16><<<(unsigned)nprob, nt, smem, st>>>(pl, b);
  }
  return hipGetLastError();
}

hipError_t launch_score_topk(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  const long long waves = (long long)pl.B * pl.Hq * pl.P * pl.C;
  if (waves == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  hipError_t e;
  // one workgroup per problem needs enough problems to fill the chip
  if (pl.topk <= 16 && (long long)pl.B * pl.Hq * pl.P >= 512) {
    e = pl.D == 64 ? score_rows<64>(pl, b, st) : score_rows<128>(pl, b, st);
  } else {
    score_topk_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(pl, b);
    e = hipGetLastError();
  }
  MUSE_KT_POST("score_topk", st);
  return e;
}

// ---------------------------------------------------------------------------
// T[ap][I][d][c] = (S[kp][c][d] + s sum_e M[kp][d][c][e] nu[ap][I][e]) / n_c
// One workgroup per (key problem, query head of its group, block of tb value
// dims d): for fixed d this is a (clusters c) x (query clusters I) product
// over the key dim e, with A = rows of M (registers) and B = nu^T (staged in
// LDS).  Small workgroups keep many in flight per CU, which hides the load
// latency of each; the workgroups of one key problem run on one XCD, so the
// query heads of its group re-read M from that XCD's L2.  Columns c in
// [C, Cp) are written as zeros.
// ---------------------------------------------------------------------------
constexpr int TILT_IC = 128;   // query clusters staged at a time

template <typename TIn, int D, int NS>
struct alignas(16) TiltSmem {
  uint16_t nu[NS][TILT_IC][D + 8];   // nu rows of one query problem, bf16 parts
};

// Value dims d0 .. d0+nd-1 of T for the staged query clusters [i0, i0 + 16 nit):
// jobs of NT2 16-cluster tiles (A = rows of M in registers).  With NT2 = 2 a
// job covers 32 consecutive clusters and MFMA row r of tile h is cluster
// 8(r/4) + 4h + r%4 of the job, so the accumulator rows a lane holds (4g ..
// 4g+3 of both tiles) are the eight consecutive clusters 8g .. 8g+7: a store
// writes 64 contiguous bytes of each of 16 rows (bf16) with no lane exchange;
// with NT2 = 1 a lane stores its four clusters.  When there are fewer pairs than waves, pairs
// would split the query clusters between waves and load each M row twice, so
// small cluster counts take NT2 = 1.  Every read stays in range (clusters past
// Ck read cluster Ck - 1, offsets past Ck offset Ck) and is issued before any
// is used; the next dim's M rows and value sums are read while this dim's
// products are formed and stored.
template <typename TIn, int D, int NS, int NT2, typename SM>
__device__ __forceinline__ void tilt_dims(const SM& sm, const float* Mk, const float* Sk, const int32_t* koffs,
                                          TIn* T, int d0, int nd, int C, int Ck, int Cp, int Cq, int i0, int nit,
                                          float s) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int njob = Cp / (16 * NT2);
  for (int job = w; job < njob; job += 4) {
    // the cluster of MFMA row r of tile h
    auto clu = [&](int h, int r) __attribute__((always_inline)) {
      return NT2 == 2 ? 32 * job + 8 * (r >> 2) + 4 * h + (r & 3) : 16 * job + r;
    };
    // the lane's four clusters of each tile (the same for every dim)
    int o0[NT2][4], o1[NT2][4];
#pragma unroll
    for (int h = 0; h < NT2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = clu(h, 4 * g + i);
        o0[h][i] = koffs[min(c, Ck)];
        o1[h][i] = koffs[min(c + 1, Ck)];
      }
    // raw M rows of one dim (A row: cluster) and the value sums of its clusters
    f32x4 mr[NT2][KS][2];
    float sr[NT2][4];
    auto fetch = [&](int d) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < NT2; ++h) {
        const int cr = max(min(clu(h, col), Ck - 1), 0);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const float* src = Mk + ((size_t)d * C + cr) * D + 32 * k + 8 * g;
          mr[h][k][0] = *reinterpret_cast<const f32x4*>(src);
          mr[h][k][1] = *reinterpret_cast<const f32x4*>(src + 4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = max(min(clu(h, 4 * g + i), Ck - 1), 0);
          sr[h][i] = Sk[(size_t)c * D + d];
        }
      }
    };
    fetch(d0);
    float inv[NT2][4];
#pragma unroll
    for (int h = 0; h < NT2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = clu(h, 4 * g + i);
        const int nc = c < Ck ? o1[h][i] - o0[h][i] : 0;
        inv[h][i] = nc > 0 ? 1.f / (float)nc : 0.f;
      }
    for (int dd = 0; dd < nd; ++dd) {
      const int d = d0 + dd;
      u16x8 a[NT2][KS][NS];
      float sv[NT2][4];
#pragma unroll
      for (int h = 0; h < NT2; ++h) {
        const bool live = clu(h, col) < Ck;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = live ? mr[h][k][j >> 2][j & 3] : 0.f;
            uint16_t hh, m, l;
            split3(v, hh, m, l);
            a[h][k][0][j] = NS == 1 ? f2bf(v) : hh;
            if (NS > 1) { a[h][k][NS > 1 ? 1 : 0][j] = m; a[h][k][NS > 2 ? 2 : 0][j] = l; }
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[h][i] = inv[h][i] > 0.f ? sr[h][i] : 0.f;
      }
      if (dd + 1 < nd) fetch(d + 1);
      // this lane's store address for query cluster i0 + col, stepped by 16
      // query clusters per iteration
      TIn* dst = T + ((size_t)(i0 + col) * D + d) * Cp + 16 * NT2 * job + (NT2 == 2 ? 8 : 4) * g;
      const size_t dstep = (size_t)16 * D * Cp;
      for (int it = 0; it < nit; ++it, dst += dstep) {
        f32x4 acc[NT2];
#pragma unroll
        for (int h = 0; h < NT2; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          u16x8 bb[NS];
#pragma unroll
          for (int sp = 0; sp < NS; ++sp)
            bb[sp] = *reinterpret_cast<const u16x8*>(&sm.nu[sp][16 * it + col][32 * k + 8 * g]);
#pragma unroll
          for (int h = 0; h < NT2; ++h) acc[h] = mfma_split<NS, NS>(a[h][k], bb, acc[h]);
        }
        // lane (col, g) holds MFMA rows 4g .. 4g+3 of each tile (clusters
        // clu(h, 4g + i)) for query cluster i0 + 16 it + col, WB dwords per tile
        constexpr int WB = sizeof(TIn) == 2 ? 2 : 4;
        uint32_t pw[NT2][WB];
#pragma unroll
        for (int h = 0; h < NT2; ++h) {
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = (sv[h][i] + s * acc[h][i]) * inv[h][i];
          if constexpr (sizeof(TIn) == 2) {
            pw[h][0] = pk_bf16(o[0], o[1]);
            pw[h][1] = pk_bf16(o[2], o[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[h][i] = __float_as_uint(o[i]);
          }
        }
        const int I = i0 + 16 * it + col;
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        if constexpr (NT2 == 1) {
          if (I < Cq) {
            if constexpr (sizeof(TIn) == 2) *reinterpret_cast<u32x2*>(dst) = u32x2{pw[0][0], pw[0][1]};
            else *reinterpret_cast<u32x4*>(dst) = u32x4{pw[0][0], pw[0][1], pw[0][2], pw[0][3]};
          }
        } else {
          // tile 0 holds clusters 8g .. 8g+3 of the job, tile 1 8g+4 .. 8g+7
          const uint32_t (&f)[NT2][WB] = pw;
          if (I < Cq) {
            if constexpr (sizeof(TIn) == 2) {
              *reinterpret_cast<u32x4*>(dst) = u32x4{f[0][0], f[0][1], f[1][0], f[1][1]};
            } else {
              *reinterpret_cast<u32x4*>(dst) = u32x4{f[0][0], f[0][1], f[0][2], f[0][3]};
              *reinterpret_cast<u32x4*>(dst + 4) = u32x4{f[1][0], f[1][1], f[1][2], f[1][3]};
            }
          }
        }
      }
    }
  }
}

// Workgroup blk of the tilt grid (the grid's XCD order: blk % 8 = XCD).
template <typename TIn, int D, int NS>
__device__ __forceinline__ void tilt_block(const Plan& pl, const AttnBufs& b, int tb, long long kps, int blk,
                                           TiltSmem<TIn, D, NS>& sm) {
  const int NDB = D / tb;
  const int C = pl.C, Cp = b.Cp32, Gq = pl.Hq / pl.Hkv;
  const int per = Gq * NDB;                       // workgroups per key problem
  const int xcd = blk % 8, loc = blk / 8;
  const long long kp = (long long)(loc / per) * 8 + xcd;
  if (kp >= kps) return;
  const int u = loc % per;
  const int db = u % NDB, hl = u / NDB;
  const int kvh = (int)(kp / pl.P), p = (int)(kp % pl.P);
  const int bq = kvh / pl.Hkv, kh = kvh % pl.Hkv;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn), Ck = min(C, gm.kn);
  const int tid = threadIdx.x;
  const float s = pl.dipole ? pl.scale : 0.f;
  const float* Mk = b.kst.M + kp * (size_t)D * C * D;     // [d][c][e]
  const float* Sk = b.kst.S + kp * (size_t)C * D;         // [c][d]
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const size_t ap = (size_t)(bq * pl.Hq + kh * Gq + hl) * pl.P + p;
  const float* nu = b.qs.cent + ap * (size_t)C * D;        // [I][e]
  TIn* T = reinterpret_cast<TIn*>(b.T) + ap * (size_t)C * D * Cp;   // [I][d][c]
  for (int i0 = 0; i0 < Cq; i0 += TILT_IC) {
    const int nit = (min(TILT_IC, Cq - i0) + 15) / 16;
    __syncthreads();
    // nu rows, four 8-element pieces per thread in flight at a time (rows
    // past Cq read row Cq - 1 and stage zeros)
    const int npc = nit * 16 * (D / 8);
    for (int idx0 = 0; idx0 < npc; idx0 += 4 * 256) {
      f32x4 x[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = min(idx0 + u * 256 + tid, npc - 1);
        const int I = min(i0 + idx / (D / 8), Cq - 1), e0 = (idx % (D / 8)) * 8;
        x[u][0] = *reinterpret_cast<const f32x4*>(nu + (size_t)I * D + e0);
        x[u][1] = *reinterpret_cast<const f32x4*>(nu + (size_t)I * D + e0 + 4);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = idx0 + u * 256 + tid;
        if (idx < npc) {
          const int r = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
          const bool live = i0 + r < Cq;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            split_store<NS>(live ? x[u][j >> 2][j & 3] : 0.f, &sm.nu[0][r][e0 + j], TILT_IC * (D + 8));
        }
      }
    }
    __syncthreads();
    if (Cp >= 128) tilt_dims<TIn, D, NS, 2>(sm, Mk, Sk, koffs, T, db * tb, tb, C, Ck, Cp, Cq, i0, nit, s);
    else tilt_dims<TIn, D, NS, 1>(sm, Mk, Sk, koffs, T, db * tb, tb, C, Ck, Cp, Cq, i0, nit, s);
  }
}

template <typename TIn, int D, int NS>
__global__ void __launch_bounds__(256) tilt_kernel(Plan pl, AttnBufs b, int tb, long long kps) {
  extern __shared__ __align__(16) unsigned char tilt_raw[];
  tilt_block<TIn, D, NS>(pl, b, tb, kps, (int)blockIdx.x, *reinterpret_cast<TiltSmem<TIn, D, NS>*>(tilt_raw));
}

// Scores / top-k, tilted summaries and the dim-major value copies in one
// launch (they are independent): the first nsb workgroups score (4 waves
// each), the next ntb tilt, the rest transpose values through the same LDS.
// nsb is a multiple of 8, so the tilt workgroups keep their XCD order.
template <typename TIn, int D, int NS>
__global__ void __launch_bounds__(256) score_tilt_kernel(Plan pl, AttnBufs b, int tb, long long kps, int nsb,
                                                         int ntb, int nsorted, int sfirst) {
  extern __shared__ __align__(16) unsigned char st_raw[];
  const int blk = (int)blockIdx.x;
  if (blk < nsb) {
    score_topk_wave(pl, b, blk * 4 + (threadIdx.x >> 6));
    return;
  }
  if (blk < nsb + ntb) {
    tilt_block<TIn, D, NS>(pl, b, tb, kps, blk - nsb, *reinterpret_cast<TiltSmem<TIn, D, NS>*>(st_raw));
    return;
  }
  vt_block<TIn, D>(pl, b.kst.Vp, b.V, b.Vt, b.Nv, nsorted, sfirst, blk - nsb - ntb,
                   reinterpret_cast<TIn(*)[D + 2]>(st_raw));
}

template <typename TIn, int D, int NS>
static void tilt_go(const Plan& pl, const AttnBufs& b, long long kps, int tb, hipStream_t st) {
  using SM = TiltSmem<TIn, D, NS>;
  const int per = (pl.Hq / pl.Hkv) * (pl.D / tb);
  const unsigned grid = (unsigned)(((kps + 7) / 8) * 8 * per);
  set_smem_once((const void*)tilt_kernel<TIn, D, NS>, sizeof(SM));
  tilt_kernel<TIn, D, NS><<<grid, 256, sizeof(SM), st>>>(pl, b, tb, kps);
}

// value dims per tilt workgroup: up to 4, fewer when that leaves the chip under-filled
static int tilt_dims(const Plan& pl, long long kps) {
  const long long heads = kps * (pl.Hq / pl.Hkv);
  int tb = 4;
  while (tb > 1 && heads * (pl.D / tb) < 2048) tb /= 2;
  return tb;
}

template <typename TIn, int D, int NS>
static void score_tilt_go(const Plan& pl, const AttnBufs& b, long long kps, int tb, int nsb, hipStream_t st) {
  constexpr size_t smem = std::max(sizeof(TiltSmem<TIn, D, NS>), sizeof(TIn) * VT_ROWS * (D + 2));
  const int per = (pl.Hq / pl.Hkv) * (pl.D / tb);
  const int ntb = (int)(((kps + 7) / 8) * 8 * per);
  const VtGeo g = vt_geo(pl, b.Nv);
  const unsigned grid = (unsigned)(nsb + ntb + (long long)g.nslice * g.nb);
  set_smem_once((const void*)score_tilt_kernel<TIn, D, NS>, smem);
  score_tilt_kernel<TIn, D, NS><<<grid, 256, smem, st>>>(pl, b, tb, kps, nsb, ntb, g.nsorted, g.sfirst);
}

hipError_t launch_tilt(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st) {
  const long long kps = (long long)pl.B * pl.Hkv * pl.P;
  if (kps == 0) return hipSuccess;
  const int tb = tilt_dims(pl, kps);
  MUSE_KT_PRE(st);
  if (dtype == 1) {
    if (pl.D == 64) tilt_go<uint16_t, 64, 1>(pl, b, kps, tb, st);
    else tilt_go<uint16_t, 128, 1>(pl, b, kps, tb, st);
  } else {
    if (pl.D == 64) tilt_go<float, 64, 3>(pl, b, kps, tb, st);
    else tilt_go<float, 128, 3>(pl, b, kps, tb, st);
  }
  MUSE_KT_POST("tilt", st);
  return hipGetLastError();
}

// Scores / top-k, tilted summaries and (vt_done) the dim-major value copies of
// a forward.  They are independent, so they share one launch, except when the
// per-problem score kernel applies.
hipError_t launch_score_tilt(const Plan& pl, int dtype, const AttnBufs& b, bool& vt_done, hipStream_t st) {
  vt_done = false;
  const long long waves = (long long)pl.B * pl.Hq * pl.P * pl.C;
  const long long kps = (long long)pl.B * pl.Hkv * pl.P;
  const bool rows = pl.topk <= 16 && (long long)pl.B * pl.Hq * pl.P >= 512;
  if (rows || waves == 0 || kps == 0) {
    const hipError_t e = launch_score_topk(pl, b, st);
    if (e != hipSuccess) return e;
    return launch_tilt(pl, dtype, b, st);
  }
  const int tb = tilt_dims(pl, kps);
  const int nsb = (int)(((waves + 3) / 4 + 7) / 8 * 8);   // score workgroups, a multiple of 8
  MUSE_KT_PRE(st);
  if (dtype == 1) {
    if (pl.D == 64) score_tilt_go<uint16_t, 64, 1>(pl, b, kps, tb, nsb, st);
    else score_tilt_go<uint16_t, 128, 1>(pl, b, kps, tb, nsb, st);
  } else {
    if (pl.D == 64) score_tilt_go<float, 64, 3>(pl, b, kps, tb, nsb, st);
    else score_tilt_go<float, 128, 3>(pl, b, kps, tb, nsb, st);
  }
  MUSE_KT_POST("score_tilt", st);
  vt_done = true;
  return hipGetLastError();
}

}  // namespace muse
