// Causal MuSe on spatial blocks with causally accumulated summaries
// (gist.science page, Technical Summary, Core Mechanisms: Causal
// Accumulation, Retrieval-Augmented Approximation, Exponential Tilting).
//
// Queries and keys are clustered once per head over all N rows (the acausal
// clustering, so the stable cluster-contiguous order keeps every cluster's
// rows ascending).  Block b holds rows [b B, (b + 1) B).  For query cluster
// I (centroid nu_I) and a key set A, the exactly tilted statistics are
//   lnZ = log sum_{j in A} exp(s nu_I.k_j),
//   kappa = sum w_j k_j / sum w_j,  U = sum w_j v_j / sum w_j.
// The group (I, b) -- the queries of cluster I in block b -- retrieves the
// top-k1 key clusters by lnZ over their keys in blocks < b, inside each the
// top-k2 blocks by lnZ over that block's keys (largest first, ties to the
// lower index, empty sets never chosen), attends exactly to those keys and
// to its own block, and sees every other earlier key through one far item
// per key cluster: log-weight lnZ + s (q - nu_I).kappa and value U over the
// cluster's earlier keys minus the retrieved blocks.
//
// Kernels, in launch order:
//   v4_bounds   where each block starts inside every cluster's sorted run
//   v4_part     lnZ, kappa, U of every (I, c, block): an online base-2
//               softmax per lane group over the keys of each (c, block)
//   v4_select   the two-level retrieval of every group: a running prefix
//               of lnZ per key cluster, ranks for k1, and per retrieved
//               cluster k2 rounds of a wave-wide argmax over the blocks
//   v4_far      the far items of every group from the running prefix of
//               the (I, c, block) statistics; a retrieved cluster's item
//               leaves out its retrieved blocks
// The attention pass itself is attn_kernel's MODE_V4.
#include <climits>

#include "common.h"
#include "launch.h"

namespace muse {

constexpr int V4_MAXNB = 4096;   // blocks per sequence (checked on the host)
constexpr float PX_LOG2E = 1.4426950408889634f;
constexpr float PX_LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Block starts: bnd[c][beta] = first position of cluster c's run in the
// sorted order whose row is >= beta B (beta = nb: the run's end).  One
// thread per (set, head, cluster, beta); keys first, then queries.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) v4_bounds_kernel(Plan pl, CSet ks, CSet qs, int32_t* kb, int32_t* qb) {
  const long long nk = (long long)ks.heads * pl.Ck * (pl.nb + 1);
  const long long nq = (long long)qs.heads * pl.Cq * (pl.nb + 1);
  long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= nk + nq) return;
  const bool key = id < nk;
  if (!key) id -= nk;
  const int Cs = key ? pl.Ck : pl.Cq;
  const int beta = (int)(id % (pl.nb + 1));
  const long long hc = id / (pl.nb + 1);
  const int c = (int)(hc % Cs), head = (int)(hc / Cs);
  const int32_t* offs = (key ? ks.offs : qs.offs) + (size_t)head * (pl.C + 1);
  const int32_t* perm = (key ? ks.perm : qs.perm) + (size_t)head * pl.N;
  int lo = offs[c], hi = offs[c + 1];
  const long long lim = (long long)beta * pl.blk;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (perm[mid] < lim) lo = mid + 1;
    else hi = mid;
  }
  (key ? kb : qb)[id] = lo;
}

// E elements of a row as fp32 (E a multiple of 8).
template <typename TIn, int E>
__device__ __forceinline__ void px_load(const TIn* p, float* out) {
  static_assert(E % 8 == 0, "whole 16-byte loads");
  if constexpr (sizeof(TIn) == 2) {
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(p + 8 * i);
#pragma unroll
      for (int j = 0; j < 8; ++j) out[8 * i + j] = __uint_as_float((uint32_t)v[j] << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) out[4 * i + j] = v[j];
    }
  }
}

// x of lane l ^ 1 and of lane l ^ 2 (DPP quad permutations: no LDS trip).
__device__ __forceinline__ float px_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float px_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// fp32 -> input dtype (bf16: round to nearest even), and back.
template <typename TIn>
__device__ __forceinline__ TIn px_round(float x) {
  if constexpr (sizeof(TIn) == 2) {
    const uint32_t u = __float_as_uint(x);
    return (TIn)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  } else {
    return x;
  }
}
template <typename TIn>
__device__ __forceinline__ float px_float(TIn v) {
  if constexpr (sizeof(TIn) == 2) return __uint_as_float((uint32_t)v << 16);
  else return v;
}

// ---------------------------------------------------------------------------
// Statistics of every (I, c, block).  One wave per (q-head, 16 query
// clusters, key cluster): lane = (query cluster il, quarter ds of the
// feature dims); the four quarters' partial dot products are summed across
// lanes, and each lane accumulates its quarter of sum w k and sum w v.
// ---------------------------------------------------------------------------
template <typename TIn, int D>
__global__ void __launch_bounds__(256) v4_part_kernel(Plan pl, AttnBufs b, int nbg) {
  constexpr int E = D / 4, KU = D == 64 ? 2 : 1;
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int Cqe = min(pl.Cq, pl.N), Cke = min(pl.Ck, pl.N);
  const int nIt = (Cqe + 15) / 16;
  if (wave >= (long long)pl.B * pl.Hq * nIt * Cke * nbg) return;   // whole waves: no barriers below
  // the blocks of one (q-head, query-cluster tile, key cluster) are split
  // into nbg ranges, one wave each (the blocks are independent)
  const int bg = (int)(wave % nbg);
  const int c = (int)(wave / nbg % Cke);
  const long long r = wave / nbg / Cke;
  const int it = (int)(r % nIt), bh = (int)(r / nIt);
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  // lane = 4 il + ds: the four quarters of one query cluster are adjacent
  // lanes, summed by in-row lane swaps
  const int il = lane >> 2, ds = lane & 3;
  const int I = it * 16 + il;
  const bool Iok = I < Cqe;
  const float s2 = pl.scale * PX_LOG2E;
  float nu[E];
  {
    const float* nup = b.qs.cent + ((size_t)bh * pl.C + (Iok ? I : 0)) * D + ds * E;
#pragma unroll
    for (int e = 0; e < E; ++e) nu[e] = Iok ? nup[e] * s2 : 0.f;
  }
  const int32_t* kbr = b.kb + ((size_t)kvh * pl.Ck + c) * (pl.nb + 1);
  const TIn* Kp = reinterpret_cast<const TIn*>(b.kst.Kp) + (size_t)kvh * pl.N * D + ds * E;
  const TIn* Vp = reinterpret_cast<const TIn*>(b.kst.Vp) + (size_t)kvh * pl.N * D + ds * E;
  const size_t row = ((size_t)bh * pl.Cq + (Iok ? I : 0)) * pl.Ck + c;   // (I, c): nb entries
  const int be0 = (int)((long long)pl.nb * bg / nbg), be1 = (int)((long long)pl.nb * (bg + 1) / nbg);
  int r1 = kbr[be0];
  for (int beta = be0; beta < be1; ++beta) {
    const int r0 = r1;
    r1 = kbr[beta + 1];
    // sums relative to a reference m that moves only when a logit exceeds
    // it by more than 8 (weights stay below 2^8); KU keys per step
    float m = -INFINITY, z = 0.f, ak[E], au[E];
#pragma unroll
    for (int e = 0; e < E; ++e) { ak[e] = 0.f; au[e] = 0.f; }
    for (int j = r0; j < r1; j += KU) {
      float kx[KU][E], vx[KU][E], d[KU];
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        const int jr = min(j + k, r1 - 1);
        px_load<TIn, E>(Kp + (size_t)jr * D, kx[k]);
        px_load<TIn, E>(Vp + (size_t)jr * D, vx[k]);
      }
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        d[k] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) d[k] = fmaf(nu[e], kx[k][e], d[k]);
      }
#pragma unroll
      for (int k = 0; k < KU; ++k) d[k] += px_xor1(d[k]);
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        d[k] += px_xor2(d[k]);
        if (j + k >= r1) d[k] = -INFINITY;
      }
      float dm = d[0];
#pragma unroll
      for (int k = 1; k < KU; ++k) dm = fmaxf(dm, d[k]);
      if (dm > m + 8.f) {
        const float sc = __builtin_amdgcn_exp2f(m - dm);
        z *= sc;
#pragma unroll
        for (int e = 0; e < E; ++e) { ak[e] *= sc; au[e] *= sc; }
        m = dm;
      }
#pragma unroll
      for (int k = 0; k < KU; ++k) {
        const float p = __builtin_amdgcn_exp2f(d[k] - m);
        z += p;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ak[e] = fmaf(p, kx[k][e], ak[e]);
          au[e] = fmaf(p, vx[k][e], au[e]);
        }
      }
    }
    if (Iok) {
      const bool ne = r1 > r0;
      const float inv = ne ? 1.f / z : 0.f;
      if (ds == 0) b.pz[row * pl.nb + beta] = ne ? (m + __log2f(z)) * PX_LN2 : -INFINITY;
      float* pk = b.pk + (row * pl.nb + beta) * D + ds * E;
      float* pu = b.pu + (row * pl.nb + beta) * D + ds * E;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        *reinterpret_cast<f32x4*>(pk + e) = f32x4{ak[e], ak[e + 1], ak[e + 2], ak[e + 3]} * inv;
        *reinterpret_cast<f32x4*>(pu + e) = f32x4{au[e], au[e + 1], au[e + 2], au[e + 3]} * inv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Two-level retrieval of every group (I, b).  One workgroup per (q-head, I);
// thread c keeps the running lnZ of key cluster c over the blocks before b.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) v4_select_kernel(Plan pl, AttnBufs b) {
  __shared__ float bsc[4][V4_MAXNB];   // per wave: block scores of the cluster it ranks (-inf: not a candidate)
  __shared__ float sz[MUSE_MAXC];
  __shared__ int32_t selc[MUSE_MAXC];
  __shared__ int32_t wcnt[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int Cke = min(pl.Ck, pl.N);
  const int bh = blockIdx.x / pl.Cq, I = blockIdx.x % pl.Cq;
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  const int c = tid;
  const bool cok = c < Cke;
  const int32_t* kbr = b.kb + ((size_t)kvh * pl.Ck + (cok ? c : 0)) * (pl.nb + 1);
  const int kb0 = cok ? kbr[0] : 0;
  const size_t irow = (size_t)bh * pl.Cq + I;
  const float* pzr = b.pz + (irow * pl.Ck + (cok ? c : 0)) * pl.nb;
  const int32_t* qbr = b.qb + irow * (pl.nb + 1);
  const int k1 = min(pl.topk, Cke);
  const int k12 = pl.k1w * pl.k2w;
  const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  float run = -INFINITY;
  float znext = cok ? pzr[0] : -INFINITY;   // block bb - 1's ln Z, loaded one block ahead
  for (int bb = 0; bb < pl.nb; ++bb) {
    if (bb >= 1 && cok) {
      const float z2 = znext;
      znext = pzr[bb];
      if (z2 > -INFINITY) {
        const float zm = fmaxf(run, z2);
        run = zm + __logf(__expf(run - zm) + __expf(z2 - zm));
      }
    }
    int32_t* R1 = b.r1 + (irow * pl.nb + bb) * pl.k1w;
    int32_t* R2 = b.r2 + (irow * pl.nb + bb) * k12;
    const bool hasq = bb >= 1 && qbr[bb + 1] > qbr[bb];
    if (!hasq || k1 == 0) {
      for (int j = tid; j < pl.k1w; j += 256) R1[j] = -1;
      for (int j = tid; j < k12; j += 256) R2[j] = -1;
      continue;
    }
    // top-k1 clusters among those with keys before block bb
    const bool valid = cok && kbr[bb] > kb0;
    const float zc = valid ? run : -INFINITY;
    sz[tid] = zc;
    __syncthreads();
    int rank = 0;
    if (valid)
      for (int c2 = 0; c2 < Cke; ++c2) {
        const float z2 = sz[c2];
        rank += (z2 > zc) || (z2 == zc && c2 < c);
      }
    const bool sel = valid && rank < k1;
    const unsigned long long bal = __ballot(sel);
    if (lane == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int pre = 0;
    for (int q = 0; q < w; ++q) pre += wcnt[q];
    const int nsel = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    if (sel) {
      const int pos = pre + __popcll(bal & lt);
      R1[pos] = c;
      selc[pos] = c;
    }
    for (int j = nsel + tid; j < pl.k1w; j += 256) R1[j] = -1;
    __syncthreads();
    // top-k2 blocks of each retrieved cluster: wave w takes slots w, w + 4, ...
    // lane l owns blocks l + 64 t; bit t of `mine` marks a chosen one
    for (int j = w; j < pl.k1w; j += 4) {
      int32_t* out = R2 + (size_t)j * pl.k2w;
      if (j >= nsel) {
        for (int t = lane; t < pl.k2w; t += 64) out[t] = -1;
        continue;
      }
      const int cj = selc[j];
      const float* pzj = b.pz + (irow * pl.Ck + cj) * pl.nb;
      float* my = bsc[w];
      // each lane stages and later scans only its own blocks be = lane + 64 u
      // (an empty (cluster, block) has ln Z = -inf and is never a candidate)
      for (int be = lane; be < bb; be += 64) my[be] = pzj[be];
      unsigned long long mine = 0;
      for (int t = 0; t < pl.k2w; ++t) {
        float best = -INFINITY;
        int bi = INT_MAX;
        for (int be = lane, u = 0; be < bb; be += 64, ++u) {
          const float v = my[be];
          if (!(v > -INFINITY) || ((mine >> u) & 1)) continue;
          if (bi == INT_MAX || v > best) { best = v; bi = be; }   // blocks ascend per lane
        }
        for (int o = 32; o >= 1; o >>= 1) {
          const float ob = __shfl_xor(best, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (oi != INT_MAX && (bi == INT_MAX || ob > best || (ob == best && oi < bi))) { best = ob; bi = oi; }
        }
        if (bi == INT_MAX) break;
        if ((bi & 63) == lane) mine |= 1ull << (bi >> 6);
      }
      int pos = 0;
      for (int t = 0; 64 * t < bb; ++t) {
        const bool mt = (mine >> t) & 1;
        const unsigned long long m = __ballot(mt);
        if (mt) out[pos + __popcll(m & lt)] = 64 * t + lane;
        pos += __popcll(m);
      }
      for (int t = pos + lane; t < pl.k2w; t += 64) out[t] = -1;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Far items of every group.  One workgroup per (q-head, I, chunk of CW key
// clusters) with QN x CW threads: thread (part q, key cluster c) keeps 8
// dims of the running prefix (ln Z, kappa, U) of c over the blocks < b, so a
// wave writes 64 consecutive clusters of one value row of the (d, c) layout
// at once.  A cluster the group retrieved gets the prefix without its
// retrieved blocks: with r = 1 - sum over those blocks of Z_block / Z_prefix,
// kappa = (kappa_prefix - sum (Z_block / Z_prefix) kappa_block) / r (U alike)
// and ln Z = ln Z_prefix + ln r.  Rounding is amplified by 1 / r, so when
// r < 1/256 (the retrieved blocks hold nearly all of the prefix) the other
// blocks are merged directly instead; an empty remainder (by key count)
// gives no item.
// ---------------------------------------------------------------------------
template <int D>
struct FarGeo {
  static constexpr int DQ = 8, QN = D / DQ, CW = 1024 / QN;   // dims per thread, parts, clusters per workgroup
};

// Merge the statistics of block be of row prow (dims off .. off + DQ) into (z, k, u).
template <int D, int DQ>
__device__ __forceinline__ void far_merge(const AttnBufs& b, size_t prow, int nb, int be, int off, float& z,
                                          float* k, float* u) {
  const float z2 = b.pz[prow * nb + be];
  if (!(z2 > -INFINITY)) return;
  const float zm = fmaxf(z, z2);
  const float a = __expf(z - zm), wgt = __expf(z2 - zm);
  const float inv = 1.f / (a + wgt);
  const float* k2 = b.pk + (prow * nb + be) * D + off;
  const float* u2 = b.pu + (prow * nb + be) * D + off;
#pragma unroll
  for (int e = 0; e < DQ; e += 4) {
    const f32x4 kk = *reinterpret_cast<const f32x4*>(k2 + e);
    const f32x4 uu = *reinterpret_cast<const f32x4*>(u2 + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[e + i] = (a * k[e + i] + wgt * kk[i]) * inv;
      u[e + i] = (a * u[e + i] + wgt * uu[i]) * inv;
    }
  }
  z = zm + __logf(a + wgt);
}

template <typename TIn, int D>
__global__ void __launch_bounds__(1024) v4_far_kernel(Plan pl, AttnBufs b, int cw, int nchunk) {
  constexpr int DQ = FarGeo<D>::DQ, QN = FarGeo<D>::QN;
  __shared__ float red[QN][FarGeo<D>::CW];
  __shared__ int32_t slot[MUSE_MAXC];   // (block << 8) | retrieved slot, per key cluster
  __shared__ int32_t r2s[MUSE_MAXC];    // the group's retrieved blocks, [slot][k2w]
  const int tid = threadIdx.x;
  const int q = tid / cw, cl = tid % cw;
  const int Cke = min(pl.Ck, pl.N), Cqe = min(pl.Cq, pl.N);
  const int chunk = blockIdx.x % nchunk;
  const int bh = blockIdx.x / nchunk / pl.Cq, I = blockIdx.x / nchunk % pl.Cq;
  const int c = chunk * cw + cl;
  if (I >= Cqe) return;   // whole workgroup
  const bool cin = c < (Cke + 63) / 64 * 64;   // columns written (whole far tiles)
  const bool cok = c < Cke;
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  const float s2 = pl.scale * PX_LOG2E;
  const size_t irow = (size_t)bh * pl.Cq + I;
  const int32_t* qbr = b.qb + irow * (pl.nb + 1);
  const int32_t* kbc = b.kb + ((size_t)kvh * pl.Ck + (cok ? c : 0)) * (pl.nb + 1);
  const float* nup = b.qs.cent + ((size_t)bh * pl.C + I) * D + q * DQ;   // read where needed
  const size_t prow = irow * pl.Ck + (cok ? c : 0);
  const int k12 = pl.k1w * pl.k2w;
  __shared__ int32_t hasq[V4_MAXNB];   // 1: the group (I, block) has queries
  for (int t = tid; t < MUSE_MAXC; t += blockDim.x) slot[t] = -1;
  for (int t = tid; t < pl.nb; t += blockDim.x) hasq[t] = t >= 1 && qbr[t + 1] > qbr[t];
  __syncthreads();
  float z = -INFINITY, kap[DQ], u[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) { kap[e] = 0.f; u[e] = 0.f; }
  const int Cp = b.Cp32;
  for (int bb = 0; bb < pl.nb; ++bb) {
    if (hasq[bb]) {
      const size_t g = ((size_t)bh * pl.nb + bb) * pl.Cq + I;
      if (pl.topk > 0) {
        const int32_t* R1 = b.r1 + (irow * pl.nb + bb) * pl.k1w;
        const int32_t* R2 = b.r2 + (irow * pl.nb + bb) * k12;
        if (tid < pl.k1w) {
          const int cs = R1[tid];
          if (cs >= 0) slot[cs] = (bb << 8) | tid;
        }
        if (tid < k12) r2s[tid] = R2[tid];
      }
      // (also orders this group's writes of red after the previous group's reads)
      __syncthreads();
      float zf = z, kf[DQ], uf[DQ];
#pragma unroll
      for (int e = 0; e < DQ; ++e) { kf[e] = kap[e]; uf[e] = u[e]; }
      const int sv = cok ? slot[c] : -1;
      if (sv >= 0 && (sv >> 8) == bb) {
        const int32_t* sel = r2s + (sv & 255) * pl.k2w;
        int nrem = kbc[bb] - kbc[0];
        float rho = 0.f;
        for (int t = 0; t < pl.k2w; ++t) {
          const int be = sel[t];
          if (be < 0) break;
          nrem -= kbc[be + 1] - kbc[be];
          const float zb = b.pz[prow * pl.nb + be];
          if (!(zb > -INFINITY)) continue;
          const float wgt = __expf(zb - z);
          rho += wgt;
          const float* k2 = b.pk + (prow * pl.nb + be) * D + q * DQ;
          const float* u2 = b.pu + (prow * pl.nb + be) * D + q * DQ;
#pragma unroll
          for (int e = 0; e < DQ; e += 4) {
            const f32x4 kk = *reinterpret_cast<const f32x4*>(k2 + e);
            const f32x4 uu = *reinterpret_cast<const f32x4*>(u2 + e);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              kf[e + i] = fmaf(-wgt, kk[i], kf[e + i]);
              uf[e + i] = fmaf(-wgt, uu[i], uf[e + i]);
            }
          }
        }
        const float r = 1.f - rho;
        if (nrem == 0) {
          zf = -INFINITY;
        } else if (r >= 1.f / 256.f) {
          const float inv = 1.f / r;
#pragma unroll
          for (int e = 0; e < DQ; ++e) { kf[e] *= inv; uf[e] *= inv; }
          zf = z + __logf(r);
        } else {
          zf = -INFINITY;
#pragma unroll
          for (int e = 0; e < DQ; ++e) { kf[e] = 0.f; uf[e] = 0.f; }
          int p = 0;
          for (int be = 0; be < bb; ++be) {
            if (p < pl.k2w && sel[p] == be) { ++p; continue; }
            far_merge<D, DQ>(b, prow, pl.nb, be, q * DQ, zf, kf, uf);
          }
        }
      }
      const bool ne = cok && zf > -INFINITY;
      TIn kr[DQ];
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        kr[e] = px_round<TIn>(ne ? kf[e] : 0.f);
        dot = fmaf(nup[e], px_float<TIn>(kr[e]), dot);
      }
      dot *= s2;
      if (cin) {
        TIn* fk = reinterpret_cast<TIn*>(b.fk) + (g * Cp + c) * D + q * DQ;
#pragma unroll
        for (int e = 0; e < DQ; ++e) fk[e] = kr[e];
        TIn* fv = reinterpret_cast<TIn*>(b.fv) + (g * D + q * DQ) * Cp + c;
#pragma unroll
        for (int e = 0; e < DQ; ++e) fv[(size_t)e * Cp] = px_round<TIn>(ne ? uf[e] : 0.f);
      }
      red[q][cl] = dot;
      __syncthreads();
      if (q == 0 && cin) {
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < QN; ++i) tot += red[i][cl];
        b.fbias[g * Cp + c] = ne ? zf * PX_LOG2E - tot : -INFINITY;
      }
    }
    if (cok) far_merge<D, DQ>(b, prow, pl.nb, bb, q * DQ, z, kap, u);
  }
}

// ---------------------------------------------------------------------------
template <typename TIn, int D>
static hipError_t v4_go(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  const int Cqe = std::min(pl.Cq, pl.N), Cke = std::min(pl.Ck, pl.N);
  const long long BHq = (long long)pl.B * pl.Hq;
  {
    const long long n = ((long long)b.ks.heads * pl.Ck + (long long)b.qs.heads * pl.Cq) * (pl.nb + 1);
    MUSE_KT_PRE(st);
    v4_bounds_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(pl, b.ks, b.qs, b.kb, b.qb);
    MUSE_KT_POST("v4_bounds", st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    // about 16 waves per SIMD: split each key cluster's blocks into ranges
    const long long base = BHq * ((Cqe + 15) / 16) * Cke;
    const int nbg = (int)std::max<long long>(1, std::min<long long>(pl.nb, 16384 / std::max<long long>(base, 1)));
    const long long waves = base * nbg;
    MUSE_KT_PRE(st);
    v4_part_kernel<TIn, D><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(pl, b, nbg);
    MUSE_KT_POST("v4_part", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  MUSE_KT_PRE(st);
  v4_select_kernel<<<(unsigned)(BHq * pl.Cq), 256, 0, st>>>(pl, b);
  MUSE_KT_POST("v4_select", st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    // clusters rounded up to whole waves, in chunks of at most CW
    const int Cpk = (Cke + 63) / 64 * 64;
    const int cw = std::min(Cpk, FarGeo<D>::CW), nchunk = (Cpk + cw - 1) / cw;
    MUSE_KT_PRE(st);
    v4_far_kernel<TIn, D><<<(unsigned)(BHq * pl.Cq * nchunk), FarGeo<D>::QN * cw, 0, st>>>(pl, b, cw, nchunk);
    MUSE_KT_POST("v4_far", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_v4(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st) {
  if (dtype == 1) return pl.D == 64 ? v4_go<uint16_t, 64>(pl, b, st) : v4_go<uint16_t, 128>(pl, b, st);
  return pl.D == 64 ? v4_go<float, 64>(pl, b, st) : v4_go<float, 128>(pl, b, st);
}

}  // namespace muse
