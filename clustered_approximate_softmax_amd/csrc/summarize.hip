// Key-cluster statistics (newx.sg page, Abstract: centroid / monopole
// approximation with a dipole correction): per key cluster c the count n_c,
// centroid mu_c, value sum S_c = sum_j v_j and dipole moment
// M_c = sum_j v_j (k_j - mu_c)^T = sum_j v_j k_j^T - S_c mu_c^T.
//
// One workgroup per (key problem, cluster).  The cluster's rows are read
// through the permutation (cluster-contiguous order) in tiles of KT keys,
// staged transposed in LDS, and sum_j v_j k_j^T is an MFMA contraction over
// the tile's keys (exact products of bf16 inputs, fp32 accumulation, fixed
// order: no atomics).  The rows of tile t+1 are in flight while tile t is
// contracted, and the permutation entries of tile t+2, so that a large
// cluster's tiles do not each wait for two dependent loads.
#include "common.h"
#include "launch.h"

namespace muse {

constexpr int SU_NT = 256;

template <typename TIn, int D>
struct alignas(16) SuSmem {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  static constexpr int KT = sizeof(TIn) == 2 && D == 64 ? 64 : 32;   // keys per tile (registers at D = 128)
  static constexpr int KP = KT + 8;
  uint16_t kt[NS][D][KP];
  uint16_t vt[NS][D][KP];
  float red[SU_NT / (D / 8)][2][D];   // [key slot][k sum | v sum][dim]
};

// 8 consecutive input elements held as loaded (bf16: one 16-byte vector)
template <typename TIn>
struct Raw8 {
  static constexpr int W = sizeof(TIn) == 2 ? 1 : 2;
  typedef typename std::conditional<sizeof(TIn) == 2, u16x8, f32x4>::type V;
  V v[W];
  __device__ __forceinline__ void load(const TIn* p) {
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = *reinterpret_cast<const V*>(p + i * (8 / W));
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = V{};
  }
  __device__ __forceinline__ void store(TIn* p) const {
#pragma unroll
    for (int i = 0; i < W; ++i) *reinterpret_cast<V*>(p + i * (8 / W)) = v[i];
  }
  __device__ __forceinline__ float at(int j) const {
    if constexpr (sizeof(TIn) == 2) return bf2f(v[0][j]);
    else return v[j / 4][j % 4];
  }
};

template <typename TIn, int D>
__global__ void __launch_bounds__(SU_NT, 2) summarize_kernel(Plan pl, CSet ks, const void* Vv, KStats out) {
  using SM = SuSmem<TIn, D>;
  constexpr int NS = SM::NS, KT = SM::KT;
  constexpr int DT = D / 16;
  constexpr int U = DT * DT / 4;
  constexpr int TPK = D / 8;          // threads per key row
  constexpr int KPP = SU_NT / TPK;    // keys per load pass
  constexpr int NP = KT / KPP;        // passes per tile
  static_assert(KT % KPP == 0 && KT % 32 == 0, "tile shape");
  __shared__ SM sm;
  const int C = pl.C;
  // largest problems (highest p) first: problem rank, then head, then cluster
  const int c = blockIdx.x % C;
  const int head = (blockIdx.x / C) % ks.heads;
  const int p = pl.P - 1 - (int)(blockIdx.x / ((unsigned)C * ks.heads));
  const int hp = head * pl.P + p;     // head * P + p
  int lev, r0, n;
  cset_rows(pl, ks, p, lev, r0, n);
  const int Ceff = min(C, n);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  float* mu = out.mu + ((size_t)hp * C + c) * D;
  float* S = out.S + ((size_t)hp * C + c) * D;
  float* M = out.M + (size_t)hp * D * C * D;   // [d][c][e]
  const int32_t* offs = ks.offs + (size_t)hp * (C + 1);
  const int beg = c < Ceff ? offs[c] : 0;
  const int cnt = c < Ceff ? offs[c + 1] - beg : 0;
  TIn* mu_in = out.mu_in ? reinterpret_cast<TIn*>(out.mu_in) + ((size_t)hp * C + c) * D : nullptr;
  if (cnt == 0) {
    for (int e = tid; e < D; e += SU_NT) {
      mu[e] = 0.f;
      S[e] = 0.f;
      if (mu_in) store1<TIn>(mu_in + e, 0.f);
    }
    for (int idx = tid; idx < D * D; idx += SU_NT) {
      const int d = idx / D, e = idx % D;
      M[((size_t)d * C + c) * D + e] = 0.f;
    }
    return;
  }
  const int32_t* perm = ks.perm + ((size_t)lev * ks.heads + head) * pl.N + r0 + beg;
  const TIn* K = reinterpret_cast<const TIn*>(ks.X) + (size_t)head * pl.N * D;
  const TIn* V = reinterpret_cast<const TIn*>(Vv) + (size_t)head * pl.N * D;
  // cluster-contiguous copies: sorted position q of the problem -> row r0 + q
  const size_t cbase = (((size_t)lev * ks.heads + head) * pl.N + r0 + beg) * D;
  TIn* Kp = out.Kp ? reinterpret_cast<TIn*>(out.Kp) + cbase : nullptr;
  TIn* Vp = out.Vp ? reinterpret_cast<TIn*>(out.Vp) + cbase : nullptr;

  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float sk[8], sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) { sk[j] = 0.f; sv[j] = 0.f; }
  const int e0 = (tid % TPK) * 8, ks0 = tid / TPK;   // dims e0..e0+7 of keys ks0 + KPP * pass

  int rn[NP];            // rows of the next tile
  Raw8<TIn> kd[NP], vd[NP];
  auto rows_of = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int key = t0 + q * KPP + ks0;
      rn[q] = key < cnt ? perm[key] : -1;
    }
  };
  auto load_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      if (rn[q] >= 0) {
        kd[q].load(K + (size_t)rn[q] * D + e0);
        vd[q].load(V + (size_t)rn[q] * D + e0);
      } else {
        kd[q].zero();
        vd[q].zero();
      }
    }
  };
  rows_of(0);
  load_tile();
  if (KT < cnt) rows_of(KT);
  for (int t0 = 0; t0 < cnt; t0 += KT) {
    // tile t0 from registers: sums, cluster-contiguous copies, transposed LDS stage
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int key = q * KPP + ks0;
      if (Kp && t0 + key < cnt) {
        kd[q].store(Kp + (size_t)(t0 + key) * D + e0);
        vd[q].store(Vp + (size_t)(t0 + key) * D + e0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kv = kd[q].at(j), vv = vd[q].at(j);
        sk[j] += kv;
        sv[j] += vv;
        split_store<NS>(kv, &sm.kt[0][e0 + j][key], D * SM::KP);
        split_store<NS>(vv, &sm.vt[0][e0 + j][key], D * SM::KP);
      }
    }
    __syncthreads();
    if (t0 + KT < cnt) {
      load_tile();
      if (t0 + 2 * KT < cnt) rows_of(t0 + 2 * KT);
    }
    if (pl.dipole == 1) {
#pragma unroll
      for (int kk = 0; kk < KT / 32; ++kk)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int tau = w + 4 * u, dt = tau / DT, et = tau % DT;
          u16x8 a[NS], b[NS];
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            a[s] = *reinterpret_cast<const u16x8*>(&sm.vt[s][16 * dt + col][32 * kk + 8 * g]);
            b[s] = *reinterpret_cast<const u16x8*>(&sm.kt[s][16 * et + col][32 * kk + 8 * g]);
          }
          acc[u] = mfma_split<NS, NS>(a, b, acc[u]);
        }
    }
    __syncthreads();
  }
  // column sums over the key slots held by threads sharing e0 (fixed order)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sm.red[ks0][0][e0 + j] = sk[j];
    sm.red[ks0][1][e0 + j] = sv[j];
  }
  // reuse kt as fp32 scratch for the sums: [2][D]
  __syncthreads();
  float* fs = reinterpret_cast<float*>(&sm.kt[0][0][0]);
  if (tid < 2 * D) {
    const int which = tid / D, e = tid % D;
    float s = 0.f;
    for (int q = 0; q < KPP; ++q) s += sm.red[q][which][e];
    fs[which * D + e] = s;
  }
  __syncthreads();
  const float inv = 1.f / (float)cnt;
  for (int e = tid; e < D; e += SU_NT) {
    mu[e] = fs[e] * inv;
    S[e] = fs[D + e];
    if (mu_in) store1<TIn>(mu_in + e, fs[e] * inv);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tau = w + 4 * u, dt = tau / DT, et = tau % DT;
    const int e = 16 * et + col;
    const float mue = fs[e] * inv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * dt + 4 * g + i;
      const float v = pl.dipole == 1 ? acc[u][i] - fs[D + d] * mue : 0.f;
      M[((size_t)d * C + c) * D + e] = v;
    }
  }
}

hipError_t launch_summarize(const Plan& pl, int dtype, const CSet& ks, const void* V, KStats o,
                            hipStream_t st) {
  const int grid = ks.heads * pl.P * pl.C;
  if (grid == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  if (dtype == 1) {
    if (pl.D == 64) summarize_kernel<uint16_t, 64><<<grid, SU_NT, 0, st>>>(pl, ks, V, o);
    else summarize_kernel<uint16_t, 128><<<grid, SU_NT, 0, st>>>(pl, ks, V, o);
  } else {
    if (pl.D == 64) summarize_kernel<float, 64><<<grid, SU_NT, 0, st>>>(pl, ks, V, o);
    else summarize_kernel<float, 128><<<grid, SU_NT, 0, st>>>(pl, ks, V, o);
  }
  MUSE_KT_POST("summarize", st);
  return hipGetLastError();
}

}  // namespace muse
