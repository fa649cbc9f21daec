// Key-cluster statistics (newx.sg page, Abstract: centroid / monopole
// approximation with a dipole correction): per key cluster c the count n_c,
// centroid mu_c, value sum S_c = sum_j v_j and dipole moment
// M_c = sum_j v_j (k_j - mu_c)^T = sum_j v_j k_j^T - S_c mu_c^T.
//
// One workgroup per (key problem, cluster).  The cluster's rows are read
// through the permutation (cluster-contiguous order) in tiles of 32 keys,
// staged transposed in LDS, and sum_j v_j k_j^T is a 32-key MFMA
// contraction per tile (exact products of bf16 inputs, fp32 accumulation,
// fixed order: no atomics).
#include "common.h"
#include "launch.h"

namespace muse {

constexpr int SU_NT = 256;
constexpr int SU_KT = 32;
constexpr int SU_KP = SU_KT + 8;

template <typename TIn, int D>
struct alignas(16) SuSmem {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  uint16_t kt[NS][D][SU_KP];
  uint16_t vt[NS][D][SU_KP];
  int32_t rows[SU_KT];
  float red[SU_NT / (D / 8)][2][D];   // [key slot][k sum | v sum][dim]
};

template <typename TIn, int D>
__global__ void __launch_bounds__(SU_NT) summarize_kernel(Plan pl, CSet ks, const void* Vv, KStats out) {
  constexpr int NS = SuSmem<TIn, D>::NS;
  constexpr int DT = D / 16;
  constexpr int U = DT * DT / 4;
  constexpr int TPK = D / 8;          // threads per key row
  constexpr int KPP = SU_NT / TPK;    // keys per load pass
  __shared__ SuSmem<TIn, D> sm;
  const int C = pl.C;
  const int c = blockIdx.x % C;
  const int hp = blockIdx.x / C;      // head * P + p
  const int head = hp / pl.P, p = hp % pl.P;
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
  const int32_t* perm = ks.perm + ((size_t)lev * ks.heads + head) * pl.N + r0;
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
  const int e0 = (tid % TPK) * 8;

  for (int t0 = 0; t0 < cnt; t0 += SU_KT) {
    if (tid < SU_KT) sm.rows[tid] = (t0 + tid < cnt) ? perm[beg + t0 + tid] : -1;
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < SU_KT / KPP; ++pass) {
      const int key = pass * KPP + tid / TPK;
      const int row = sm.rows[key];
      float kv[8], vv[8];
      if (row >= 0) {
        load8_f32<TIn>(K + (size_t)row * D + e0, kv);
        load8_f32<TIn>(V + (size_t)row * D + e0, vv);
        if (Kp) {
          TIn* kd = Kp + (size_t)(t0 + key) * D + e0;
          TIn* vd = Vp + (size_t)(t0 + key) * D + e0;
          if constexpr (sizeof(TIn) == 2) {
            *reinterpret_cast<u16x8*>(kd) = *reinterpret_cast<const u16x8*>(K + (size_t)row * D + e0);
            *reinterpret_cast<u16x8*>(vd) = *reinterpret_cast<const u16x8*>(V + (size_t)row * D + e0);
          } else {
            *reinterpret_cast<f32x4*>(kd) = f32x4{kv[0], kv[1], kv[2], kv[3]};
            *reinterpret_cast<f32x4*>(kd + 4) = f32x4{kv[4], kv[5], kv[6], kv[7]};
            *reinterpret_cast<f32x4*>(vd) = f32x4{vv[0], vv[1], vv[2], vv[3]};
            *reinterpret_cast<f32x4*>(vd + 4) = f32x4{vv[4], vv[5], vv[6], vv[7]};
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { kv[j] = 0.f; vv[j] = 0.f; }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sk[j] += kv[j];
        sv[j] += vv[j];
        split_store<NS>(kv[j], &sm.kt[0][e0 + j][key], D * SU_KP);
        split_store<NS>(vv[j], &sm.vt[0][e0 + j][key], D * SU_KP);
      }
    }
    __syncthreads();
    if (pl.dipole) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tau = w + 4 * u, dt = tau / DT, et = tau % DT;
        u16x8 a[NS], b[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          a[s] = *reinterpret_cast<const u16x8*>(&sm.vt[s][16 * dt + col][8 * g]);
          b[s] = *reinterpret_cast<const u16x8*>(&sm.kt[s][16 * et + col][8 * g]);
        }
        acc[u] = mfma_split<NS, NS>(a, b, acc[u]);
      }
    }
    __syncthreads();
  }
  // column sums over the key slots held by threads sharing e0 (fixed order)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sm.red[tid / TPK][0][e0 + j] = sk[j];
    sm.red[tid / TPK][1][e0 + j] = sv[j];
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
      const float v = pl.dipole ? acc[u][i] - fs[D + d] * mue : 0.f;
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
