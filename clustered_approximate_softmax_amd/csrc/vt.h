// Dim-major copies of the values, read by the attention's value tiles: slice
// s < nsorted is the cluster-contiguous copy of level/head s, the next B*Hkv
// slices are the input V.  Vt[s][d][j] = V_s[j][d] for the rows j that hold
// values, zero for the others and for N <= j < Nv.  Each workgroup transposes
// VT_ROWS rows of one slice through LDS.
#pragma once
#include <type_traits>

#include "common.h"

namespace muse {

constexpr int VT_ROWS = 64;

struct VtGeo {
  int nsorted, sfirst, nslice, nb;   // sorted slices, first slice built, slices built, blocks per slice
};

// without retrieval no tile reads the sorted copies: only the input-order
// slices (causal local blocks) are needed
__host__ __device__ inline VtGeo vt_geo(const Plan& pl, int Nv) {
  VtGeo g;
  g.nsorted = pl.nlev * pl.B * pl.Hkv;
  g.sfirst = pl.topk > 0 ? 0 : g.nsorted;
  g.nslice = g.nsorted + (pl.causal ? pl.B * pl.Hkv : 0) - g.sfirst;
  g.nb = (Nv + VT_ROWS - 1) / VT_ROWS;
  return g;
}

// Workgroup blk_id of the transpose grid (nslice * nb workgroups); tile is
// VT_ROWS x (D + 2) elements of LDS.
template <typename TIn, int D>
__device__ __forceinline__ void vt_block(const Plan& pl, const void* Vp, const void* V, void* Vt, int Nv,
                                         int nsorted, int sfirst, int blk_id, TIn (*tile)[D + 2]) {
  const int N = pl.N;
  constexpr int E = 16 / (int)sizeof(TIn), CH = D / E;
  using V16 = typename std::conditional<sizeof(TIn) == 2, u16x8, f32x4>::type;
  const int nb = (Nv + VT_ROWS - 1) / VT_ROWS;
  const int s = sfirst + blk_id / nb, blk = blk_id % nb;
  const TIn* src = s < nsorted ? reinterpret_cast<const TIn*>(Vp) + (size_t)s * N * D
                               : reinterpret_cast<const TIn*>(V) + (size_t)(s - nsorted) * N * D;
  TIn* dst = reinterpret_cast<TIn*>(Vt) + (size_t)s * D * Nv;
  const int j0 = blk * VT_ROWS;
  // causal levels: only the key segments [2tm, 2tm + m), t < nseg, of a
  // level's sorted copy are written; every other column becomes zero
  const int lev = s < nsorted && pl.causal ? s / (pl.B * pl.Hkv) : -1;
  const int m = lev >= 0 ? pl.lev_m[lev] : 0, nseg = lev >= 0 ? pl.lev_nseg[lev] : 0;
  for (int idx = threadIdx.x; idx < VT_ROWS * CH; idx += 256) {
    const int r = idx / CH, e0 = (idx % CH) * E;
    const int j = j0 + r;
    V16 v{};
    if (j < N && (m == 0 || ((j / m) % 2 == 0 && j / (2 * m) < nseg)))
      v = *reinterpret_cast<const V16*>(src + (size_t)j * D + e0);
#pragma unroll
    for (int e = 0; e < E; ++e) tile[r][e0 + e] = v[e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < D * (VT_ROWS / E); idx += 256) {
    const int d = idx / (VT_ROWS / E), jj = (idx % (VT_ROWS / E)) * E;
    if (j0 + jj >= Nv) continue;
    V16 v;
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = tile[jj + e][d];
    *reinterpret_cast<V16*>(dst + (size_t)d * Nv + j0 + jj) = v;
  }
}

}  // namespace muse
