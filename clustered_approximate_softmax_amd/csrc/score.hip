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

namespace muse {

// One wave per (attention problem, query cluster).
__global__ void __launch_bounds__(256) score_topk_kernel(Plan pl, AttnBufs b) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
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

hipError_t launch_score_topk(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  const long long waves = (long long)pl.B * pl.Hq * pl.P * pl.C;
  if (waves == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  score_topk_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(pl, b);
  MUSE_KT_POST("score_topk", st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// T[ap][I][d][c] = S[kp][c][d] + s sum_e M[kp][d][c][e] nu[ap][I][e]
// One workgroup per (attention problem, value dim d).  For fixed d this is
// a (clusters c) x (query clusters I) product over the key dim e.
// ---------------------------------------------------------------------------
template <typename TIn, int D, int NS>
__global__ void __launch_bounds__(256) tilt_kernel(Plan pl, AttnBufs b) {
  const int C = pl.C, Cp = b.Cp32;
  const int d = blockIdx.x % D;
  const int ap = blockIdx.x / D;
  const int bh = ap / pl.P, p = ap % pl.P;
  const int bq = bh / pl.Hq, hq = bh % pl.Hq;
  const int kv = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  const size_t kp = (size_t)kv * pl.P + p;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(C, gm.qn), Ck = min(C, gm.kn);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const float s = pl.dipole ? pl.scale : 0.f;
  const float* Md = b.kst.M + (kp * D + d) * (size_t)C * D;      // [c][e]
  const float* S = b.kst.S + kp * C * D;                          // [c][d]
  const float* nu = b.qs.cent + (size_t)ap * C * D;               // [I][e]
  TIn* T = reinterpret_cast<TIn*>(b.T) + (size_t)ap * C * D * Cp;  // [I][d][c], T / n_c
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const int nct = (Ck + 15) / 16, nit = (Cq + 15) / 16;
  constexpr int KS = D / 32;
  for (int ct = w; ct < nct; ct += 4) {
    u16x8 a[KS][NS];
    const int cr = 16 * ct + col;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float v[8];
      if (cr < Ck) {
        const float* src = Md + (size_t)cr * D + 32 * k + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t h, m, l;
        split3(v[j], h, m, l);
        a[k][0][j] = h;
        if (NS > 1) { a[k][1][j] = m; a[k][2][j] = l; }
      }
    }
    for (int it = 0; it < nit; ++it) {
      const int ir = 16 * it + col;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u16x8 bb[NS];
        float v[8];
        if (ir < Cq) {
          const float* src = nu + (size_t)ir * D + 32 * k + 8 * g;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = src[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint16_t h, m, l;
          split3(v[j], h, m, l);
          bb[0][j] = h;
          if (NS > 1) { bb[1][j] = m; bb[2][j] = l; }
        }
        acc = mfma_split<NS, NS>(a[k], bb, acc);
      }
      if (ir < Cq) {
        TIn* dst = T + ((size_t)ir * D + d) * Cp + 16 * ct + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * ct + 4 * g + i;
          const int nc = c < Ck ? koffs[c + 1] - koffs[c] : 0;
          store1<TIn>(dst + i, nc > 0 ? (S[(size_t)c * D + d] + s * acc[i]) / (float)nc : 0.f);
        }
      }
    }
  }
  // zero the padding columns [16*nct, Cp) so consumers may read whole 32-wide chunks
  for (int idx = threadIdx.x; idx < Cq * (Cp - 16 * nct); idx += 256) {
    const int I = idx / (Cp - 16 * nct), c = 16 * nct + idx % (Cp - 16 * nct);
    store1<TIn>(T + ((size_t)I * D + d) * Cp + c, 0.f);
  }
}

hipError_t launch_tilt(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st) {
  const long long grid = (long long)pl.B * pl.Hq * pl.P * pl.D;
  if (grid == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  if (dtype == 1) {
    if (pl.D == 64) tilt_kernel<uint16_t, 64, 1><<<(unsigned)grid, 256, 0, st>>>(pl, b);
    else tilt_kernel<uint16_t, 128, 1><<<(unsigned)grid, 256, 0, st>>>(pl, b);
  } else {
    if (pl.D == 64) tilt_kernel<float, 64, 3><<<(unsigned)grid, 256, 0, st>>>(pl, b);
    else tilt_kernel<float, 128, 3><<<(unsigned)grid, 256, 0, st>>>(pl, b);
  }
  MUSE_KT_POST("tilt", st);
  return hipGetLastError();
}

}  // namespace muse
