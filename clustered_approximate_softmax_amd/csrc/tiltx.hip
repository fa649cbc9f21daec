// Exactly tilted key-cluster statistics (gist.science page, Technical
// Summary, Core Mechanisms: Exponential Tilting: key-cluster centroids and
// summaries weighted by the attention of each query-cluster centroid, so
// they are specific to the query cluster; Decomposition: only the residual
// cross term is dropped).  For query cluster I with centroid nu_I and key
// cluster c, with w_j = exp(s nu_I.k_j) over the keys j of c:
//   lnZ_Ic   = log sum_j w_j                 (log tilted mass: retrieval score)
//   kappa_Ic = sum_j w_j k_j / sum_j w_j     (tilted key centroid)
//   U_Ic     = sum_j w_j v_j / sum_j w_j     (tilted value mean)
// The far item of c for a query q of I then has log-weight
// lnZ_Ic + s (q - nu_I).kappa_Ic and value U_Ic; the attention kernel reads
// it as key row kappa_Ic, value U_Ic and base-2 bias
// log2 Z_Ic - s log2(e) nu_I.kappa_Ic (kappa rounded to the input dtype, as
// the attention kernel reads it).
//
// This is attention with the query-cluster centroids as queries, the keys of
// one cluster as keys and [k_j | v_j] as values: per key tile, S = K nu^T on
// MFMA (nu split into bf16 parts so the scores keep fp32 accuracy), an online
// base-2 softmax per (query cluster, key cluster), and O^T += [K|V]^T P^T on
// MFMA with the tile staged feature-major in LDS.  One workgroup takes 32
// query clusters (16 per wave) and CB consecutive key clusters, so that the
// tilted value means of one (I, d) are written as one 16-byte run of the
// (I, d, c) layout the far tiles read.  The CB clusters' keys are one range
// of the sorted copy, tiled as a whole: small clusters share a tile, each
// cluster masking the others' keys out of its softmax.
#include "common.h"
#include "launch.h"

namespace muse {

constexpr int TX_KT = 32;      // keys per tile
constexpr int TX_WAVES = 2;    // waves per workgroup, 16 query clusters each
constexpr int TX_IB = 16 * TX_WAVES;
constexpr float TX_LOG2E = 1.4426950408889634f;
constexpr float TX_LN2 = 0.6931471805599453f;

template <typename TIn, int D>
struct TxGeo {
  static constexpr int CB = 16 / (int)sizeof(TIn);            // key clusters per workgroup
  static constexpr int ROW = TX_KT * (int)sizeof(TIn) + 16;   // LDS bytes per feature row (padded)
  static constexpr int NSK = sizeof(TIn) == 2 ? 1 : 3;        // parts of keys / values / P
  static constexpr int NSN = sizeof(TIn) == 2 ? 2 : 3;        // parts of nu
};

template <typename TIn, int D>
struct alignas(16) TxSmem {
  using G = TxGeo<TIn, D>;
  unsigned char kv[2 * D][G::ROW];   // [K | V]^T of the current tile, feature-major
  TIn ust[TX_IB][D][G::CB];          // U of the block's clusters, (I, d, c)
  float lz[TX_IB][G::CB];
  float fb[TX_IB][G::CB];
};

// 8 consecutive keys of feature row f as NS bf16 parts.
template <typename TIn, int NS>
__device__ __forceinline__ void tx_frag(const unsigned char* row, int k8, u16x8* out) {
  if constexpr (sizeof(TIn) == 2) {
    out[0] = *reinterpret_cast<const u16x8*>(row + 16 * k8);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + 32 * k8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + 32 * k8 + 16);
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t h, m, l;
      split3(v[j], h, m, l);
      out[0][j] = h;
      if (NS > 1) { out[NS > 1 ? 1 : 0][j] = m; out[NS > 2 ? 2 : 0][j] = l; }
    }
  }
}

template <typename TIn>
__device__ __forceinline__ TIn tx_round(float x) {
  if constexpr (sizeof(TIn) == 2) { TIn r; r.v = f2bf(x); return r; }
  else return x;
}
template <typename TIn>
__device__ __forceinline__ float tx_value(TIn x) {
  if constexpr (sizeof(TIn) == 2) return bf2f(x.v);
  else return x;
}

// Element type held in LDS and global arrays: bf16 as a 16-bit pattern.
template <typename TIn>
using TxElem = typename std::conditional<sizeof(TIn) == 2, bf16_t, float>::type;

template <typename TIn, int D>
__global__ void __launch_bounds__(64 * TX_WAVES) tiltx_kernel(Plan pl, AttnBufs b, long long kps) {
  using G = TxGeo<TIn, D>;
  using E = TxElem<TIn>;
  constexpr int CB = G::CB, NSK = G::NSK, NSN = G::NSN;
  constexpr int KS = D / 32, FT = 2 * D / 16;
  extern __shared__ __align__(16) unsigned char tx_raw[];
  TxSmem<E, D>& sm = *reinterpret_cast<TxSmem<E, D>*>(tx_raw);
  const int C = pl.C, Cp = b.Cp32, Gq = pl.Hq / pl.Hkv;
  const int nib = (C + TX_IB - 1) / TX_IB, ncb = Cp / CB;
  const int per = Gq * nib * ncb;                   // workgroups per key problem
  // the workgroups of one key problem share an XCD (blockIdx % 8), so the
  // query heads of its group re-read the keys from one L2
  const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
  const long long kp = (long long)(loc / per) * 8 + xcd;
  if (kp >= kps) return;
  int u = loc % per;
  const int cb = u % ncb;
  u /= ncb;
  const int ib = u % nib, hl = u / nib;
  const int kvh = (int)(kp / pl.P), p = (int)(kp % pl.P);
  const int bq = kvh / pl.Hkv, kh = kvh % pl.Hkv;
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(pl.Cq, gm.qn), Ck = min(pl.Ck, gm.kn);
  const int i0 = ib * TX_IB;
  if (i0 >= Cq) return;
  const size_t ap = (size_t)(bq * pl.Hq + kh * Gq + hl) * pl.P + p;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, col = lane & 15, g = lane >> 4;
  const float s2 = pl.scale * TX_LOG2E;
  const int32_t* koffs = b.ks.offs + kp * (C + 1);
  const size_t slice = (size_t)gm.lev * pl.B * pl.Hkv + kvh;
  const TIn* Kp = reinterpret_cast<const TIn*>(b.kst.Kp) + (slice * pl.N + gm.k0) * D;
  const TIn* Vp = reinterpret_cast<const TIn*>(b.kst.Vp) + (slice * pl.N + gm.k0) * D;
  const float* nu_all = b.qs.cent + ap * (size_t)C * D;
  E* kap = reinterpret_cast<E*>(b.kap) + (ap * C) * (size_t)Cp * D;
  E* T = reinterpret_cast<E*>(b.T) + (ap * C) * (size_t)D * Cp;
  float* lzg = b.lz + (ap * C) * (size_t)Cp;
  float* fbg = b.fb + (ap * C) * (size_t)Cp;

  // this lane's query cluster (B operand column) and its centroid fragments
  const int Iw = i0 + 16 * w + col;
  const bool Iok = Iw < Cq;
  const float* nu = nu_all + (size_t)(Iok ? Iw : 0) * D;
  u16x8 nf[KS][NSN];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = Iok ? nu[32 * k + 8 * g + j] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t h, m, l;
      split3(v[j], h, m, l);
      nf[k][0][j] = h;
      nf[k][1][j] = m;
      if (NSN > 2) nf[k][NSN > 2 ? 2 : 0][j] = l;
    }
  }
  // the lane's features of the output tiles: f = 16 ft + 4 g + i
  float nuf[D / 16][4];
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) nuf[ft][i] = Iok ? nu[16 * ft + 4 * g + i] : 0.f;

  // The block's clusters are consecutive, so their keys are one range [L, H)
  // of the sorted copy.  It is walked in full tiles (small clusters share a
  // tile instead of each padding its own); every cluster with keys in a tile
  // takes the tile's scores under its own mask, in cluster order, with one
  // running softmax state: the open cluster's.
  const int cfirst = cb * CB;
  const int L = cfirst < Ck ? koffs[cfirst] : 0;
  const int H = cfirst < Ck ? koffs[min(cfirst + CB, Ck)] : 0;
  int cl = 0, c = cfirst;
  int lo = c < Ck ? koffs[c] : 0, hi = c < Ck ? koffs[c + 1] : 0;
  f32x4 acc[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lp = 0.f;
  // write the open cluster's statistics, then open the next one
  auto finish = [&]() __attribute__((always_inline)) {
    // normalise; every lane of a column ends with the same m and total
    float lt = lp + __shfl_xor(lp, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const bool ok = hi > lo;
    const float inv = ok ? 1.f / lt : 0.f;
    // tilted key centroid (rounded as the attention kernel reads it) and nu.kappa
    float dot = 0.f;
    E* krow = kap + ((size_t)(Iok ? Iw : 0) * Cp + c) * D;
#pragma unroll
    for (int ft = 0; ft < D / 16; ++ft) {
      E kr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = tx_round<E>(acc[ft][i] * inv);
        dot = fmaf(nuf[ft][i], tx_value<E>(kr[i]), dot);
      }
      if (Iok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) krow[16 * ft + 4 * g + i] = kr[i];
      }
    }
    dot += __shfl_xor(dot, 16, 64);
    dot += __shfl_xor(dot, 32, 64);
    const int il = 16 * w + col;
#pragma unroll
    for (int ft = D / 16; ft < FT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.ust[il][16 * (ft - D / 16) + 4 * g + i][cl] = tx_round<E>(acc[ft][i] * inv);
    if (g == 0) {
      const float l2z = m + __log2f(lt);
      sm.lz[il][cl] = ok ? l2z * TX_LN2 : -INFINITY;
      sm.fb[il][cl] = ok ? l2z - s2 * dot : -INFINITY;
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    lp = 0.f;
    ++cl;
    c = cfirst + cl;
    lo = c < Ck ? koffs[c] : 0;
    hi = c < Ck ? koffs[c + 1] : 0;
  };
  for (int t0 = L; t0 < H; t0 += TX_KT) {
    // The tile's global reads go out together, before the barriers: the key
    // rows of S = K nu^T (row tile rt, A row r: key 8 (r / 4) + 4 rt + r % 4,
    // so lane (col, g) ends with keys 8 g + 4 rt + i of query cluster col)
    // and, for bf16, the feature-major staging runs of [K | V]^T (4
    // consecutive keys x 8 features per item, keys past the block zero).
    constexpr int NIT = (TX_KT / 4) * (2 * D / 8) / (64 * TX_WAVES);
    static_assert(NIT * 64 * TX_WAVES == (TX_KT / 4) * (2 * D / 8), "staging items cover the workgroup");
    u16x8 ka[2][KS][NSK];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int key = min(t0 + 8 * (col >> 2) + 4 * rt + (col & 3), H - 1);
#pragma unroll
      for (int k = 0; k < KS; ++k) load8_split<TIn, NSK>(Kp + (size_t)key * D + 32 * k + 8 * g, ka[rt][k]);
    }
    u16x8 rr[sizeof(TIn) == 2 ? NIT : 1][4];
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int q = tid + it * 64 * TX_WAVES;
        const int kb = q % (TX_KT / 4), f0 = (q / (TX_KT / 4)) * 8;
        const TIn* src = f0 < D ? Kp + f0 : Vp + (f0 - D);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int key = t0 + 4 * kb + u;
          rr[it][u] = key < H ? *reinterpret_cast<const u16x8*>(src + (size_t)key * D)
                               : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
    }
    __syncthreads();   // the previous tile's stage is consumed
    // each feature's 4 keys written as one run
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int q = tid + it * 64 * TX_WAVES;
      const int kb = q % (TX_KT / 4), f0 = (q / (TX_KT / 4)) * 8;
      if constexpr (sizeof(TIn) == 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<u16x4*>(sm.kv[f0 + j] + 8 * kb) = u16x4{rr[it][0][j], rr[it][1][j], rr[it][2][j], rr[it][3][j]};
      } else {
        const TIn* src = f0 < D ? Kp + f0 : Vp + (f0 - D);
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int key = t0 + 4 * kb + u;
          if (key < H) {
            load8_f32<TIn>(src + (size_t)key * D, v[u]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[u][j] = 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<f32x4*>(sm.kv[f0 + j] + 16 * kb) = f32x4{v[0][j], v[1][j], v[2][j], v[3][j]};
      }
    }
    __syncthreads();
    float xs[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) sc = mfma_split<NSK, NSN>(ka[rt][k], nf[k], sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[rt][i] = t0 + 8 * g + 4 * rt + i < H ? s2 * sc[i] : -INFINITY;
    }
    // the clusters with keys in this tile (empty ones finish as they come)
    while (cl < CB) {
      if (hi <= lo) {
        finish();
        continue;
      }
      if (lo >= t0 + TX_KT) break;   // starts in a later tile
      float x[2][4];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = t0 + 8 * g + 4 * rt + i;
          x[rt][i] = key >= lo && key < hi ? xs[rt][i] : -INFINITY;
        }
      float mt = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, x[rt][i]);
      mt = max4_lanes(mt);
      if (mt > m) {
        const float alpha = __builtin_amdgcn_exp2f(m - mt);   // 0 on the first tile
        lp *= alpha;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) acc[ft] *= alpha;
        m = mt;
      }
      float pr[8];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[4 * rt + i] = __builtin_amdgcn_exp2f(x[rt][i] - m);
          lp += pr[4 * rt + i];
        }
      // P^T slots 8 g + j hold keys 8 g + j (natural order)
      u16x8 pb[NSK];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t h, mm, l;
        split3(pr[j], h, mm, l);
        pb[0][j] = NSK == 1 ? f2bf(pr[j]) : h;
        if (NSK > 1) { pb[NSK > 1 ? 1 : 0][j] = mm; pb[NSK > 2 ? 2 : 0][j] = l; }
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        u16x8 a[NSK];
        tx_frag<TIn, NSK>(sm.kv[16 * ft + col], g, a);
        acc[ft] = mfma_split<NSK, NSK>(a, pb, acc[ft]);
      }
      if (hi > t0 + TX_KT) break;   // continues in the next tile
      finish();
    }
  }
  // clusters left (empty, or all of them when the block holds no key)
  while (cl < CB) finish();
  __syncthreads();
  // U rows of the block's clusters: one 16-byte run per (I, d)
  const int c0 = cb * CB;
  for (int q = tid; q < TX_IB * D; q += 64 * TX_WAVES) {
    const int il = q / D, d = q % D;
    const int I = i0 + il;
    if (I >= Cq) continue;
    *reinterpret_cast<f32x4*>(T + ((size_t)I * D + d) * Cp + c0) = *reinterpret_cast<const f32x4*>(&sm.ust[il][d][0]);
  }
  for (int q = tid; q < TX_IB * CB; q += 64 * TX_WAVES) {
    const int il = q / CB, cl = q % CB;
    const int I = i0 + il;
    if (I >= Cq) continue;
    lzg[(size_t)I * Cp + c0 + cl] = sm.lz[il][cl];
    fbg[(size_t)I * Cp + c0 + cl] = sm.fb[il][cl];
  }
}

// Retrieval sets from the exact log tilted masses: one wave per (attention
// problem, query cluster), the top-k1 non-empty clusters by lnZ, ties to
// the lower index, stored in ascending order (-1 padded).
__global__ void __launch_bounds__(256) lz_topk_kernel(Plan pl, AttnBufs b) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int C = pl.C, Cp = b.Cp32;
  if (wave >= (long long)pl.B * pl.Hq * pl.P * C) return;
  const size_t ap = wave / C;
  const int I = (int)(wave % C);
  const int p = (int)(ap % pl.P);
  const Geom gm = prob_geom(pl, p);
  const int Cq = min(pl.Cq, gm.qn), Ck = min(pl.Ck, gm.kn);
  int32_t* R = b.R + (ap * C + I) * pl.k1w;
  const int32_t* qoffs = b.qs.offs + ap * (C + 1);
  const int mI = I < Cq ? qoffs[I + 1] - qoffs[I] : 0;
  if (mI == 0 || pl.topk <= 0) {
    for (int q = lane; q < pl.k1w; q += 64) R[q] = -1;
    return;
  }
  const float* lz = b.lz + (ap * C + I) * (size_t)Cp;
  float sig[4];
  bool sel[4];
  int nvalid = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int c = lane + 64 * r;
    sig[r] = c < Ck ? lz[c] : -INFINITY;
    sel[r] = false;
    nvalid += sig[r] > -INFINITY ? 1 : 0;
  }
  for (int mm = 32; mm >= 1; mm >>= 1) nvalid += __shfl_xor(nvalid, mm, 64);
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
    for (int mm = 32; mm >= 1; mm >>= 1) {
      const float ov = __shfl_xor(bv, mm, 64);
      const int oc = __shfl_xor(bc, mm, 64);
      if (ov > bv || (ov == bv && oc < bc)) { bv = ov; bc = oc; }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (lane + 64 * r == bc) sel[r] = true;
  }
  int base = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned long long bal = __ballot(sel[r]);
    const unsigned long long lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if (sel[r]) R[base + __popcll(bal & lt)] = lane + 64 * r;
    base += __popcll(bal);
  }
  for (int q = base + lane; q < pl.k1w; q += 64) R[q] = -1;
}

template <typename TIn, int D>
static hipError_t tiltx_go(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  using G = TxGeo<TIn, D>;
  const long long kps = (long long)pl.B * pl.Hkv * pl.P;
  const int nib = (pl.C + TX_IB - 1) / TX_IB, ncb = b.Cp32 / G::CB;
  const long long per = (long long)(pl.Hq / pl.Hkv) * nib * ncb;
  const long long grid = ((kps + 7) / 8) * 8 * per;
  if (grid == 0) return hipSuccess;
  using E = TxElem<TIn>;
  const size_t smem = sizeof(TxSmem<E, D>);
  set_smem_once((const void*)tiltx_kernel<TIn, D>, smem);
  MUSE_KT_PRE(st);
  tiltx_kernel<TIn, D><<<(unsigned)grid, 64 * TX_WAVES, smem, st>>>(pl, b, kps);
  MUSE_KT_POST("tilt_exact", st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long waves = (long long)pl.B * pl.Hq * pl.P * pl.C;
  MUSE_KT_PRE(st);
  lz_topk_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(pl, b);
  MUSE_KT_POST("score_topk", st);
  return hipGetLastError();
}

hipError_t launch_tilt_exact(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st) {
  if ((long long)pl.B * pl.Hkv * pl.P == 0) return hipSuccess;
  if (dtype == 1) return pl.D == 64 ? tiltx_go<uint16_t, 64>(pl, b, st) : tiltx_go<uint16_t, 128>(pl, b, st);
  return pl.D == 64 ? tiltx_go<float, 64>(pl, b, st) : tiltx_go<float, 128>(pl, b, st);
}

}  // namespace muse
