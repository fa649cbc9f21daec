// Stage two of the two-stage attention and the exact parts of the causal
// hierarchy (gist.science page, Technical Summary, Core Mechanisms:
// Decomposition, Hierarchical Two-Stage Attention, Retrieval-Augmented
// Approximation; newx.sg page, Abstract: exact local blocks).
//
// For a query i of query cluster I the softmax runs over two kinds of
// items: every key j of a retrieved cluster (logit s q_i.k_j, weight 1,
// value v_j) and every other non-empty key cluster c (logit s q_i.mu_c,
// weight n_c, value T_Ic / n_c).  Both kinds go through the same tile loop:
// a tile is 64 items staged in LDS as rows (A operand of S^T = K Q^T) and as
// a transposed value block (A operand of O^T = V^T P^T), plus a log-weight
// per item; one online softmax (base 2) covers all tiles.  The local causal
// block uses the same loop over contiguous keys with the causal mask.
//
// Pipeline: the next tile is loaded into registers while the current one is
// consumed, then written to the other LDS buffer (one barrier per tile).
// Exact tiles read the cluster-contiguous key/value copies; the row of
// each item is computed two tiles ahead into a small LDS ring.
// Each wave holds QG groups of 16 queries so that every K/V fragment read
// from LDS feeds QG matrix instructions.
#include "common.h"
#include "launch.h"

namespace muse {

enum { MODE_ACAUSAL = 0, MODE_LEVEL = 1, MODE_LOCAL = 2 };
constexpr int AT_KT = 64;   // items per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename TIn, int D, int WAVES, int QG>
struct alignas(16) AtSmem {
  static constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  static constexpr int NB = NS == 1 ? 2 : 1;   // LDS tile buffers
  uint16_t ks[NB][NS][AT_KT][D + 8];
  uint16_t vt[NB][NS][D][AT_KT + 8];
  float bias[NB][AT_KT];
  int32_t krow[NB][AT_KT];
  int32_t ring[4][AT_KT];      // item -> row, up to three tiles ahead
  int32_t qrow[16 * QG * WAVES];
  float far_bias[MUSE_MAXC];   // log2 n_c, or -inf (empty or retrieved)
  int32_t rbeg[MUSE_MAXC];
  int32_t rcum[MUSE_MAXC + 1];
  int32_t sel[4];
};

template <typename TIn, int D, int WAVES>
struct TileRegs {
  static constexpr int NT = 64 * WAVES;
  static constexpr int KC = (AT_KT * D / 8 + NT - 1) / NT;          // 8-wide key chunks
  static constexpr int VB = ((AT_KT / 4) * (D / 8) + NT - 1) / NT;  // 4 items x 8 dims blocks
  using V8 = typename std::conditional<sizeof(TIn) == 2, u16x8, f32x8>::type;
  using V4 = typename std::conditional<sizeof(TIn) == 2, u16x4, f32x4>::type;
  V8 kf[KC];
  V4 vf[VB][8];
  float bias;
  int krow;
};

struct TileSrc {
  int mode;             // 1: far tiles then exact tiles; 2: local rows
  int nfar, nex;
  const void* mu;       // far: [C][D] centroids (input dtype)
  const void* T;        // far: [D][Cp] T_Ic / n_c of this query cluster (input dtype)
  int Ck, Cp;
  const void* Kp;       // exact: sorted keys of the problem
  const void* Vp;
  int nret;
  const void* K;        // local: keys / values of the head
  const void* V;
  int k0, klast;
};

template <typename TIn, typename V8>
__device__ __forceinline__ V8 ld8(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) {
    return *reinterpret_cast<const u16x8*>(p);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

template <typename TIn, typename V4>
__device__ __forceinline__ V4 ld4(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) return *reinterpret_cast<const u16x4*>(p);
  else return *reinterpret_cast<const f32x4*>(p);
}

template <int NS, typename ST>
__device__ __forceinline__ void to_parts(ST x, uint16_t& a, uint16_t& b, uint16_t& c) {
  if constexpr (sizeof(ST) == 2) {
    a = x; b = 0; c = 0;
  } else {
    split3(x, a, b, c);
  }
}

// two floats -> packed bf16 pair (hardware round to nearest even)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Row of item `it` of tile t (exact: sorted position; local: absolute row).
template <typename SM>
__device__ __forceinline__ int item_row(const SM& sm, const TileSrc& src, int t, int it) {
  if (src.mode == 2) {
    const int j = src.k0 + t * AT_KT + it;
    return j <= src.klast ? j : -1;
  }
  if (t < src.nfar) return -1;
  const int v = (t - src.nfar) * AT_KT + it;
  if (v >= src.nret) return -1;
  int r = 0;
  while (sm.rcum[r + 1] <= v) ++r;
  return sm.rbeg[r] + (v - sm.rcum[r]);
}

template <typename TIn, int D, int WAVES, int QG>
__device__ __forceinline__ void tile_load(const AtSmem<TIn, D, WAVES, QG>& sm, const TileSrc& src, int t,
                                          TileRegs<TIn, D, WAVES>& R) {
  using TR = TileRegs<TIn, D, WAVES>;
  constexpr int NT = TR::NT;
  const int tid = threadIdx.x;
  const bool far = src.mode == 1 && t < src.nfar;
  const int base = t * AT_KT;
  const int* ring = sm.ring[t & 3];
#pragma unroll
  for (int q = 0; q < TR::KC; ++q) {
    const int idx = tid + q * NT;
    const int it = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
    const TIn* p = nullptr;
    if (idx < AT_KT * D / 8) {
      if (far) {
        if (base + it < src.Ck) p = reinterpret_cast<const TIn*>(src.mu) + (size_t)(base + it) * D + e0;
      } else {
        const int row = ring[it];
        if (row >= 0)
          p = reinterpret_cast<const TIn*>(src.mode == 1 ? src.Kp : src.K) + (size_t)row * D + e0;
      }
    }
    R.kf[q] = p ? ld8<TIn, typename TR::V8>(p) : typename TR::V8{};
  }
  // value blocks: items 4kb..4kb+3 x dims e0..e0+7, kb fastest across lanes
#pragma unroll
  for (int q = 0; q < TR::VB; ++q) {
    const int idx = tid + q * NT;
    const int kb = idx % (AT_KT / 4), e0 = (idx / (AT_KT / 4)) * 8;
    if (idx >= (AT_KT / 4) * (D / 8)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) R.vf[q][j] = typename TR::V4{};
    } else if (far) {
      const TIn* p = reinterpret_cast<const TIn*>(src.T) + (size_t)e0 * src.Cp + base + 4 * kb;
#pragma unroll
      for (int j = 0; j < 8; ++j) R.vf[q][j] = ld4<TIn, typename TR::V4>(p + (size_t)j * src.Cp);
    } else {
      typename TR::V8 rowv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = ring[4 * kb + r];
        rowv[r] = row >= 0 ? ld8<TIn, typename TR::V8>(
                                 reinterpret_cast<const TIn*>(src.mode == 1 ? src.Vp : src.V) +
                                 (size_t)row * D + e0)
                           : typename TR::V8{};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) R.vf[q][j][r] = rowv[r][j];
    }
  }
  if (tid < AT_KT) {
    if (far) {
      R.bias = base + tid < src.Ck ? sm.far_bias[base + tid] : -INFINITY;
      R.krow = -1;
    } else {
      const int row = ring[tid];
      R.bias = row >= 0 ? 0.f : -INFINITY;
      R.krow = row;
    }
  }
}

template <typename TIn, int D, int WAVES, int QG>
__device__ __forceinline__ void tile_store(AtSmem<TIn, D, WAVES, QG>& sm, int buf,
                                           const TileRegs<TIn, D, WAVES>& R) {
  using TR = TileRegs<TIn, D, WAVES>;
  constexpr int NS = AtSmem<TIn, D, WAVES, QG>::NS;
  constexpr int NT = TR::NT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < TR::KC; ++q) {
    const int idx = tid + q * NT;
    if (idx < AT_KT * D / 8) {
      const int it = idx / (D / 8), e0 = (idx % (D / 8)) * 8;
      if constexpr (NS == 1) {
        *reinterpret_cast<u16x8*>(&sm.ks[buf][0][it][e0]) = R.kf[q];
      } else {
        u16x8 h[NS];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint16_t a, b, c;
          to_parts<NS>(R.kf[q][j], a, b, c);
          h[0][j] = a; h[NS > 1 ? 1 : 0][j] = b; h[NS > 2 ? 2 : 0][j] = c;
        }
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) *reinterpret_cast<u16x8*>(&sm.ks[buf][sp][it][e0]) = h[sp];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < TR::VB; ++q) {
    const int idx = tid + q * NT;
    if (idx < (AT_KT / 4) * (D / 8)) {
      const int kb = idx % (AT_KT / 4), e0 = (idx / (AT_KT / 4)) * 8;
      // items 4kb..4kb+3 land at their contraction slots: within a 32-item
      // block, item r sits at 8(r/4 % 4) + 4(r/16) + r%4
      const int vpos = 32 * (kb / 8) + 8 * (kb % 4) + 4 * ((kb % 8) / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (NS == 1) {
          *reinterpret_cast<u16x4*>(&sm.vt[buf][0][e0 + j][vpos]) = R.vf[q][j];
        } else {
          u16x4 h[NS];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint16_t a, b, c;
            to_parts<NS>(R.vf[q][j][r], a, b, c);
            h[0][r] = a; h[NS > 1 ? 1 : 0][r] = b; h[NS > 2 ? 2 : 0][r] = c;
          }
#pragma unroll
          for (int sp = 0; sp < NS; ++sp) *reinterpret_cast<u16x4*>(&sm.vt[buf][sp][e0 + j][vpos]) = h[sp];
        }
      }
    }
  }
  if (tid < AT_KT) {
    sm.bias[buf][tid] = R.bias;
    sm.krow[buf][tid] = R.krow;
  }
}

template <int D>
struct AtState {
  float m, lpart;         // running max (base 2) and this lane's partial sum
  f32x4 o[D / 16];
};

// Consume a staged tile for the QG query groups of this wave.
template <typename TIn, int D, int WAVES, int QG, bool CAUSAL>
__device__ __forceinline__ void consume_tile(const AtSmem<TIn, D, WAVES, QG>& sm, int buf,
                                             const u16x8 (&qf)[QG][D / 32][AtSmem<TIn, D, WAVES, QG>::NS],
                                             AtState<D> (&st)[QG], float s2, const int (&qrow)[QG]) {
  constexpr int NS = AtSmem<TIn, D, WAVES, QG>::NS;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int RT = AT_KT / 16, PS = AT_KT / 32;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  f32x4 sc[QG][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) sc[qg][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u16x8 a[NS];
#pragma unroll
      for (int sp = 0; sp < NS; ++sp)
        a[sp] = *reinterpret_cast<const u16x8*>(&sm.ks[buf][sp][16 * rt + col][32 * k + 8 * g]);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) sc[qg][rt] = mfma_split<NS, NS>(a, qf[qg][k], sc[qg][rt]);
    }
  }
  f32x4 bv[RT];
  int4 kr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    bv[rt] = *reinterpret_cast<const f32x4*>(&sm.bias[buf][16 * rt + 4 * g]);
    if (CAUSAL) kr[rt] = *reinterpret_cast<const int4*>(&sm.krow[buf][16 * rt + 4 * g]);
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float x[RT * 4];
    float mloc = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = fmaf(s2, sc[qg][rt][i], bv[rt][i]);
        if (CAUSAL) {
          const int krow = i == 0 ? kr[rt].x : i == 1 ? kr[rt].y : i == 2 ? kr[rt].z : kr[rt].w;
          if (krow > qrow[qg]) v = -INFINITY;
        }
        x[rt * 4 + i] = v;
        mloc = fmaxf(mloc, v);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mnew = fmaxf(st[qg].m, mloc);
    const float alpha = __builtin_amdgcn_exp2f(st[qg].m - mnew);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < RT * 4; ++j) {
      x[j] = __builtin_amdgcn_exp2f(x[j] - mnew);
      psum += x[j];
    }
    st[qg].lpart = st[qg].lpart * alpha + psum;
    st[qg].m = mnew;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st[qg].o[dt] *= alpha;
    }
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      // contraction slots of two 16-row tiles: 8g+j -> 4g+j (j<4), 16+4g+(j-4) (j>=4)
      u16x8 pb[NS];
      if constexpr (NS == 1) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const float* pp = &x[ps * 8];
        u32x4 wv = {pk_bf16(pp[0], pp[1]), pk_bf16(pp[2], pp[3]), pk_bf16(pp[4], pp[5]),
                    pk_bf16(pp[6], pp[7])};
        pb[0] = __builtin_bit_cast(u16x8, wv);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint16_t h, mm, l;
          split3(x[ps * 8 + j], h, mm, l);
          pb[0][j] = h; pb[NS > 1 ? 1 : 0][j] = mm; pb[NS > 2 ? 2 : 0][j] = l;
        }
      }
      // V^T fragments of this 32-item block (read per query group: fewer live registers)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u16x8 va[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
          va[sp] = *reinterpret_cast<const u16x8*>(&sm.vt[buf][sp][16 * dt + col][32 * ps + 8 * g]);
        st[qg].o[dt] = mfma_split<NS, NS>(va, pb, st[qg].o[dt]);
      }
    }
  }
}

template <typename TIn, typename TOut, int D, int WAVES, int QG, int MODE>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(D == 64 && WAVES == 4 ? 2 : 1)))
attn_kernel(Plan pl, AttnBufs b, int lev) {
  using SM = AtSmem<TIn, D, WAVES, QG>;
  constexpr int NS = SM::NS, NB = SM::NB;
  constexpr int NT = 64 * WAVES, QT = 16 * QG * WAVES;
  constexpr int KS = D / 32, DT = D / 16;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const float s2 = pl.scale * LOG2E;
  const int C = pl.C;

  int bh, kvh, ap = 0, I = 0, tile, kp = 0, Ck = 0, q0 = 0, k0 = 0;
  int qlo = 0, qhi = 0;
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
    // workgroups are dispatched round-robin over the 8 XCDs: keep every
    // problem on one XCD so its keys and values stay in that XCD's L2
    const int nprob = pl.B * pl.Hq * nseg;
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int slot = loc % spp;
    const int pid = (loc / spp) * 8 + xcd;
    if (pid >= nprob) return;
    const int t = pid % nseg;
    bh = pid / nseg;
    const int p = pl.lev_pfirst[lev] + t;
    ap = bh * pl.P + p;
    const Geom gm = prob_geom(pl, p);
    const int Cq = min(C, gm.qn);
    Ck = min(C, gm.kn);
    k0 = gm.k0;
    q0 = gm.q0;
    const int32_t* qoffs = b.qs.offs + (size_t)ap * (C + 1);
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
          sm.sel[3] = qoffs[c];
        }
        run += v[q];
      }
      if (tid == 63) sm.sel[2] = inc;
    }
    __syncthreads();
    if (slot >= sm.sel[2]) return;
    I = sm.sel[0];
    tile = sm.sel[1];
    qlo = sm.sel[3] + tile * QT;
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

  for (int r = tid; r < QT; r += NT) {
    int row = -1;
    if (qlo + r < qhi) {
      if (MODE == MODE_LOCAL) {
        row = qlo + r;
      } else {
        const int32_t* qperm = b.qs.perm + ((size_t)lev * pl.B * pl.Hq + bh) * pl.N + q0;
        row = qperm[qlo + r];
      }
    }
    sm.qrow[r] = row;
  }
  TileSrc src;
  src.mode = MODE == MODE_LOCAL ? 2 : 1;
  src.nfar = 0;
  if (MODE != MODE_LOCAL) {
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    const int32_t* Rr = b.R + ((size_t)ap * C + I) * pl.k1w;
    for (int c = tid; c < MUSE_MAXC; c += NT) {
      float bias = -INFINITY;
      if (c < Ck) {
        const int nc = koffs[c + 1] - koffs[c];
        if (nc > 0) bias = __log2f((float)nc);
      }
      sm.far_bias[c] = bias;
    }
    int cc[4];
    if (tid < 64) {
      int v[4], bg[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = tid * 4 + q;
        cc[q] = r < pl.k1w ? Rr[r] : -1;
        bg[q] = cc[q] >= 0 ? koffs[cc[q]] : 0;
        v[q] = cc[q] >= 0 ? koffs[cc[q] + 1] - bg[q] : 0;
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
    __syncthreads();
    // retrieved clusters leave the far field
    if (tid < 64) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (cc[q] >= 0) sm.far_bias[cc[q]] = -INFINITY;
    }
    src.nret = sm.rcum[MUSE_MAXC];
    src.nfar = (Ck + AT_KT - 1) / AT_KT;
    src.nex = (src.nret + AT_KT - 1) / AT_KT;
    src.mu = reinterpret_cast<const TIn*>(b.kst.mu_in) + (size_t)kp * C * D;
    src.T = reinterpret_cast<const TIn*>(b.T) + ((size_t)ap * C + I) * D * b.Cp32;
    src.Ck = Ck;
    src.Cp = b.Cp32;
    const size_t kb = (((size_t)lev * pl.B * pl.Hkv + kvh) * pl.N + k0) * D;
    src.Kp = reinterpret_cast<const TIn*>(b.kst.Kp) + kb;
    src.Vp = reinterpret_cast<const TIn*>(b.kst.Vp) + kb;
  } else {
    src.K = reinterpret_cast<const TIn*>(b.K) + (size_t)kvh * pl.N * D;
    src.V = reinterpret_cast<const TIn*>(b.V) + (size_t)kvh * pl.N * D;
    src.k0 = k0;
    src.klast = qhi - 1;
    src.nex = (qhi - k0 + AT_KT - 1) / AT_KT;
  }
  const int ntiles = src.nfar + src.nex;
  if (tid < AT_KT) {
    sm.ring[0][tid] = item_row(sm, src, 0, tid);
    sm.ring[1][tid] = item_row(sm, src, 1, tid);
    sm.ring[2][tid] = item_row(sm, src, 2, tid);
  }
  __syncthreads();

  int myq[QG];
  u16x8 qf[QG][KS][NS];
  AtState<D> st[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    myq[qg] = sm.qrow[(w * QG + qg) * 16 + col];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (myq[qg] >= 0) {
        load8_split<TIn, NS>(Qh + (size_t)myq[qg] * D + 32 * k + 8 * g, qf[qg][k]);
      } else {
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
#pragma unroll
          for (int j = 0; j < 8; ++j) qf[qg][k][sp][j] = 0;
      }
    }
    st[qg].m = -1e30f;
    st[qg].lpart = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st[qg].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int qmask[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) qmask[qg] = myq[qg] < 0 ? 0x7fffffff : myq[qg];

  if constexpr (NB == 2) {
    // two tiles in flight in registers: the loads of tile t+2 are issued
    // before tile t is consumed and written to LDS after tile t+1 is
    TileRegs<TIn, D, WAVES> R0, R1;
    if (ntiles > 0) tile_load(sm, src, 0, R0);
    if (ntiles > 1) tile_load(sm, src, 1, R1);
    if (ntiles > 0) tile_store(sm, 0, R0);
    __syncthreads();
    auto step = [&](int t, TileRegs<TIn, D, WAVES>& Rload, const TileRegs<TIn, D, WAVES>& Rstore) {
      if (tid < AT_KT && t + 3 < ntiles) sm.ring[(t + 3) & 3][tid] = item_row(sm, src, t + 3, tid);
      if (t + 2 < ntiles) tile_load(sm, src, t + 2, Rload);
      consume_tile<TIn, D, WAVES, QG, MODE == MODE_LOCAL>(sm, t & 1, qf, st, s2, qmask);
      if (t + 1 < ntiles) tile_store(sm, (t + 1) & 1, Rstore);
      __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, R0, R1);
      if (t + 1 < ntiles) step(t + 1, R1, R0);
    }
  } else {
    TileRegs<TIn, D, WAVES> R;
    if (ntiles > 0) {
      tile_load(sm, src, 0, R);
      tile_store(sm, 0, R);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      if (tid < AT_KT && t + 2 < ntiles) sm.ring[(t + 2) & 3][tid] = item_row(sm, src, t + 2, tid);
      if (more) tile_load(sm, src, t + 1, R);
      consume_tile<TIn, D, WAVES, QG, MODE == MODE_LOCAL>(sm, 0, qf, st, s2, qmask);
      __syncthreads();
      if (more) tile_store(sm, 0, R);
      __syncthreads();
    }
  }

  // ---- finish: normalise, write or merge (lse in natural log units) ----
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float l = st[qg].lpart;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = myq[qg];
    if (row < 0) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (st[qg].m + __log2f(l)) * LN2 : -INFINITY;
    if (MODE == MODE_ACAUSAL) {
      TOut* O = reinterpret_cast<TOut*>(b.O) + ((size_t)bh * pl.N + row) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if constexpr (sizeof(TOut) == 2) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          u32x2 wv = {pk_bf16(st[qg].o[dt][0] * inv, st[qg].o[dt][1] * inv),
                      pk_bf16(st[qg].o[dt][2] * inv, st[qg].o[dt][3] * inv)};
          *reinterpret_cast<u32x2*>(O + 16 * dt + 4 * g) = wv;
        } else {
          *reinterpret_cast<f32x4*>(O + 16 * dt + 4 * g) = st[qg].o[dt] * inv;
        }
      }
      if (g == 0) b.lse[(size_t)bh * pl.N + row] = lse;
    } else {
      float* oa = b.oacc + ((size_t)bh * pl.N + row) * D;
      float* la = b.lacc + (size_t)bh * pl.N + row;
      if (MODE == MODE_LOCAL) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = st[qg].o[dt] * inv;
        if (g == 0) *la = lse;
      } else {
        if (!(l > 0.f)) continue;
        const float lold = *la;
        const float L = fmaxf(lold, lse);
        const float wo = __expf(lold - L), wn = __expf(lse - L);
        const float tot = wo + wn;
        const float fo = wo / tot, fn = wn * inv / tot;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          f32x4 prev = *reinterpret_cast<const f32x4*>(oa + 16 * dt + 4 * g);
          *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = prev * fo + st[qg].o[dt] * fn;
        }
        if (g == 0) *la = L + logf(tot);
      }
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
template <typename TIn, int D, int WAVES, int QG>
static hipError_t attn_level(const Plan& pl, const AttnBufs& b, int lev, hipStream_t st) {
  constexpr int QT = 16 * QG * WAVES;
  const int spp = (pl.lev_m[lev] + QT - 1) / QT + pl.C;
  const long long nprob = (long long)pl.B * pl.Hq * pl.lev_nseg[lev];
  const long long grid = ((nprob + 7) / 8) * 8 * spp;
  if (grid == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  if (pl.causal)
    attn_kernel<TIn, TIn, D, WAVES, QG, MODE_LEVEL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, lev);
  else
    attn_kernel<TIn, TIn, D, WAVES, QG, MODE_ACAUSAL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, lev);
  MUSE_KT_POST(pl.causal ? "attn_level" : "attn_far_retrieve", st);
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t attn_all(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  hipError_t e = hipSuccess;
  constexpr int QG = sizeof(TIn) == 2 ? 2 : 1;
  if (pl.causal) {
    constexpr int WAVES = 4, QT = 16 * QG * 4;
    const int nblk = (pl.N + pl.blk - 1) / pl.blk;
    const long long grid = (long long)pl.B * pl.Hq * nblk * ((pl.blk + QT - 1) / QT);
    MUSE_KT_PRE(st);
    attn_kernel<TIn, TIn, D, WAVES, QG, MODE_LOCAL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, 0);
    MUSE_KT_POST("attn_local", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  for (int lev = 0; lev < pl.nlev; ++lev) {
    // query clusters of ~m/C rows: the query tile (rows per workgroup) follows
    // the mean cluster size so that ragged clusters waste few tile rows
    const int avg = pl.lev_m[lev] / (pl.C > 0 ? pl.C : 1);
    if (QG == 2 && avg >= 160) e = attn_level<TIn, D, 4, QG>(pl, b, lev, st);
    else if (avg >= 48) e = attn_level<TIn, D, 4, 1>(pl, b, lev, st);
    else e = attn_level<TIn, D, 1, 1>(pl, b, lev, st);
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
