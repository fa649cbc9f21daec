// Stage two of the two-stage attention and the exact parts of the causal
// hierarchy (gist.science page, Technical Summary, Core Mechanisms:
// Decomposition, Hierarchical Two-Stage Attention, Retrieval-Augmented
// Approximation; newx.sg page, Abstract: exact local blocks).
//
// For a query i of query cluster I the softmax runs over two kinds of
// items: every key j of a retrieved cluster (logit s q_i.k_j, weight 1,
// value v_j) and every other non-empty key cluster c (logit s q_i.mu_c,
// weight n_c, value T_Ic / n_c).  Both kinds go through the same tile loop:
// a tile is 64 items, staged in LDS as key rows (A operand of S^T = K Q^T)
// and as value columns (A operand of O^T = V^T P^T); one online softmax
// (base 2) covers all tiles.  The local causal block uses the same loop over
// contiguous keys with the causal mask.
//
// Tiles.  A far tile is 64 consecutive key clusters (centroid rows, and the
// columns of T_I, which is stored dim-major).  An exact tile is 64
// consecutive rows of the cluster-contiguous key copy, starting at a multiple
// of 8: a retrieved cluster [lo, hi) is covered by tiles from lo rounded down
// to 8 in steps of 64, and rows outside [lo, hi) are masked.  Values come
// from a dim-major copy of the same rows (built by vt_kernel), so both halves
// of a tile are 64 x 16-byte row segments: they are copied global -> LDS by
// the direct-to-LDS loads, with no register staging and no transposition.
// One-wave workgroups (query clusters of under 48 rows, where key clusters
// are as small) gather their exact tiles instead: a tile is 8 chunks of 8
// rows, each chunk from a multiple of 8 inside one retrieved cluster, so
// several small clusters share a tile rather than each padding its own.
//
// Pipeline: ST LDS stages, tile t+ST-1 is in flight while tile t is
// consumed; one barrier per tile.  One-wave workgroups use a single stage
// (copy, wait, consume): at half the LDS twice as many run per CU, and their
// copies overlap each other's work.  The waits on the copies are explicit
// (s_waitcnt vmcnt with the number of copies issued after the tile), so the
// loop holds no other global loads.  LDS rows are 16-byte-chunk swizzled so
// that the fragment reads are free of bank conflicts.
//
// Contraction order: the S^T MFMA of row tile rt reads, for its A row c, the
// key item 32(rt/2) + 8(c/4) + 4(rt%2) + c%4, so that the scores a lane holds
// for two consecutive row tiles are 8 consecutive items: they pack directly
// into the P^T operand of the value MFMA, whose V^T operand is then a plain
// 16-byte read of one value column.
// Each wave holds QG groups of 16 queries so that every fragment read from
// LDS feeds QG matrix instructions.
#include <utility>

#include "common.h"
#include "launch.h"
#include "vt.h"

namespace muse {

enum { MODE_ACAUSAL = 0, MODE_LEVEL = 1, MODE_LOCAL = 2, MODE_V4 = 3 };
constexpr int AT_KT = 64;   // items per tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// One 16-byte direct-to-LDS copy per lane: lane l's 16 bytes at `src` land
// at LDS byte lds + 16 l (lds wave-uniform).  Written as assembly so that the
// compiler does not track it: it would otherwise wait for every copy in
// flight before any read of the stage array, and the loop's explicit waits
// cover these copies.  The instruction writes no register.
__device__ __forceinline__ void lds_copy16(const void* src, const void* lds) {
  const uint32_t a = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(a), "v"(src) : "memory", "m0");
}

// The same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the saddr form): a tile's per-lane offsets do not
// change from tile to tile, so each copy costs no address arithmetic.
template <int IMM>
__device__ __forceinline__ void lds_copy16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %0, %3\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds), "v"(voff), "s"(sbase),
               "i"(IMM) : "memory", "m0");
}
// copies M... of one half of a tile: destination l0 + OFF + M * STEP
template <int OFF, int STEP, size_t... M>
__device__ __forceinline__ void lds_copies_s(const void* sbase, const uint32_t* voff, uint32_t l0,
                                             std::index_sequence<M...>) {
  (lds_copy16_s<OFF + (int)M * STEP>(sbase, voff[M], l0), ...);
}

// s_waitcnt immediate for vmcnt(v) and lgkmcnt(l), expcnt left alone.
__host__ __device__ constexpr int at_wait(int v, int l) {
  return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (l << 8);
}

template <typename TIn, int D>
struct AtGeo {
  static constexpr int E = 16 / (int)sizeof(TIn);            // elements per 16-byte chunk
  static constexpr int CHK = D / E;                           // chunks per key row
  static constexpr int CHV = AT_KT / E;                       // chunks per value column row
  static constexpr int KB = AT_KT * D * (int)sizeof(TIn);     // key block bytes
  static constexpr int SB = 2 * KB;                           // stage bytes
  static constexpr int ST = SB <= 16384 ? 3 : 2;              // stages
};

// chunk swizzles (chunk position = logical chunk ^ key).  The 16 key rows of
// one fragment read differ in bits 0, 1, 3 and 4 of r: with 8 chunks a row
// (128 bytes, rows alternating bank halves) 3 key bits spread them over
// distinct banks; with 16 or more (256-byte rows, all starting on bank 0)
// it takes 4.
template <int CHK>
__device__ __forceinline__ int keyk(int r) {
  return CHK >= 16 ? (r & 3) | ((r >> 1) & 12) : (r & 3) | ((r >> 1) & 4);
}
__device__ __forceinline__ int keyv(int d) { return d & 7; }

// Everything in LDS but the tile stages, which are a __shared__ array of
// their own: the compiler then sees that reads of these tables cannot alias
// the copies in flight and does not wait for them.
template <typename TIn, int D, int WAVES, int QG>
struct alignas(16) AtSmem {
  float far_bias[MUSE_MAXC];   // (log2 n_c or the tilt bias) / s2, or -inf (empty or retrieved)
  int32_t seg_lo[MUSE_MAXC];   // retrieved clusters (non-empty), absolute rows
  int32_t seg_hi[MUSE_MAXC];
  int32_t qrow[16 * QG * WAVES];
  int32_t sel[8];
};

struct TileSrc {
  const void* Kx;     // key rows, absolute row index (sorted copy or input K)
  const void* Vt;     // value columns [D][nv] of the same rows
  int nv;             // Vt row length (multiple of 8)
  int kmax;           // last key row that may be read
  const void* mu;     // far: centroid rows [C][D]
  const void* T;      // far: T_I / n_c, [D][Cp]
  int Ck, Cp;
  int nfar, nseg;
};

// Walks the tile list in order: nfar far tiles, then for each retrieved
// cluster the tiles covering it.  All fields are wave-uniform.
struct Cursor {
  int t, j, row0, lo, hi;
};

template <typename SM>
__device__ __forceinline__ Cursor cur_seg(const SM& sm, const TileSrc& src, int t, int j) {
  const bool ok = j < src.nseg;
  const int lo = __builtin_amdgcn_readfirstlane(sm.seg_lo[ok ? j : 0]);
  const int hi = __builtin_amdgcn_readfirstlane(sm.seg_hi[ok ? j : 0]);
  Cursor c;
  c.t = t;
  c.j = j;
  c.lo = ok ? lo : 0;
  c.hi = ok ? hi : 0;
  c.row0 = c.lo & ~7;
  return c;
}

template <typename SM>
__device__ __forceinline__ Cursor cur_first(const SM& sm, const TileSrc& src) {
  Cursor c = cur_seg(sm, src, 0, 0);
  if (src.nfar > 0) c.row0 = 0;
  return c;
}

template <typename SM>
__device__ __forceinline__ Cursor cur_next(const SM& sm, const TileSrc& src, Cursor c) {
  const int t = c.t + 1;
  if (t < src.nfar) {
    c.t = t;
    c.row0 = AT_KT * t;
    return c;
  }
  if (t == src.nfar) return cur_seg(sm, src, t, 0);
  if (c.row0 + AT_KT >= c.hi && c.j < src.nseg) return cur_seg(sm, src, t, c.j + 1);
  c.t = t;
  c.row0 += AT_KT;
  return c;
}

// Copy tile (cursor c) into stage s: every thread issues the same number of
// 16-byte direct-to-LDS loads; rows past the end read clamped, valid rows.
template <typename TIn, int D, int WAVES>
__device__ __forceinline__ void issue_tile(unsigned char* stg, const TileSrc& src, const Cursor& c) {
  using G = AtGeo<TIn, D>;
  constexpr int NT = 64 * WAVES;
  static_assert(AT_KT * G::CHK % NT == 0 && D * G::CHV % NT == 0, "copies must cover the workgroup");
  const int tid = threadIdx.x, w = tid >> 6;
  const bool far = c.t < src.nfar;
  unsigned char* kst = stg;
  unsigned char* vst = stg + G::KB;
  const TIn* kb = reinterpret_cast<const TIn*>(far ? src.mu : src.Kx);
  const int kcap = far ? src.Ck - 1 : src.kmax;
#pragma unroll
  for (int m = 0; m < AT_KT * G::CHK / NT; ++m) {
    const int ci = m * NT + tid;
    const int r = ci / G::CHK, pos = ci % G::CHK;
    const int row = min(c.row0 + r, kcap);
    const TIn* p = kb + (size_t)row * D + (pos ^ keyk<G::CHK>(r)) * G::E;
    lds_copy16(p, kst + (m * NT + 64 * w) * 16);
  }
  const TIn* vb = reinterpret_cast<const TIn*>(far ? src.T : src.Vt);
  const int vstride = far ? src.Cp : src.nv;
  const int vcap = far ? src.Cp - G::E : src.nv - G::E;
#pragma unroll
  for (int m = 0; m < D * G::CHV / NT; ++m) {
    const int ci = m * NT + tid;
    const int d = ci / G::CHV, pos = ci % G::CHV;
    const int col = min(c.row0 + (pos ^ keyv(d)) * G::E, vcap);
    const TIn* p = vb + (size_t)d * vstride + col;
    lds_copy16(p, vst + (m * NT + 64 * w) * 16);
  }
}

// Per-lane byte offsets of a contiguous tile's copies (issue_tile's layout):
// key rows (row stride D) and value columns (row stride vstride).
template <typename TIn, int D, int WAVES>
struct TileOffs {
  static constexpr int NT = 64 * WAVES;
  static constexpr int MK = AT_KT * AtGeo<TIn, D>::CHK / NT, MV = D * AtGeo<TIn, D>::CHV / NT;
  uint32_t k[MK], vx[MV], vf[MV];
  __device__ __forceinline__ void init(int tid, int nv, int cp) {
    using G = AtGeo<TIn, D>;
    constexpr int esz = (int)sizeof(TIn);
#pragma unroll
    for (int m = 0; m < MK; ++m) {
      const int ci = m * NT + tid, r = ci / G::CHK, pos = ci % G::CHK;
      k[m] = (uint32_t)((r * D + (pos ^ keyk<G::CHK>(r)) * G::E) * esz);
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      const int ci = m * NT + tid, d = ci / G::CHV, pos = ci % G::CHV;
      const int col = (pos ^ keyv(d)) * G::E;
      vx[m] = (uint32_t)((d * nv + col) * esz);
      vf[m] = (uint32_t)((d * cp + col) * esz);
    }
  }
};

// issue_tile for a tile whose 64 key rows and value columns all lie inside
// their arrays (no clamping needed): bases in SGPRs, offsets from TileOffs.
template <typename TIn, int D, int WAVES>
__device__ __forceinline__ void issue_tile_fast(unsigned char* stg, const void* kb, const void* vb,
                                                const uint32_t* koff, const uint32_t* voff, int ws) {
  using G = AtGeo<TIn, D>;
  using O = TileOffs<TIn, D, WAVES>;
  // LDS destinations: one wave-uniform base plus immediate offsets
  const uint32_t l0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)stg) + 64 * 16 * ws;
  lds_copies_s<0, O::NT * 16>(kb, koff, l0, std::make_index_sequence<O::MK>{});
  lds_copies_s<G::KB, O::NT * 16>(vb, voff, l0, std::make_index_sequence<O::MV>{});
}

// Gathered tiles (small clusters).  A tile is 8 chunks of 8 consecutive rows.  Far tile t: clusters 64t ..
// 64t+63.  Exact tile: the next 8 chunks of the retrieved clusters, each
// chunk 8 rows from a multiple of 8 inside one cluster's rows (rows outside
// the cluster are masked), so small clusters share a tile.  All fields are
// wave-uniform.
struct TDesc {
  int far;
  int base[8];         // first row (exact) or cluster (far) of each chunk
  uint32_t vlo, vhi;   // exact: valid items 0..31, 32..63
};

// Position in the chunk list: next tile, current cluster and next chunk row.
struct Chunks {
  int t, j, base, lo, hi;
};

template <typename SM>
__device__ __forceinline__ Chunks chunks_first(const SM& sm, const TileSrc& src) {
  Chunks c;
  const bool ok = src.nseg > 0;
  c.t = 0;
  c.j = 0;
  c.lo = ok ? __builtin_amdgcn_readfirstlane(sm.seg_lo[0]) : 0;
  c.hi = ok ? __builtin_amdgcn_readfirstlane(sm.seg_hi[0]) : 0;
  c.base = c.lo & ~7;
  return c;
}

// Descriptor of the next tile; advances c.  Past the end, chunks read rows
// 0..7 with no valid item.
template <typename SM>
__device__ __forceinline__ TDesc take_tile(const SM& sm, const TileSrc& src, Chunks& c) {
  TDesc d;
  const int t = c.t;
  c.t = t + 1;
  d.far = t < src.nfar;
  if (d.far) {
#pragma unroll
    for (int k = 0; k < 8; ++k) d.base[k] = AT_KT * t + 8 * k;
    d.vlo = ~0u;
    d.vhi = ~0u;
    return d;
  }
  int j = c.j, base = c.base, lo = c.lo, hi = c.hi;
  uint32_t vm0 = 0, vm1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (base >= hi && j < src.nseg) {   // next cluster (non-empty by construction)
      ++j;
      const bool ok = j < src.nseg;
      const int nlo = __builtin_amdgcn_readfirstlane(sm.seg_lo[ok ? j : 0]);
      const int nhi = __builtin_amdgcn_readfirstlane(sm.seg_hi[ok ? j : 0]);
      lo = ok ? nlo : 0;
      hi = ok ? nhi : 0;
      base = lo & ~7;
    }
    // past the last cluster every chunk stays on rows 0..7 (rows every
    // sorted copy holds), with no valid item
    if (j >= src.nseg) base = 0;
    d.base[k] = base;
    const int a = max(lo - base, 0), b = min(hi - base, 8);
    const uint32_t bits = b > a ? (1u << b) - (1u << a) : 0u;
    if (k < 4) vm0 |= bits << (8 * k);
    else vm1 |= bits << (8 * (k - 4));
    base += 8;
  }
  c.j = j;
  c.base = base;
  c.lo = lo;
  c.hi = hi;
  d.vlo = vm0;
  d.vhi = vm1;
  return d;
}

// base[k] for a wave-uniform or per-lane chunk index k
// (a select tree on the bits of k, so that base[] is never indexed at run time)
__device__ __forceinline__ int pick8(const TDesc& d, int k) {
  const bool b0 = k & 1, b1 = k & 2, b2 = k & 4;
  const int x01 = b0 ? d.base[1] : d.base[0], x23 = b0 ? d.base[3] : d.base[2];
  const int x45 = b0 ? d.base[5] : d.base[4], x67 = b0 ? d.base[7] : d.base[6];
  const int x03 = b1 ? x23 : x01, x47 = b1 ? x67 : x45;
  return b2 ? x47 : x03;
}

// Copy tile d into stage stg: every thread issues the same number of
// 16-byte direct-to-LDS loads; rows past the end read clamped, valid rows.
// One load instruction of a wave covers 1 KB of key rows, never more than
// one chunk, so the key chunk of an instruction is wave-uniform; each lane's
// 16 bytes of a value row hold items of a single chunk.
template <typename TIn, int D, int WAVES>
__device__ __forceinline__ void issue_tile_g(unsigned char* stg, const TileSrc& src, const TDesc& d) {
  using G = AtGeo<TIn, D>;
  constexpr int NT = 64 * WAVES;
  static_assert(AT_KT * G::CHK % NT == 0 && D * G::CHV % NT == 0, "copies must cover the workgroup");
  static_assert(8 * G::CHK >= 64, "a 1 KB copy must stay inside one chunk");
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned char* kst = stg;
  unsigned char* vst = stg + G::KB;
  // (fields read into values first: a select between field addresses would
  // keep the source descriptor in memory)
  const bool far = d.far;
  const TIn *mu = reinterpret_cast<const TIn*>(src.mu), *kx = reinterpret_cast<const TIn*>(src.Kx);
  const TIn *tt = reinterpret_cast<const TIn*>(src.T), *vt = reinterpret_cast<const TIn*>(src.Vt);
  const int ck = src.Ck, kmax = src.kmax, cp = src.Cp, nv = src.nv;
  const TIn* kb = far ? mu : kx;
  const int kcap = far ? ck - 1 : kmax;
#pragma unroll
  for (int m = 0; m < AT_KT * G::CHK / NT; ++m) {
    const int ci = m * NT + tid;
    const int r = ci / G::CHK, pos = ci % G::CHK;
    const int kchunk = (m * NT + 64 * w) / (8 * G::CHK);   // wave-uniform
    const int row = min(pick8(d, kchunk) + (r & 7), kcap);
    const TIn* p = kb + (size_t)row * D + (pos ^ keyk<G::CHK>(r)) * G::E;
    lds_copy16(p, kst + (m * NT + 64 * w) * 16);
  }
  const TIn* vb = far ? tt : vt;
  const int vstride = far ? cp : nv;
  const int vcap = (far ? cp : nv) - G::E;
#pragma unroll
  for (int m = 0; m < D * G::CHV / NT; ++m) {
    const int ci = m * NT + tid;
    const int dd = ci / G::CHV, pos = ci % G::CHV;
    const int lj = pos ^ keyv(dd);             // logical 16-byte chunk of the row
    const int kc = lj * G::E / 8;              // its 8-item chunk
    const int col = min(pick8(d, kc) + (lj * G::E) % 8, vcap);
    const TIn* p = vb + (size_t)dd * vstride + col;
    lds_copy16(p, vst + (m * NT + 64 * w) * 16);
  }
}

// Gathered exact tiles from a chunk table (one-wave workgroups, bf16 at
// D = 64).  The exact chunks of a workgroup are listed once, in tile order:
// lane l of tab.b[i] holds the first row of chunk 64i + l, and lane l of
// tab.m the valid-row bytes of chunks 4l .. 4l+3 (zero past the last chunk).
// A tile's descriptor is then eight lane reads of the table, and its copies
// use scalar row bases with per-lane offsets that never change.
constexpr int GX_MAXCH = 256;   // chunks the table holds (32 tiles)
struct GxTab {
  int b0, b1, b2, b3;    // chunk bases (four registers: GX_MAXCH = 256)
  uint32_t m;
  uint32_t voff_k[2];   // key-copy byte offsets within a chunk (even, odd copy)
};
static_assert(GX_MAXCH == 256, "the table is four registers of chunk bases");

// List the exact chunks of the nseg retrieved segments (row ranges in
// seg_lo/seg_hi) into scratch LDS (bases at cb[], valid-row bytes at cm[]),
// then read them into the register table.  nch = total chunks <= GX_MAXCH.
template <typename SM>
__device__ __forceinline__ void gx_build(const SM& sm, int nseg, int nch, int32_t* cb, uint8_t* cm, GxTab& tab) {
  const int lane = threadIdx.x & 63;
  int run = 0;   // chunks before this round of 64 segments
  for (int j0 = 0; j0 < nseg; j0 += 64) {
    const int j = j0 + lane;
    const int lo = j < nseg ? sm.seg_lo[j] : 0, hi = j < nseg ? sm.seg_hi[j] : 0;
    const int first = lo & ~7;
    const int cnt = j < nseg ? (hi - first + 7) >> 3 : 0;
    int inc = cnt;
    for (int mm = 1; mm < 64; mm <<= 1) {
      const int o = __shfl_up(inc, mm, 64);
      if (lane >= mm) inc += o;
    }
    const int start = run + inc - cnt;
    for (int c = 0; c < cnt; ++c) {
      const int base = first + 8 * c;
      const int a = max(lo - base, 0), bb = min(hi - base, 8);
      if (start + c < GX_MAXCH) {
        cb[start + c] = base;
        cm[start + c] = (uint8_t)(bb > a ? (1u << bb) - (1u << a) : 0u);
      }
    }
    run += __shfl(inc, 63, 64);
  }
  __syncthreads();
  tab.b0 = lane < nch ? cb[lane] : 0;
  tab.b1 = 64 + lane < nch ? cb[64 + lane] : 0;
  tab.b2 = 128 + lane < nch ? cb[128 + lane] : 0;
  tab.b3 = 192 + lane < nch ? cb[192 + lane] : 0;
  uint32_t mw = *reinterpret_cast<const uint32_t*>(cm + 4 * lane);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 * lane + q >= nch) mw &= ~(0xffu << (8 * q));
  tab.m = mw;
  // key copy of chunk m: lane t takes row (t/8) & 7 of the chunk, 16-byte
  // piece (t & 7) ^ keyk(8m + t/8) (issue_tile_g's layout)
  const int r7 = (lane >> 3) & 7;
#pragma unroll
  for (int p = 0; p < 2; ++p)
    tab.voff_k[p] = (uint32_t)((r7 * 64 + (((lane & 7) ^ ((r7 & 3) | (p << 2))) * 8)) * 2);
  // the tile stage is overwritten next: every table read must have returned
  __builtin_amdgcn_s_waitcnt(at_wait(63, 0));
  __syncthreads();
}

// Descriptor of exact tile te (chunks 8te .. 8te+7) from the table.
__device__ __forceinline__ TDesc gx_tile(const GxTab& tab, int te) {
  TDesc d;
  d.far = 0;
  const int r = te >> 3;
  const int reg = r == 0 ? tab.b0 : r == 1 ? tab.b1 : r == 2 ? tab.b2 : tab.b3;
  const int l0 = (8 * te) & 63;
#pragma unroll
  for (int k = 0; k < 8; ++k) d.base[k] = __builtin_amdgcn_readlane(reg, l0 + k);
  d.vlo = (uint32_t)__builtin_amdgcn_readlane((int)tab.m, (2 * te) & 63);
  d.vhi = (uint32_t)__builtin_amdgcn_readlane((int)tab.m, (2 * te + 1) & 63);
  return d;
}

// key copies of chunks M..: row base (scalar) + the lane's fixed offset
template <size_t... M>
__device__ __forceinline__ void gx_kcopies(const unsigned char* kx, const TDesc& d, const uint32_t (&vo)[2],
                                           uint32_t l0, std::index_sequence<M...>) {
  (lds_copy16_s<(int)M * 1024>(kx + (size_t)d.base[M] * 128, vo[M & 1], l0), ...);
}
// value copies M..: value rows 8M + t/8 at the lane's chunk column
template <size_t... M>
__device__ __forceinline__ void gx_vcopies(const unsigned char* vt, size_t rstep, uint32_t vo, uint32_t l0,
                                           std::index_sequence<M...>) {
  (lds_copy16_s<8192 + (int)M * 1024>(vt + M * rstep, vo, l0), ...);
}

// issue_tile_g for an exact bf16 D = 64 tile of the table whose rows all lie
// inside the key array (one wave): 8 key and 8 value copies of 1 KB.
__device__ __forceinline__ void issue_tile_gx(unsigned char* stg, const TileSrc& src, const TDesc& d,
                                              const GxTab& tab) {
  const int lane = threadIdx.x & 63;
  const uint32_t l0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)stg);
  gx_kcopies(reinterpret_cast<const unsigned char*>(src.Kx), d, tab.voff_k, l0, std::make_index_sequence<8>{});
  // value column chunk of this lane: (t & 7) ^ ((t/8) & 7), fixed per lane
  const int lj = (lane & 7) ^ ((lane >> 3) & 7);
  const int col = pick8(d, lj);
  const uint32_t vo = (uint32_t)((((lane >> 3) & 7) * src.nv + col) * 2);
  gx_vcopies(reinterpret_cast<const unsigned char*>(src.Vt), (size_t)16 * src.nv, vo, l0,
             std::make_index_sequence<8>{});
}

// What consume_tile needs to know of a tile: far or exact, plain (no mask
// at all), its first row (far: first cluster; local: first key row) and the
// lane's valid items (bit rt*4 + i for item 32(rt/2) + 8g + 4(rt%2) + i).
struct TileView {
  int far, plain, row0;
  uint32_t okm;
};

__device__ __forceinline__ TileView view_of(const TDesc& d) {
  TileView v;
  const int g = (threadIdx.x & 63) >> 4;
  v.far = d.far;
  v.row0 = d.base[0];
  v.plain = !d.far && d.vlo == ~0u && d.vhi == ~0u;
  v.okm = ((d.vlo >> (8 * g)) & 0xffu) | (((d.vhi >> (8 * g)) & 0xffu) << 8);
  return v;
}

template <bool CAUSAL>
__device__ __forceinline__ TileView view_of(const TileSrc& src, const Cursor& c, int qmin) {
  TileView v;
  v.far = c.t < src.nfar;
  v.row0 = c.row0;
  // a plain tile lies inside [lo, hi) and (causal) below every query row of the workgroup
  v.plain = !v.far && c.row0 >= c.lo && c.row0 + AT_KT <= c.hi && (!CAUSAL || c.row0 + AT_KT - 1 <= qmin);
  uint32_t ok = 0xffffu;
  if (!v.far && !v.plain) {
    // tile items [a, b) lie in [lo, hi): a 64-bit range mask (wave-uniform);
    // the lane's items 8g + 0..7 and 32 + 8g + 0..7 are byte g of each half
    const int a = min(max(c.lo - c.row0, 0), AT_KT), b = min(max(c.hi - c.row0, 0), AT_KT);
    const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1, below_b = b >= 64 ? ~0ull : (1ull << b) - 1;
    const uint64_t rng = below_b & ~below_a;
    const int g8 = 8 * ((threadIdx.x & 63) >> 4);
    ok = (((uint32_t)rng >> g8) & 0xffu) | ((((uint32_t)(rng >> 32)) >> g8) & 0xffu) << 8;
  }
  v.okm = ok;
  return v;
}

// The highest causal level whose query half holds row i, or -1 when only
// the local block does.  Level l has span m = blk 2^l and its t-th segment
// takes queries [2tm + m, 2tm + 2m): the rows whose local block index
// q = floor(i / blk) has bit l set (and segment q >> (l+1) exists).
__device__ __forceinline__ int last_level(const Plan& pl, int i) {
  const int q = i / pl.blk;
  if (pl.v4) return q >= 1 ? 0 : -1;   // spatial blocks: one pass for every block after the first
  int last = -1;
  for (int l = 0; l < pl.nlev; ++l)
    if (((q >> l) & 1) && (q >> (l + 1)) < pl.lev_nseg[l]) last = l;
  return last;
}

// 8 consecutive elements (logical 8-element group lg of a row) as NS bf16 parts.
template <typename TIn, int NS>
__device__ __forceinline__ void lds_frag(const unsigned char* row, int lg, int key, u16x8* out) {
  if constexpr (sizeof(TIn) == 2) {
    out[0] = *reinterpret_cast<const u16x8*>(row + ((lg ^ key) << 4));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + (((2 * lg) ^ key) << 4));
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + (((2 * lg + 1) ^ key) << 4));
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


template <int D>
struct AtState {
  float m;                // running max (base 2)
  f32x4 lsum;             // row sums from the matrix cores: element 0 of lanes 0..15 (tile row 0)
  f32x4 o[D / 16];
};

// Consume the tile (cursor c) staged in stage s for the QG query groups of
// this wave.  Score slot (rt, 4g + i) of a lane is item
// 32(rt/2) + 8g + 4(rt%2) + i of the tile.
// Consume the tile (cursor c) staged in stage s for the QG query groups of
// this wave.  Score slot (rt, 4g + i) of a lane is item
// 32(rt/2) + 8g + 4(rt%2) + i of the tile.
//
// Every item's logit is s2 (score + b): b = 0 for exact keys, and for far
// items their bias divided by s2 (the log-count or tilt bias, minus infinity
// for retrieved and empty clusters).  The raw scores are adjusted in place
// (far tiles add b; tiles with invalid items replace those scores by minus
// infinity, not offset them, since rows outside the key segments of a level
// hold unspecified values), and one softmax step follows for every kind of
// tile, with the scale folded into the exponent.
template <typename TIn, int D, int WAVES, int QG, bool CAUSAL>
__device__ __forceinline__ void consume_tile(const AtSmem<TIn, D, WAVES, QG>& sm, const unsigned char* stg,
                                             const TileView& tv,
                                             const u16x8 (&qf)[QG][D / 32][sizeof(TIn) == 2 ? 1 : 3],
                                             AtState<D> (&st)[QG], float s2, const int (&qrow)[QG],
                                             const u16x8& ones) {
  using G = AtGeo<TIn, D>;
  constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int RT = AT_KT / 16, PS = AT_KT / 32;
  constexpr int KROW = D * (int)sizeof(TIn), VROW = AT_KT * (int)sizeof(TIn);
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const unsigned char* kst = stg;
  const unsigned char* vst = stg + G::KB;
  f32x4 sc[QG][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 32 * (rt >> 1) + 8 * (col >> 2) + 4 * (rt & 1) + (col & 3);
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) sc[qg][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      u16x8 a[NS];
      lds_frag<TIn, NS>(kst + r * KROW, 4 * k + g, keyk<G::CHK>(r), a);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) sc[qg][rt] = mfma_split<NS, NS>(a, qf[qg][k], sc[qg][rt]);
    }
  }
  if (tv.far) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int it0 = 32 * (rt >> 1) + 8 * g + 4 * (rt & 1);
      const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.far_bias[tv.row0 + it0]);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) sc[qg][rt] += b;
    }
  } else if (!tv.plain) {
    const uint32_t ok = tv.okm;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int it0 = 32 * (rt >> 1) + 8 * g + 4 * (rt & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // an all-ones / all-zeros mask from the item's bit selects the score
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)ok, rt * 4 + i, 1);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float v = __uint_as_float((__float_as_uint(sc[qg][rt][i]) & keep) | (0xff800000u & ~keep));
          if (CAUSAL && tv.row0 + it0 + i > qrow[qg]) v = -INFINITY;
          sc[qg][rt][i] = v;
        }
      }
    }
  }
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float mloc = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sc[qg][rt][i]);
    mloc = max4_lanes(mloc * s2);
    // lazy rescale: the running max of a row moves only when the tile's max
    // exceeds it by more than 8 (weights stay below 2^8, exact in the end
    // since output and normaliser share the same max)
    const float mcand = fmaxf(st[qg].m, mloc);
    const bool grow = mcand > st[qg].m + 8.f;
    if (__any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(st[qg].m - mcand) : 1.f;
      st[qg].lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st[qg].o[dt] *= alpha;
      st[qg].m = grow ? mcand : st[qg].m;
    }
    const float mref = st[qg].m;
    float x[RT * 4];
#pragma unroll
    for (int j = 0; j < RT * 4; ++j) x[j] = __builtin_amdgcn_exp2f(fmaf(sc[qg][j / 4][j % 4], s2, -mref));
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      // P^T slots 8g + j: items 32ps + 8g + j
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
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + col;
        u16x8 va[NS];
        lds_frag<TIn, NS>(vst + d * VROW, 4 * ps + g, keyv(d), va);
        st[qg].o[dt] = mfma_split<NS, NS>(va, pb, st[qg].o[dt]);
      }
      // the row sums of the same (rounded) weights: a row of ones times P^T
      st[qg].lsum = mfma_split<1, NS>(&ones, pb, st[qg].lsum);
    }
  }
}

template <typename TIn, typename TOut, int D, int WAVES, int QG, int MODE>
__global__ void __launch_bounds__(64 * WAVES) attn_kernel(Plan pl, AttnBufs b, int lev) {
  using SM = AtSmem<TIn, D, WAVES, QG>;
  using G = AtGeo<TIn, D>;
  constexpr int NS = sizeof(TIn) == 2 ? 1 : 3;
  constexpr int NT = 64 * WAVES, QT = 16 * QG * WAVES;
  constexpr int KS = D / 32, DT = D / 16;
  // small query clusters (one-wave workgroups) and the spatial-block groups,
  // whose retrieved (cluster, block) ranges hold a few keys each: tiles
  // gathered from 8-row chunks
  constexpr bool GATHER = (WAVES == 1 || MODE == MODE_V4) && MODE != MODE_LOCAL;
  // gathered tiles keep one stage (one-wave workgroups: twice as many fit per
  // CU, and the copy latency of one hides behind the others' work); four
  // waves with one query group keep two (four workgroups per CU)
  constexpr int ST = GATHER ? 1 : QG == 1 ? 2 : G::ST, PD = ST - 1;
  constexpr int LPT = (AT_KT * G::CHK + D * G::CHV) / NT;   // copies per thread per tile
  static_assert(PD * LPT <= 63, "copies in flight exceed the counter");
  __shared__ SM sm;
  __shared__ __attribute__((aligned(16))) unsigned char stg[ST][G::SB];   // tile stages [key rows | value columns]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ws = __builtin_amdgcn_readfirstlane(w);
  const int col = lane & 15, g = lane >> 4;
  const float s2 = pl.scale * LOG2E;
  const int C = pl.C;

  int bh, kvh, ap = 0, I = 0, tile, kp = 0, Ck = 0, q0 = 0, k0 = 0, vb = 0;
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
    // MODE_V4: problem t is query block t + 1 of a head; its query groups
    // are the query clusters' runs inside that block (q_perm positions
    // v4 qb[I][block] .. qb[I][block + 1])
    constexpr bool V4 = MODE == MODE_V4;
    const int nseg = V4 ? pl.nb - 1 : pl.lev_nseg[lev];
    const int m = V4 ? pl.blk : pl.lev_m[lev];
    const int Cqs = V4 ? min(pl.Cq, pl.N) : C;
    const int spp = (m + QT - 1) / QT + Cqs;
    // workgroups are dispatched round-robin over the 8 XCDs: keep every
    // problem on one XCD so its keys and values stay in that XCD's L2
    const int nprob = pl.B * pl.Hq * nseg;
    const int xcd = blockIdx.x % 8, loc = blockIdx.x / 8;
    const int slot = loc % spp;
    const int pid = (loc / spp) * 8 + xcd;
    if (pid >= nprob) return;
    const int t = pid % nseg;
    bh = pid / nseg;
    const int p = V4 ? 0 : pl.lev_pfirst[lev] + t;
    vb = t + 1;
    ap = bh * pl.P + p;
    const Geom gm = prob_geom(pl, p);
    const int Cq = V4 ? Cqs : min(C, gm.qn);
    Ck = V4 ? min(pl.Ck, pl.N) : min(C, gm.kn);
    k0 = gm.k0;
    q0 = gm.q0;
    // query group c of this problem: q_perm positions [qpos(c, 0), qpos(c, 1))
    const int32_t* qoffs = V4 ? b.qb + (size_t)bh * pl.Cq * (pl.nb + 1) + vb : b.qs.offs + (size_t)ap * (C + 1);
    const int qstr = V4 ? pl.nb + 1 : 1;
    auto qpos = [&](int c, int e) __attribute__((always_inline)) {
      return V4 ? qoffs[c * qstr + e] : qoffs[c + e];
    };
    if (tid < 64) {
      // every offset is read unconditionally (clusters past Cq read cluster
      // Cq - 1), so the reads are one round trip
      int lo[4], hi[4], v[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = max(min(tid * 4 + q, Cq - 1), 0);
        lo[q] = qpos(c, 0);
        hi[q] = qpos(c, 1);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = tid * 4 + q < Cq ? (hi[q] - lo[q] + QT - 1) / QT : 0;
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
          sm.sel[0] = tid * 4 + q;
          sm.sel[1] = slot - run;
          sm.sel[3] = lo[q];
          sm.sel[6] = hi[q];
        }
        run += v[q];
      }
      if (tid == 63) sm.sel[2] = inc;
    }
    __syncthreads();
    if (slot >= sm.sel[2]) return;
    // the selection is the workgroup's own (uniform)
    I = __builtin_amdgcn_readfirstlane(sm.sel[0]);
    tile = __builtin_amdgcn_readfirstlane(sm.sel[1]);
    qlo = __builtin_amdgcn_readfirstlane(sm.sel[3]) + tile * QT;
    qhi = min(__builtin_amdgcn_readfirstlane(sm.sel[6]), qlo + QT);
    const int bq = bh / pl.Hq, hq = bh % pl.Hq;
    kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
    kp = kvh * pl.P + p;
  }
  if (MODE == MODE_LOCAL) {
    const int bq = bh / pl.Hq, hq = bh % pl.Hq;
    kvh = bq * pl.Hkv + (hq * pl.Hkv) / pl.Hq;
  }
  const TIn* Qh = reinterpret_cast<const TIn*>(b.Q) + (size_t)bh * pl.N * D;

  // the workgroup's query rows, one per thread (QT <= NT).  The row list,
  // far-item and retrieved-cluster reads below are all issued before any of
  // them is used, every index kept in range, so they overlap in flight.
  static_assert(QT <= NT, "one query row per thread");
  int qrow_t;
  if (MODE == MODE_LOCAL) {
    qrow_t = qlo + tid < qhi ? qlo + tid : -1;
  } else {
    const int32_t* qperm = b.qs.perm + ((size_t)lev * pl.B * pl.Hq + bh) * pl.N + q0;
    const int v = qperm[min(qlo + tid, qhi - 1)];   // qlo < qhi
    qrow_t = qlo + tid < qhi ? v : -1;
  }
  const size_t esz = sizeof(TIn);
  TileSrc src;
  src.nv = b.Nv;
  src.kmax = pl.N - 1;
  src.Ck = 1;
  src.Cp = b.Cp32;
  src.mu = b.kst.mu_in;
  src.T = b.T;
  src.nfar = 0;
  if (MODE != MODE_LOCAL) {
    const int32_t* koffs = b.ks.offs + (size_t)kp * (C + 1);
    const int32_t* Rr = b.R + ((size_t)ap * C + I) * pl.k1w;
    // far items: log2 n_c (value T_Ic / n_c), or with the exact tilt the
    // bias log2 Z_Ic - s log2(e) nu_I.kappa_Ic (key row kappa_Ic, value U_Ic)
    constexpr bool V4 = MODE == MODE_V4;
    const bool xt = pl.dipole == 2;
    // MODE_V4: the far items of group (I, block vb), one per key cluster
    const size_t grp = V4 ? ((size_t)bh * pl.nb + vb) * pl.Cq + I : 0;
    const float* fbI = V4 ? b.fbias + grp * b.Cp32 : b.fb + ((size_t)ap * C + I) * b.Cp32;
    // far item c of this thread: c = tid + i NT
    constexpr int FBN = MUSE_MAXC / NT;
    float fbv[FBN];
    int kn0[FBN], kn1[FBN];
#pragma unroll
    for (int i = 0; i < FBN; ++i) {
      const int c = tid + i * NT;
      if (xt) {
        fbv[i] = fbI[max(min(c, Ck - 1), 0)];
        kn0[i] = kn1[i] = 0;
      } else {
        fbv[i] = 0.f;
        kn0[i] = koffs[min(c, Ck)];
        kn1[i] = koffs[min(c + 1, Ck)];
      }
    }
    int cc[4];
    if (tid < 64) {
      // compact the non-empty retrieved clusters into segments of absolute rows
      int lo[4], hi[4], v[4], sum = 0;
      if constexpr (V4) {
        // retrieved (cluster, block) pairs: entry r is block slot r % k2w of
        // retrieved cluster slot r / k2w
        const size_t g1 = (((size_t)bh * pl.Cq + I) * pl.nb + vb) * pl.k1w;
        const int nr = pl.k1w * pl.k2w;
        int c1[4], be[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = min(tid * 4 + q, nr - 1);
          c1[q] = b.r1[g1 + r / pl.k2w];
          be[q] = b.r2[g1 * pl.k2w + r];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = tid * 4 + q < nr && c1[q] >= 0 && be[q] >= 0;
          const int32_t* kbr = b.kb + ((size_t)kvh * pl.Ck + min(max(c1[q], 0), pl.Ck - 1)) * (pl.nb + 1) +
                               min(max(be[q], 0), pl.nb - 1);
          const int a = kbr[0], e = kbr[1];
          cc[q] = -1;   // retrieved clusters keep their far item (the rest of their keys)
          lo[q] = ok ? a : 0;
          hi[q] = ok ? e : 0;
        }
      } else {
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
          lo[q] = cc[q] >= 0 ? a : 0;
          hi[q] = cc[q] >= 0 ? e : 0;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = hi[q] > lo[q] ? 1 : 0;
        sum += v[q];
      }
      int inc = sum;
      for (int mm = 1; mm < 64; mm <<= 1) {
        const int o = __shfl_up(inc, mm, 64);
        if (tid >= mm) inc += o;
      }
      int run = inc - sum;
      int ntl = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (v[q]) {
          const int alo = k0 + lo[q], ahi = k0 + hi[q];
          sm.seg_lo[run] = alo;
          sm.seg_hi[run] = ahi;
          ntl += GATHER ? (ahi - (alo & ~7) + 7) >> 3                // 8-row chunks
                        : (ahi - (alo & ~7) + AT_KT - 1) / AT_KT;  // tiles
          ++run;
        }
      }
      // total exact tiles
      for (int mm = 32; mm >= 1; mm >>= 1) ntl += __shfl_xor(ntl, mm, 64);
      if (tid == 63) { sm.sel[4] = inc; sm.sel[5] = ntl; }   // inclusive total, and the all-reduced count
    }
#pragma unroll
    for (int i = 0; i < FBN; ++i) {
      const int c = tid + i * NT;
      float bias = -INFINITY;
      if (c < Ck) {
        const int nc = kn1[i] - kn0[i];
        bias = xt ? fbv[i] : nc > 0 ? __log2f((float)nc) : -INFINITY;
      }
      sm.far_bias[c] = bias / s2;   // the logit is s2 (score + bias / s2)
    }
    if (tid < QT) sm.qrow[tid] = qrow_t;
    __syncthreads();
    // retrieved clusters leave the far field
    if (tid < 64) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (cc[q] >= 0) sm.far_bias[cc[q]] = -INFINITY;
    }
    src.nseg = __builtin_amdgcn_readfirstlane(sm.sel[4]);
    src.nfar = (Ck + AT_KT - 1) / AT_KT;
    src.Ck = max(Ck, 1);
    if constexpr (V4) {
      src.mu = reinterpret_cast<const unsigned char*>(b.fk) + grp * b.Cp32 * D * esz;
      src.T = reinterpret_cast<const unsigned char*>(b.fv) + grp * D * b.Cp32 * esz;
    } else {
      src.mu = xt ? reinterpret_cast<const unsigned char*>(b.kap) + ((size_t)ap * C + I) * b.Cp32 * D * esz
                  : reinterpret_cast<const unsigned char*>(b.kst.mu_in) + (size_t)kp * C * D * esz;
      src.T = reinterpret_cast<const unsigned char*>(b.T) + ((size_t)ap * C + I) * D * b.Cp32 * esz;
    }
    const size_t slice = (size_t)lev * pl.B * pl.Hkv + kvh;
    src.Kx = reinterpret_cast<const unsigned char*>(b.kst.Kp) + slice * pl.N * D * esz;
    src.Vt = reinterpret_cast<const unsigned char*>(b.Vt) + slice * D * (size_t)b.Nv * esz;
  } else {
    // the block's keys up to its last query row
    if (tid == 0) {
      sm.seg_lo[0] = k0;
      sm.seg_hi[0] = qhi;
    }
    if (tid < QT) sm.qrow[tid] = qrow_t;
    src.nseg = 1;
    src.Kx = reinterpret_cast<const TIn*>(b.K) + (size_t)kvh * pl.N * D;
    const size_t slice = (size_t)pl.nlev * pl.B * pl.Hkv + kvh;   // input-order copy follows the levels
    src.Vt = reinterpret_cast<const unsigned char*>(b.Vt) + slice * D * (size_t)b.Nv * esz;
  }
  __syncthreads();
  // exact part: tiles (contiguous) or 8-row chunks, 8 to a tile (gathered)
  const int nex = MODE == MODE_LOCAL ? (qhi - (k0 & ~7) + AT_KT - 1) / AT_KT
                                     : __builtin_amdgcn_readfirstlane(sm.sel[5]);
  const int ntiles = (MODE == MODE_LOCAL ? 0 : src.nfar) + (GATHER ? (nex + 7) / 8 : nex);
  // one-wave bf16 workgroups at D = 64 list their exact chunks once (the
  // tile stage is free until the first copy)
  constexpr bool GXC = GATHER && WAVES == 1 && sizeof(TIn) == 2 && D == 64;
  GxTab gxt = {0, 0, 0, 0, 0u, {0u, 0u}};
  const bool gx = GXC && nex <= GX_MAXCH;
  if constexpr (GXC) {
    if (gx)
      gx_build(sm, src.nseg, nex, reinterpret_cast<int32_t*>(&stg[0][0]),
               reinterpret_cast<uint8_t*>(&stg[0][0]) + 4 * GX_MAXCH, gxt);
  }

  // ---- tile loop ----
  // two cursors: copies run PD tiles ahead of consumption.  Contiguous tiles
  // step through each cluster 64 rows at a time, gathered tiles 8 at a time.
  Cursor lc = cur_first(sm, src), cc = lc;
  TileOffs<TIn, D, WAVES> toffs;
  toffs.init(tid, src.nv, src.Cp);
  Chunks lgc = chunks_first(sm, src);
  TDesc gd;   // gathered tiles: the tile just issued (one stage: the next one consumed)
  auto issue_next = [&](unsigned char* dst) __attribute__((always_inline)) {
    if constexpr (GATHER) {
      if constexpr (GXC) {
        if (gx && lgc.t >= src.nfar) {
          // exact tile from the chunk table
          gd = gx_tile(gxt, lgc.t - src.nfar);
          ++lgc.t;
          int mx = gd.base[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) mx = max(mx, gd.base[k]);
          if (mx + 7 <= src.kmax) issue_tile_gx(dst, src, gd, gxt);
          else issue_tile_g<TIn, D, WAVES>(dst, src, gd);
          return;
        }
      }
      gd = take_tile(sm, src, lgc);
      // far tiles are 64 consecutive clusters: scalar bases when in range
      if (gd.far && gd.base[0] + AT_KT <= src.Ck && gd.base[0] + AT_KT <= src.Cp) {
        const size_t r0 = (size_t)gd.base[0] * sizeof(TIn);
        issue_tile_fast<TIn, D, WAVES>(dst, reinterpret_cast<const unsigned char*>(src.mu) + r0 * D,
                                       reinterpret_cast<const unsigned char*>(src.T) + r0, toffs.k, toffs.vf, ws);
      } else {
        issue_tile_g<TIn, D, WAVES>(dst, src, gd);
      }
    } else {
      // a tile whose rows and value columns all lie inside their arrays is
      // copied with scalar bases; tiles at an array's end clamp (issue_tile)
      const bool far = lc.t < src.nfar;
      const int kcap = far ? src.Ck - 1 : src.kmax;
      const int vstride = far ? src.Cp : src.nv;
      if (lc.row0 + AT_KT - 1 <= kcap && lc.row0 + AT_KT <= vstride) {
        const size_t r0 = (size_t)lc.row0 * sizeof(TIn);
        if (far)
          issue_tile_fast<TIn, D, WAVES>(dst, reinterpret_cast<const unsigned char*>(src.mu) + r0 * D,
                                         reinterpret_cast<const unsigned char*>(src.T) + r0, toffs.k, toffs.vf, ws);
        else
          issue_tile_fast<TIn, D, WAVES>(dst, reinterpret_cast<const unsigned char*>(src.Kx) + r0 * D,
                                         reinterpret_cast<const unsigned char*>(src.Vt) + r0, toffs.k, toffs.vx, ws);
      } else {
        issue_tile<TIn, D, WAVES>(dst, src, lc);
      }
      lc = cur_next(sm, src, lc);
    }
  };
  auto view_next = [&]() __attribute__((always_inline)) -> TileView {
    if constexpr (GATHER) {
      static_assert(!GATHER || PD == 0, "gathered tiles are consumed right after they are issued");
      return view_of(gd);
    } else {
      const TileView v = view_of<MODE == MODE_LOCAL>(src, cc, qlo);
      cc = cur_next(sm, src, cc);
      return v;
    }
  };
  // the first copies (one stage: the first tile) go out before the query
  // reads, so that their latencies overlap
  constexpr int P0 = PD == 0 ? 1 : PD;
#pragma unroll
  for (int p = 0; p < P0; ++p)
    if (p < ntiles) issue_next(stg[p]);
  // query fragments, and at causal levels with one query group at D = 64 the
  // row's fp32 partial that the result merges into (read now, not after the
  // last tile)
  constexpr bool PREF = MODE == MODE_LEVEL && D == 64 && QG == 1;
  int myq[QG];
  u16x8 qf[QG][KS][NS];
  AtState<D> st[QG];
  f32x4 opre[DT];
  float lpre = 0.f;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    myq[qg] = sm.qrow[(w * QG + qg) * 16 + col];
    // lanes without a query row load row 0; their outputs are not written
#pragma unroll
    for (int k = 0; k < KS; ++k)
      load8_split<TIn, NS>(Qh + (size_t)max(myq[qg], 0) * D + 32 * k + 8 * g, qf[qg][k]);
  }
  if constexpr (PREF) {
    const size_t r = (size_t)bh * pl.N + max(myq[0], 0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) opre[dt] = *reinterpret_cast<const f32x4*>(b.oacc + r * D + 16 * dt + 4 * g);
    lpre = b.lacc[r];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+v"(opre[dt]));
    asm volatile("" : "+v"(lpre));
  }
  // keep the fragments in registers (a read-only load could otherwise be
  // re-issued inside the tile loop)
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) asm volatile("" : "+v"(qf[qg][k][sp]));
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    st[qg].m = -1e30f;
    st[qg].lsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st[qg].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // A operand of the row sums: row 0 all ones, the other rows zero (lane l
  // holds row l % 16)
  u16x8 ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = col == 0 ? (uint16_t)0x3F80 : (uint16_t)0;
  int qmask[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) qmask[qg] = myq[qg] < 0 ? -1 : myq[qg];

  // query rows of the tile are a prefix; a wave whose rows all lie past it
  // (ragged query tiles) only copies and waits
  const int nrow = __builtin_amdgcn_readfirstlane(qhi - qlo);
  const bool wlive = 16 * QG * ws < nrow;

  int sl = PD % ST, sc_ = 0;   // stage of the next copy, stage being consumed
  for (int t = 0; t < ntiles; ++t) {
    // this thread's copies of tile t have landed (the PD-1 later tiles, when
    // they exist, may be in flight); after the barrier every thread's have,
    // and tile t-1 is consumed.  Only real tiles are copied.
    asm volatile("" ::: "memory");
    if constexpr (PD == 0) {
      // one stage: after every wave is done with tile t-1, copy tile t (tile
      // 0 went out before the query reads) and wait for it
      if (t > 0) {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue_next(stg[0]);
        asm volatile("" ::: "memory");
      }
      __builtin_amdgcn_s_waitcnt(at_wait(0, 0));
      __builtin_amdgcn_s_barrier();
    } else {
      if (t + PD - 1 < ntiles) __builtin_amdgcn_s_waitcnt(at_wait((PD - 1) * LPT, 0));
      else __builtin_amdgcn_s_waitcnt(at_wait(0, 0));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + PD < ntiles) issue_next(stg[sl]);
    }
    const TileView tv = view_next();
    if (wlive) consume_tile<TIn, D, WAVES, QG, MODE == MODE_LOCAL>(sm, stg[sc_], tv, qf, st, s2, qmask, ones);
    sl = sl + 1 == ST ? 0 : sl + 1;
    sc_ = sc_ + 1 == ST ? 0 : sc_ + 1;
  }
  // no copy into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(at_wait(0, 0));

  // ---- finish: normalise, write or merge (lse in natural log units) ----
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    // rows 1..15 of the row-sum tile are zero: lanes 16..63 and elements
    // 1..3 hold nothing, lane col element 0 holds the sum of query col
    float l = st[qg].lsum[0];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = myq[qg];
    if (row < 0) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse = l > 0.f ? (st[qg].m + __log2f(l)) * LN2 : -INFINITY;
    // the output row in the output dtype (16 dims per dt, 4 per lane)
    auto write_out = [&](const f32x4 (&v)[DT], float lse_out) __attribute__((always_inline)) {
      TOut* O = reinterpret_cast<TOut*>(b.O) + ((size_t)bh * pl.N + row) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if constexpr (sizeof(TOut) == 2) {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          u32x2 wv = {pk_bf16(v[dt][0], v[dt][1]), pk_bf16(v[dt][2], v[dt][3])};
          *reinterpret_cast<u32x2*>(O + 16 * dt + 4 * g) = wv;
        } else {
          *reinterpret_cast<f32x4*>(O + 16 * dt + 4 * g) = v[dt];
        }
      }
      if (g == 0) b.lse[(size_t)bh * pl.N + row] = lse_out;
    };
    f32x4 on[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) on[dt] = st[qg].o[dt] * inv;
    if (MODE == MODE_ACAUSAL) {
      write_out(on, lse);
    } else {
      // causal: partials of the local block and of each level a row belongs
      // to are merged in fp32; the last of them writes the output itself
      float* oa = b.oacc + ((size_t)bh * pl.N + row) * D;
      float* la = b.lacc + (size_t)bh * pl.N + row;
      const bool fin = last_level(pl, row) == (MODE == MODE_LOCAL ? -1 : lev);
      if (MODE == MODE_LOCAL) {
        if (fin) {
          write_out(on, lse);
        } else {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = on[dt];
          if (g == 0) *la = lse;
        }
      } else {
        if (!(l > 0.f) && !fin) continue;
        const float lold = PREF ? lpre : *la;
        float fo = 1.f, fn = 0.f, lnew = lold;
        if (l > 0.f) {
          const float L = fmaxf(lold, lse);
          const float wo = __expf(lold - L), wn = __expf(lse - L);
          const float tot = wo + wn;
          fo = wo / tot;
          fn = 1.f / tot;
          lnew = L + logf(tot);
          fn *= wn;
        }
        f32x4 mv[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          mv[dt] = (PREF ? opre[dt] : *reinterpret_cast<const f32x4*>(oa + 16 * dt + 4 * g)) * fo + on[dt] * fn;
        if (fin) {
          write_out(mv, lnew);
        } else {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(oa + 16 * dt + 4 * g) = mv[dt];
          if (g == 0) *la = lnew;
        }
      }
    }
  }
}

template <typename TIn, int D>
__global__ void __launch_bounds__(256) vt_kernel(Plan pl, const void* Vp, const void* V, void* Vt, int Nv,
                                                 int nsorted, int sfirst) {
  __shared__ TIn tile[VT_ROWS][D + 2];
  vt_block<TIn, D>(pl, Vp, V, Vt, Nv, nsorted, sfirst, (int)blockIdx.x, tile);
}

// ---------------------------------------------------------------------------
template <typename TIn, int D>
static hipError_t launch_vt(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  const VtGeo g = vt_geo(pl, b.Nv);
  const long long grid = (long long)g.nslice * g.nb;
  if (grid == 0) return hipSuccess;
  MUSE_KT_PRE(st);
  vt_kernel<TIn, D><<<(unsigned)grid, 256, 0, st>>>(pl, b.kst.Vp, b.V, b.Vt, b.Nv, g.nsorted, g.sfirst);
  MUSE_KT_POST("value_transpose", st);
  return hipGetLastError();
}

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
  static const char* const lname[8] = {"attn_level_L0", "attn_level_L1", "attn_level_L2", "attn_level_L3",
                                       "attn_level_L4", "attn_level_L5", "attn_level_L6", "attn_level_L7"};
  MUSE_KT_POST(pl.causal ? (lev < 8 ? lname[lev] : "attn_level") : "attn_far_retrieve", st);
  return hipGetLastError();
}

// Spatial blocks: one launch over the groups (query cluster, block) of
// every block after the first.
template <typename TIn, int D, int WAVES>
static hipError_t attn_v4(const Plan& pl, const AttnBufs& b, hipStream_t st) {
  constexpr int QT = 16 * WAVES;
  const int spp = (pl.blk + QT - 1) / QT + std::min(pl.Cq, pl.N);
  const long long nprob = (long long)pl.B * pl.Hq * (pl.nb - 1);
  const long long grid = ((nprob + 7) / 8) * 8 * spp;
  if (nprob <= 0) return hipSuccess;
  MUSE_KT_PRE(st);
  attn_kernel<TIn, TIn, D, WAVES, 1, MODE_V4><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, 0);
  MUSE_KT_POST("attn_v4", st);
  return hipGetLastError();
}

template <typename TIn, int D>
static hipError_t attn_all(const Plan& pl, const AttnBufs& b, bool vt_done, hipStream_t st) {
  hipError_t e = vt_done ? hipSuccess : launch_vt<TIn, D>(pl, b, st);
  if (e != hipSuccess) return e;
  // One group of 16 queries per wave, except at causal levels of query
  // clusters of 128 rows and more (bf16, D = 64): there two groups per wave,
  // which halve the LDS fragment reads per MFMA, measured 1 % faster at 64k
  // (at 8k, and at smaller clusters, the workgroups lost per CU to their
  // 200 VGPRs cost more than the reads save; 285 VGPRs at D = 128).
  if (pl.causal) {
    // local blocks: 128-row query tiles (two query groups per wave) for
    // bf16 at D = 64, else 64-row tiles
    constexpr int WAVES = 4, QGL = (sizeof(TIn) == 2 && D == 64) ? 2 : 1, QT = 16 * QGL * 4;
    const int nblk = (pl.N + pl.blk - 1) / pl.blk;
    const long long grid = (long long)pl.B * pl.Hq * nblk * ((pl.blk + QT - 1) / QT);
    MUSE_KT_PRE(st);
    attn_kernel<TIn, TIn, D, WAVES, QGL, MODE_LOCAL><<<(unsigned)grid, 64 * WAVES, 0, st>>>(pl, b, 0);
    MUSE_KT_POST("attn_local", st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pl.v4) {
    const int avg = pl.blk / std::max(1, std::min(pl.Cq, pl.N));
    if (avg >= 48) return attn_v4<TIn, D, 4>(pl, b, st);
    if constexpr (sizeof(TIn) == 2 || D == 64) return attn_v4<TIn, D, 1>(pl, b, st);
    return attn_v4<TIn, D, 4>(pl, b, st);
  }
  for (int lev = 0; lev < pl.nlev; ++lev) {
    // query clusters of ~m/C rows: the query tile (rows per workgroup) follows
    // the mean cluster size so that ragged clusters waste few tile rows
    const int avg = pl.lev_m[lev] / (pl.C > 0 ? pl.C : 1);
    if (sizeof(TIn) == 2 && D == 64 && pl.causal && avg >= 128) e = attn_level<TIn, D, 4, 2>(pl, b, lev, st);
    else if (avg >= 48) e = attn_level<TIn, D, 4, 1>(pl, b, lev, st);
    else if constexpr (sizeof(TIn) == 2 || D == 64) e = attn_level<TIn, D, 1, 1>(pl, b, lev, st);
    else e = attn_level<TIn, D, 4, 1>(pl, b, lev, st);   // one wave could not keep a tile's copies counted
    if (e != hipSuccess) return e;
  }
  return e;
}

hipError_t launch_attn(const Plan& pl, int dtype, const AttnBufs& b, bool vt_done, hipStream_t st) {
  if (dtype == 1)
    return pl.D == 64 ? attn_all<uint16_t, 64>(pl, b, vt_done, st) : attn_all<uint16_t, 128>(pl, b, vt_done, st);
  return pl.D == 64 ? attn_all<float, 64>(pl, b, vt_done, st) : attn_all<float, 128>(pl, b, vt_done, st);
}

}  // namespace muse
