// Host engine behind the C ABI of include/muse.h: argument checks, the
// problem plan of a call, the state/workspace layout and the launch order
// on the caller's stream.  Nothing here allocates device memory or
// synchronises (except muse_timing_collect, which waits for its events).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/muse.h"
#include "common.h"
#include "launch.h"

namespace muse {

hipError_t launch_perm_only(const Plan& pl, const CSet& s0, hipStream_t st);

// Problems whose point count is at most this run all Lloyd iterations in one
// workgroup; larger ones are split into chunks with one launch per iteration.
static const int KM_LOCAL_MAX = 2048;

int g_ktime_on = 0;
namespace {
struct KtRec {
  hipEvent_t a, b;
  const char* name;
};
std::vector<hipEvent_t> g_pool;
std::vector<KtRec> g_pending;
hipEvent_t g_pre = nullptr;
struct KtTot {
  std::string name;
  double ms;
  int64_t n;
};
std::vector<KtTot> g_tot;
std::string g_hip_err;

hipEvent_t ev_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void ktime_pre(hipStream_t st) {
  g_pre = ev_get();
  if (g_pre) (void)hipEventRecord(g_pre, st);
}
void ktime_post(const char* name, hipStream_t st) {
  hipEvent_t e = ev_get();
  if (!e || !g_pre) return;
  (void)hipEventRecord(e, st);
  g_pending.push_back({g_pre, e, name});
  g_pre = nullptr;
}

void set_smem_once(const void* fn, size_t bytes) {
  static std::unordered_set<const void*> done;
  if (done.count(fn)) return;
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  done.insert(fn);
}

// ---------------------------------------------------------------------------
static int build_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, const muse_cfg* cfg,
                      Plan& pl) {
  memset(&pl, 0, sizeof(pl));
  if (!cfg) return MUSE_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || (D != 64 && D != 128)) return MUSE_EINVAL;
  if (Hq % Hkv != 0) return MUSE_EINVAL;
  if (cfg->cq < 1 || cfg->cq > MUSE_MAX_CLUSTERS || cfg->ck < 1 || cfg->ck > MUSE_MAX_CLUSTERS)
    return MUSE_EINVAL;
  if (cfg->iters < 1 || cfg->topk < 0) return MUSE_EINVAL;
  if (cfg->causal < 0 || cfg->causal > 2) return MUSE_EINVAL;
  if (cfg->init_mode != 0 && cfg->init_mode != 1) return MUSE_EINVAL;
  if (cfg->dipole < 0 || cfg->dipole > 2) return MUSE_EINVAL;
  if (cfg->causal && cfg->block < 1) return MUSE_EINVAL;
  if (B * Hq * N * D >= (int64_t)1 << 40 || N >= ((int64_t)1 << 30)) return MUSE_EUNSUPPORTED;
  pl.B = (int)B; pl.Hq = (int)Hq; pl.Hkv = (int)Hkv; pl.N = (int)N; pl.D = (int)D;
  pl.Cq = cfg->cq;
  pl.Ck = cfg->ck;
  pl.C = std::max(cfg->cq, cfg->ck);
  pl.iters = cfg->iters;
  pl.topk = cfg->topk;
  pl.k1w = std::max(1, std::min(cfg->topk, cfg->ck));
  pl.dipole = cfg->dipole;
  pl.warm = cfg->init_mode;
  pl.causal = cfg->causal ? 1 : 0;
  pl.blk = cfg->causal ? cfg->block : 0;
  pl.scale = cfg->scale > 0.f ? cfg->scale : (float)(1.0 / sqrt((double)D));
  if (cfg->causal == 2) {
    // spatial blocks with accumulated summaries: one clustering problem per
    // head over all rows (the acausal geometry), exact local blocks, and one
    // pass over the groups (query cluster, block) for everything earlier
    if (cfg->dipole != 2) return MUSE_EUNSUPPORTED;
    if (cfg->topk2 < 0 || (cfg->topk > 0 && cfg->topk2 < 1)) return MUSE_EINVAL;
    const int64_t nb = (N + pl.blk - 1) / pl.blk;
    if (nb > 4096) return MUSE_EUNSUPPORTED;
    pl.v4 = 1;
    pl.nb = (int)nb;
    pl.topk2 = cfg->topk2;
    pl.k2w = (int)std::max<int64_t>(1, std::min<int64_t>(cfg->topk2, nb));
    if (pl.k1w * pl.k2w > MUSE_MAXC) return MUSE_EUNSUPPORTED;
    pl.nlev = 1;
    pl.lev_m[0] = (int)N;
    pl.lev_nseg[0] = 1;
    pl.lev_pfirst[0] = 0;
    pl.lev_pfirst[1] = 1;
    pl.P = 1;
    return MUSE_OK;
  }
  if (!pl.causal) {
    pl.nlev = 1;
    pl.lev_m[0] = (int)N;
    pl.lev_nseg[0] = 1;
    pl.lev_pfirst[0] = 0;
    pl.lev_pfirst[1] = 1;
    pl.P = 1;
    return MUSE_OK;
  }
  const int64_t nb = (N + pl.blk - 1) / pl.blk;
  int L = 0;
  while (((int64_t)1 << L) < nb) ++L;
  if (L > MUSE_MAXLEV) return MUSE_EUNSUPPORTED;
  pl.nlev = L;
  int P = 0;
  for (int l = 0; l < L; ++l) {
    const int64_t m = (int64_t)pl.blk << l;
    const int64_t nseg = N > m ? (N - m + 2 * m - 1) / (2 * m) : 0;
    pl.lev_m[l] = (int)m;
    pl.lev_nseg[l] = (int)nseg;
    pl.lev_pfirst[l] = P;
    P += (int)nseg;
  }
  pl.lev_pfirst[L] = P;
  pl.P = P;
  return MUSE_OK;
}

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// the kernels move tensor rows, state and workspace with 16-byte vector accesses
static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Layout {
  muse_layout L;
  int plocal;
  KmLarge lg;
};

static void build_kmlarge(const Plan& pl, int heads_total, int dtype, int& plocal, KmLarge& lg) {
  memset(&lg, 0, sizeof(lg));
  plocal = 0;
  const int sub = kmeans_sub(dtype, pl.D);
  int first_large = pl.nlev;
  for (int l = 0; l < pl.nlev; ++l) {
    if (pl.lev_m[l] > KM_LOCAL_MAX) { first_large = l; break; }
    plocal += pl.lev_nseg[l];
  }
  int64_t pts = 0;
  for (int l = first_large; l < pl.nlev; ++l) pts += (int64_t)heads_total * pl.lev_nseg[l] * pl.lev_m[l];
  // points per chunk: at least two sub-tiles (fewer partial sums to reduce),
  // smaller while that leaves fewer than 1024 chunks
  int ch = 2048;
  while (ch > 2 * sub && pts / ch < 1024) ch /= 2;
  lg.ch = ch;
  const int ncb = (pl.C + 256 / pl.D - 1) / (256 / pl.D);   // reduce workgroups per problem
  int nl = 0, cf = 0, pf = 0, wf = 0, rf = 0;
  for (int l = first_large; l < pl.nlev; ++l) {
    if (pl.lev_nseg[l] == 0) continue;
    lg.lev[nl] = l;
    lg.nch[nl] = (pl.lev_m[l] + ch - 1) / ch;
    lg.cfirst[nl] = cf;
    lg.pfirst[nl] = pf;
    lg.wfirst[nl] = wf;
    lg.rfirst[nl] = rf;
    const int np = heads_total * pl.lev_nseg[l];
    cf += np * lg.nch[nl];
    pf += np;
    wf += (np + 7) / 8 * 8 * lg.nch[nl];
    rf += (np + 7) / 8 * 8 * ncb;
    ++nl;
  }
  lg.nl = nl;
  lg.cfirst[nl] = cf;
  lg.pfirst[nl] = pf;
  lg.wfirst[nl] = wf;
  lg.rfirst[nl] = rf;
}

// k-means scratch: chunk partial sums and counts.
static void km_ws_bytes(const KmLarge& lg, int C, int D, size_t& part, size_t& pcnt) {
  part = al((size_t)lg.cfirst[lg.nl] * C * D * 4);
  pcnt = al((size_t)lg.cfirst[lg.nl] * C * 4);
}

static void build_layout(const Plan& pl, int dtype, Layout& out) {
  muse_layout& L = out.L;
  memset(&L, 0, sizeof(L));
  const size_t BHq = (size_t)pl.B * pl.Hq, BHk = (size_t)pl.B * pl.Hkv;
  const size_t N = pl.N, D = pl.D, C = pl.C, P = pl.P, nl = pl.nlev;
  L.P = pl.P;
  L.L = pl.nlev;
  L.C = pl.C;
  L.k1w = pl.k1w;
  L.Cp32 = (pl.C + 63) / 64 * 64;   // T rows padded to whole 64-cluster tiles
  L.Nv = (pl.N + 7) / 8 * 8;         // value-column rows padded to whole 16-byte chunks
  size_t o = 0;
  L.q_labels = o; o = al(o + nl * BHq * N * 4);
  L.k_labels = o; o = al(o + nl * BHk * N * 4);
  L.q_perm = o; o = al(o + nl * BHq * N * 4);
  L.k_perm = o; o = al(o + nl * BHk * N * 4);
  L.q_offs = o; o = al(o + BHq * P * (C + 1) * 4);
  L.k_offs = o; o = al(o + BHk * P * (C + 1) * 4);
  L.q_cent = o; o = al(o + BHq * P * C * D * 4);
  L.k_cent = o; o = al(o + BHk * P * C * D * 4);
  L.mu = o; o = al(o + BHk * P * C * D * 4);
  L.S = o; o = al(o + BHk * P * C * D * 4);
  L.M = o; o = al(o + BHk * P * D * C * D * 4);
  L.R = o; o = al(o + BHq * P * C * pl.k1w * 4);
  const size_t eb = dtype == 1 ? 2 : 4;
  L.Kp = o; o = al(o + nl * BHk * N * D * eb);
  L.Vp = o; o = al(o + nl * BHk * N * D * eb);
  L.mu_in = o; o = al(o + BHk * P * C * D * eb);
  // spatial-block scheme: retrieval of every group and block bounds
  const size_t nb = pl.v4 ? pl.nb : 0, Cq = pl.Cq, Ck = pl.Ck;
  L.nb = (int64_t)nb;
  L.k2w = pl.v4 ? pl.k2w : 0;
  L.v4_R1 = o; o = al(o + BHq * Cq * nb * pl.k1w * 4);
  L.v4_R2 = o; o = al(o + BHq * Cq * nb * pl.k1w * (size_t)L.k2w * 4);
  L.v4_kb = o; o = al(o + (pl.v4 ? BHk * Ck * (nb + 1) * 4 : 0));
  L.v4_qb = o; o = al(o + (pl.v4 ? BHq * Cq * (nb + 1) * 4 : 0));
  L.state_bytes = std::max<size_t>(o, 256);
  build_kmlarge(pl, (int)(BHq + BHk), dtype, out.plocal, out.lg);
  size_t w = 0;
  L.ws_T = w; w = al(w + (pl.v4 ? 0 : BHq * P * C * D * L.Cp32 * eb));
  L.ws_oacc = w; w = al(w + (pl.causal ? BHq * N * D * 4 : 0));
  L.ws_lacc = w; w = al(w + (pl.causal ? BHq * N * 4 : 0));
  L.ws_Vt = w; w = al(w + (nl + (pl.causal ? 1 : 0)) * BHk * D * (size_t)L.Nv * eb);
  size_t kp_bytes, kc_bytes;
  km_ws_bytes(out.lg, pl.C, pl.D, kp_bytes, kc_bytes);
  L.ws_part = w; w = al(w + kp_bytes);
  L.ws_pcnt = w; w = al(w + kc_bytes);
  // exact tilt: tilted key centroids per (I, c) and the two per-pair floats
  const bool xt = pl.dipole == 2 && !pl.v4;
  L.ws_kap = w; w = al(w + (xt ? BHq * P * C * L.Cp32 * D * eb : 0));
  L.ws_lz = w; w = al(w + (xt ? BHq * P * C * L.Cp32 * 4 : 0));
  L.ws_fb = w; w = al(w + (xt ? BHq * P * C * L.Cp32 * 4 : 0));
  L.ws_v4pz = w; w = al(w + BHq * Cq * Ck * nb * 4);
  L.ws_v4pk = w; w = al(w + BHq * Cq * Ck * nb * D * 4);
  L.ws_v4pu = w; w = al(w + BHq * Cq * Ck * nb * D * 4);
  L.ws_v4kap = w; w = al(w + BHq * nb * Cq * L.Cp32 * D * eb);
  L.ws_v4T = w; w = al(w + BHq * nb * Cq * D * L.Cp32 * eb);
  L.ws_v4fb = w; w = al(w + BHq * nb * Cq * L.Cp32 * 4);
  L.ws_bytes = std::max<size_t>(w, 256);
}

// Backward scratch: recomputed T, Delta, fp32 gradient accumulators and the
// per-level cluster gradients (sized for the level with the most segments).
struct BwdLayout {
  size_t T, delta, dq, dk, dv, dT, G, dnu, dS, dmu, dM, bytes;
};

static void build_bwd_layout(const Plan& pl, int dtype, BwdLayout& o) {
  const size_t BHq = (size_t)pl.B * pl.Hq, BHk = (size_t)pl.B * pl.Hkv;
  const size_t N = pl.N, D = pl.D, C = pl.C, P = pl.P;
  const size_t Cp = (pl.C + 63) / 64 * 64;
  const size_t eb = dtype == 1 ? 2 : 4;
  size_t ms = 0;
  for (int l = 0; l < pl.nlev; ++l) ms = std::max<size_t>(ms, (size_t)pl.lev_nseg[l]);
  size_t w = 0;
  o.T = w; w = al(w + BHq * P * C * D * Cp * eb);
  o.delta = w; w = al(w + BHq * N * 4);
  o.dq = w; w = al(w + BHq * N * D * 4);
  o.dk = w; w = al(w + BHk * N * D * 4);
  o.dv = w; w = al(w + BHk * N * D * 4);
  o.dT = w; w = al(w + BHq * ms * C * D * C * eb);
  o.G = w; w = al(w + BHq * ms * C * C * D * 4);
  o.dnu = w; w = al(w + BHq * ms * C * D * 4);
  o.dS = w; w = al(w + BHk * ms * C * D * 4);
  o.dmu = w; w = al(w + BHk * ms * C * D * 4);
  o.dM = w; w = al(w + BHk * ms * D * C * D * 4);
  o.bytes = std::max<size_t>(w, 256);
}

static int hip_fail(hipError_t e) {
  g_hip_err = hipGetErrorString(e);
  return MUSE_EHIP;
}

// Forward workspace for callers that cannot allocate (museattn_fwd_noalloc):
// one array per GPU, held until the process ends.  In host code the name
// `scratch` is only a host-side stand-in; kernels and copies take the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MUSE_NOALLOC_WS_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // indexed by HIP device ordinal
}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!p) return MUSE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUSE_OK;
}

}  // namespace muse

using namespace muse;

extern "C" {

const char* muse_strerror(int code) {
  switch (code) {
    case MUSE_OK: return "success";
    case MUSE_EINVAL: return "invalid argument (shape, dtype, pointer or parameter)";
    case MUSE_EWORKSPACE: return "workspace or state buffer too small";
    case MUSE_EUNSUPPORTED: return "unsupported request";
    case MUSE_EHIP: return "HIP launch or runtime error";
    default: return "unknown error";
  }
}

const char* muse_last_hip_error(void) { return g_hip_err.c_str(); }

int muse_plan(int64_t N, const muse_cfg* cfg, int32_t* out, int64_t cap, int64_t* count) {
  if (!count) return MUSE_EINVAL;
  Plan pl;
  int rc = build_plan(1, 1, 1, N, 64, cfg, pl);
  if (rc) return rc;
  *count = pl.P;
  for (int p = 0; p < pl.P && p < cap; ++p) {
    if (!out) return MUSE_EINVAL;
    Geom g = prob_geom(pl, p);
    int32_t* r = out + 6 * (size_t)p;
    r[0] = g.lev;
    r[1] = p - pl.lev_pfirst[g.lev];
    r[2] = g.k0; r[3] = g.kn; r[4] = g.q0; r[5] = g.qn;
  }
  return MUSE_OK;
}

int muse_layout_query(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, muse_dtype dtype,
                      const muse_cfg* cfg, muse_layout* out) {
  if (!out || (dtype != MUSE_F32 && dtype != MUSE_BF16)) return MUSE_EINVAL;
  Plan pl;
  int rc = build_plan(B, Hq, Hkv, N, D, cfg, pl);
  if (rc) return rc;
  Layout lay;
  build_layout(pl, (int)dtype, lay);
  *out = lay.L;
  return MUSE_OK;
}

int museattn_fwd(const void* Q, const void* K, const void* V, muse_dtype dtype, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t N, int64_t D, const muse_cfg* cfg, const int32_t* init_q,
                 const int32_t* init_k, void* O, float* lse, void* state, size_t state_bytes,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!Q || !K || !V || !O || !lse || !state || !ws) return MUSE_EINVAL;
  if (!al16(Q) || !al16(K) || !al16(V) || !al16(O) || !al16(state) || !al16(ws)) return MUSE_EINVAL;
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_EINVAL;
  Plan pl;
  int rc = build_plan(B, Hq, Hkv, N, D, cfg, pl);
  if (rc) return rc;
  Layout lay;
  build_layout(pl, (int)dtype, lay);
  const muse_layout& L = lay.L;
  if (state_bytes < L.state_bytes || ws_bytes < L.ws_bytes) return MUSE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* sb = (char*)state;
  char* wb = (char*)ws;
  CSet qs{Q, pl.B * pl.Hq, 1, init_q, (int32_t*)(sb + L.q_labels), (int32_t*)(sb + L.q_perm),
          (int32_t*)(sb + L.q_offs), (float*)(sb + L.q_cent), pl.Cq};
  CSet ks{K, pl.B * pl.Hkv, 0, init_k, (int32_t*)(sb + L.k_labels), (int32_t*)(sb + L.k_perm),
          (int32_t*)(sb + L.k_offs), (float*)(sb + L.k_cent), pl.Ck};
  AttnBufs ab;
  memset(&ab, 0, sizeof(ab));
  ab.Q = Q; ab.K = K; ab.V = V;
  ab.qs = qs; ab.ks = ks;
  ab.kst = KStats{(float*)(sb + L.mu), (float*)(sb + L.S), (float*)(sb + L.M), sb + L.mu_in,
                  sb + L.Kp, sb + L.Vp};
  ab.R = (int32_t*)(sb + L.R);
  ab.T = wb + L.ws_T;
  ab.Cp32 = (int32_t)L.Cp32;
  ab.oacc = (float*)(wb + L.ws_oacc);
  ab.lacc = (float*)(wb + L.ws_lacc);
  ab.Vt = wb + L.ws_Vt;
  ab.Nv = (int32_t)L.Nv;
  ab.O = O;
  ab.lse = lse;
  ab.kap = wb + L.ws_kap;
  ab.lz = (float*)(wb + L.ws_lz);
  ab.fb = (float*)(wb + L.ws_fb);
  ab.r1 = (int32_t*)(sb + L.v4_R1);
  ab.r2 = (int32_t*)(sb + L.v4_R2);
  ab.kb = (int32_t*)(sb + L.v4_kb);
  ab.qb = (int32_t*)(sb + L.v4_qb);
  ab.pz = (float*)(wb + L.ws_v4pz);
  ab.pk = (float*)(wb + L.ws_v4pk);
  ab.pu = (float*)(wb + L.ws_v4pu);
  ab.fk = wb + L.ws_v4kap;
  ab.fv = wb + L.ws_v4T;
  ab.fbias = (float*)(wb + L.ws_v4fb);
  hipError_t e = hipGetLastError();  // clear stale errors from earlier calls
  (void)e;
  bool vt_done = false;   // the value copies built with the scores
  if (pl.P > 0) {
    if ((e = launch_kmeans(pl, (int)dtype, qs, ks, lay.plocal, lay.lg, (float*)(wb + L.ws_part),
                           (int32_t*)(wb + L.ws_pcnt), st)) != hipSuccess)
      return hip_fail(e);
    if ((e = launch_summarize(pl, (int)dtype, ks, V, ab.kst, st)) != hipSuccess) return hip_fail(e);
    if (pl.v4) {
      if ((e = launch_v4(pl, (int)dtype, ab, st)) != hipSuccess) return hip_fail(e);
    } else if (pl.dipole == 2) {
      if ((e = launch_tilt_exact(pl, (int)dtype, ab, st)) != hipSuccess) return hip_fail(e);
    } else if ((e = launch_score_tilt(pl, (int)dtype, ab, vt_done, st)) != hipSuccess) {
      return hip_fail(e);
    }
  }
  if ((e = launch_attn(pl, (int)dtype, ab, vt_done, st)) != hipSuccess) return hip_fail(e);
  return MUSE_OK;
}

int museattn_fwd_noalloc(const void* Q, const void* K, const void* V, muse_dtype dtype, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t N, int64_t D, const muse_cfg* cfg,
                         const int32_t* init_q, const int32_t* init_k, void* O, float* lse, void* state,
                         size_t state_bytes, void* stream) {
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_EINVAL;
  Plan pl;
  int rc = build_plan(B, Hq, Hkv, N, D, cfg, pl);
  if (rc) return rc;
  Layout lay;
  build_layout(pl, (int)dtype, lay);
  if (lay.L.ws_bytes > (size_t)MUSE_NOALLOC_WS_BYTES) return MUSE_EWORKSPACE;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != MUSE_OK) return rc;
  return museattn_fwd(Q, K, V, dtype, B, Hq, Hkv, N, D, cfg, init_q, init_k, O, lse, state, state_bytes, ws,
                      (size_t)MUSE_NOALLOC_WS_BYTES, stream);
}

size_t muse_cluster_ws_size(int64_t G, int64_t n, int64_t D, muse_dtype dtype, int32_t C) {
  muse_cfg cfg{C, C, 1, 0, 0, 0, 1, 0, 0.f};
  Plan pl;
  if (build_plan(1, G, G, n, D, &cfg, pl)) return 0;
  int plocal;
  KmLarge lg;
  build_kmlarge(pl, (int)G, (int)dtype, plocal, lg);
  size_t a, b;
  km_ws_bytes(lg, C, (int)D, a, b);
  return a + b + 256;
}

int musecluster(const void* X, muse_dtype dtype, int64_t G, int64_t n, int64_t D, int32_t C,
                int32_t iters, const int32_t* init_idx, int32_t* assign, float* centroids,
                int32_t* perm, int32_t* offs, void* ws, size_t ws_bytes, void* stream) {
  if (!X || !assign || !centroids || !perm || !offs) return MUSE_EINVAL;
  if (!al16(X) || !al16(centroids) || (ws && !al16(ws))) return MUSE_EINVAL;
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_EINVAL;
  muse_cfg cfg{C, C, iters, 0, 0, 0, 1, 0, 0.f};
  Plan pl;
  int rc = build_plan(1, G, G, n, D, &cfg, pl);
  if (rc) return rc;
  int plocal;
  KmLarge lg;
  build_kmlarge(pl, (int)G, (int)dtype, plocal, lg);
  const size_t need = muse_cluster_ws_size(G, n, D, dtype, C);
  if (lg.nl > 0 && (!ws || ws_bytes < need)) return MUSE_EWORKSPACE;
  CSet s0{X, (int)G, 1, init_idx, assign, perm, offs, centroids, C};
  CSet s1{nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, C};
  size_t kp_bytes, kc_bytes;
  km_ws_bytes(lg, C, (int)D, kp_bytes, kc_bytes);
  float* part = (float*)ws;
  int32_t* pcnt = ws ? (int32_t*)((char*)ws + kp_bytes) : nullptr;
  (void)hipGetLastError();
  hipError_t e = launch_kmeans(pl, (int)dtype, s0, s1, plocal, lg, part, pcnt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return MUSE_OK;
}

int musesummarize(const void* K, const void* V, muse_dtype dtype, int64_t G, int64_t n, int64_t D,
                  int32_t C, const int32_t* assign, int32_t* perm, int32_t* offs, float* mu,
                  float* S, float* M, void* stream) {
  if (!K || !V || !assign || !perm || !offs || !mu || !S || !M) return MUSE_EINVAL;
  if (!al16(K) || !al16(V)) return MUSE_EINVAL;
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_EINVAL;
  muse_cfg cfg{C, C, 1, 0, 0, 0, 1, 0, 0.f};
  Plan pl;
  int rc = build_plan(1, G, G, n, D, &cfg, pl);
  if (rc) return rc;
  CSet ks{K, (int)G, 0, nullptr, const_cast<int32_t*>(assign), perm, offs, nullptr, C};
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipError_t e = launch_perm_only(pl, ks, st);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_summarize(pl, (int)dtype, ks, V, KStats{mu, S, M, nullptr, nullptr, nullptr}, st);
  if (e != hipSuccess) return hip_fail(e);
  return MUSE_OK;
}

size_t muse_bwd_ws_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, muse_dtype dtype,
                        const muse_cfg* cfg) {
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return 0;
  Plan pl;
  if (build_plan(B, Hq, Hkv, N, D, cfg, pl)) return 0;
  BwdLayout bl;
  build_bwd_layout(pl, (int)dtype, bl);
  return bl.bytes;
}

int museattn_bwd(const void* Q, const void* K, const void* V, const void* O, const float* lse,
                 const void* dO, muse_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                 int64_t D, const muse_cfg* cfg, const void* state, size_t state_bytes, void* dQ,
                 void* dK, void* dV, void* ws, size_t ws_bytes, void* stream) {
  if (!Q || !K || !V || !O || !lse || !dO || !state || !dQ || !dK || !dV || !ws) return MUSE_EINVAL;
  const void* vec[] = {Q, K, V, O, dO, dQ, dK, dV, state, ws};
  for (const void* p : vec)
    if (!al16(p)) return MUSE_EINVAL;
  if (dtype != MUSE_F32 && dtype != MUSE_BF16) return MUSE_EINVAL;
  Plan pl;
  int rc = build_plan(B, Hq, Hkv, N, D, cfg, pl);
  if (rc) return rc;
  if (pl.dipole == 2) return MUSE_EUNSUPPORTED;   // the exact tilt has no backward here
  // the item-centric pass indexes query rows of all heads with 32-bit integers
  if ((int64_t)pl.B * pl.Hq * pl.N >= ((int64_t)1 << 31)) return MUSE_EUNSUPPORTED;
  Layout lay;
  build_layout(pl, (int)dtype, lay);
  const muse_layout& L = lay.L;
  BwdLayout bl;
  build_bwd_layout(pl, (int)dtype, bl);
  if (state_bytes < L.state_bytes || ws_bytes < bl.bytes) return MUSE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* sb = (char*)const_cast<void*>(state);
  char* wb = (char*)ws;
  AttnBufs ab;
  memset(&ab, 0, sizeof(ab));
  ab.Q = Q; ab.K = K; ab.V = V;
  ab.qs = CSet{Q, pl.B * pl.Hq, 1, nullptr, (int32_t*)(sb + L.q_labels), (int32_t*)(sb + L.q_perm),
               (int32_t*)(sb + L.q_offs), (float*)(sb + L.q_cent), pl.Cq};
  ab.ks = CSet{K, pl.B * pl.Hkv, 0, nullptr, (int32_t*)(sb + L.k_labels), (int32_t*)(sb + L.k_perm),
               (int32_t*)(sb + L.k_offs), (float*)(sb + L.k_cent), pl.Ck};
  ab.kst = KStats{(float*)(sb + L.mu), (float*)(sb + L.S), (float*)(sb + L.M), sb + L.mu_in,
                  sb + L.Kp, sb + L.Vp};
  ab.R = (int32_t*)(sb + L.R);
  ab.T = wb + bl.T;
  ab.Cp32 = (int32_t)L.Cp32;
  ab.O = const_cast<void*>(O);
  ab.lse = const_cast<float*>(lse);
  hipError_t e = hipGetLastError();  // clear stale errors from earlier calls
  (void)e;
  if (pl.P > 0 && (e = launch_tilt(pl, (int)dtype, ab, st)) != hipSuccess) return hip_fail(e);
  BwdLaunch bw;
  bw.pl = pl;
  bw.dtype = (int)dtype;
  bw.a = ab;
  bw.dO = dO;
  bw.lse = lse;
  bw.delta = (float*)(wb + bl.delta);
  bw.dq = (float*)(wb + bl.dq);
  bw.dk = (float*)(wb + bl.dk);
  bw.dv = (float*)(wb + bl.dv);
  bw.dT = (void*)(wb + bl.dT);
  bw.G = (float*)(wb + bl.G);
  bw.dnu = (float*)(wb + bl.dnu);
  bw.dS = (float*)(wb + bl.dS);
  bw.dmu = (float*)(wb + bl.dmu);
  bw.dM = (float*)(wb + bl.dM);
  bw.dQ = dQ; bw.dK = dK; bw.dV = dV;
  if ((e = launch_bwd(bw, st)) != hipSuccess) return hip_fail(e);
  return MUSE_OK;
}

int muse_timing_enable(int on) {
  g_ktime_on = on ? 1 : 0;
  return MUSE_OK;
}

int muse_timing_collect(void) {
  for (auto& r : g_pending) {
    (void)hipEventSynchronize(r.b);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, r.a, r.b);
    auto it = std::find_if(g_tot.begin(), g_tot.end(), [&](const KtTot& t) { return t.name == r.name; });
    if (it == g_tot.end()) g_tot.push_back({r.name, (double)ms, 1});
    else { it->ms += ms; it->n += 1; }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_pending.clear();
  return MUSE_OK;
}

int muse_timing_reset(void) {
  muse_timing_collect();
  g_tot.clear();
  return MUSE_OK;
}

int muse_timing_get(int i, const char** name, double* total_ms, int64_t* launches) {
  if (i < 0 || i >= (int)g_tot.size()) return MUSE_EINVAL;
  if (name) *name = g_tot[i].name.c_str();
  if (total_ms) *total_ms = g_tot[i].ms;
  if (launches) *launches = g_tot[i].n;
  return MUSE_OK;
}

}  // extern "C"
