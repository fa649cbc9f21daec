// Internal launch interface between the host engine and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "common.h"

namespace muse {

// Large k-means problems: the levels whose span exceeds the in-workgroup
// limit, each split into chunks of `ch` points (one workgroup per chunk).
struct KmLarge {
  int32_t nl;                       // number of large levels
  int32_t ch;                       // points per chunk
  int32_t lev[MUSE_MAXLEV];         // plan level of each entry
  int32_t nch[MUSE_MAXLEV];         // chunks per problem
  int32_t cfirst[MUSE_MAXLEV + 1];  // first chunk of each entry (both sets)
  int32_t wfirst[MUSE_MAXLEV + 1];  // first workgroup of each entry (XCD-padded)
  int32_t rfirst[MUSE_MAXLEV + 1];  // first reduce workgroup of each entry (XCD-padded)
  int32_t pfirst[MUSE_MAXLEV + 1];  // first problem of each entry (both sets)
};

// Per-kernel timing with HIP events on the launch stream (off by default).
extern int g_ktime_on;
void ktime_pre(hipStream_t st);
void ktime_post(const char* name, hipStream_t st);
void set_smem_once(const void* fn, size_t bytes);

hipError_t launch_kmeans(const Plan& pl, int dtype, const CSet& s0, const CSet& s1, int plocal,
                         const KmLarge& lg, float* part, int32_t* pcnt, hipStream_t st);
size_t kmeans_smem_bytes(int dtype, int D, int C);
int kmeans_sub(int dtype, int D);

// Key-cluster statistics n, mu, S, M of every key problem of `ks`.
struct KStats {
  float* mu;    // [heads][P][C][D]
  float* S;     // [heads][P][C][D]
  float* M;     // [heads][P][D][C][D]  (value dim, cluster, key dim)
  void* mu_in;  // [heads][P][C][D] centroids in the input dtype (or null)
  void* Kp;     // [nlev][heads][N][D] keys in cluster-contiguous order (or null)
  void* Vp;     // [nlev][heads][N][D] values, same order (or null)
};
hipError_t launch_summarize(const Plan& pl, int dtype, const CSet& ks, const void* V, KStats st_,
                            hipStream_t st);

// Scores + top-k retrieval, and tilted summaries.
struct AttnBufs {
  const void* Q; const void* K; const void* V;
  CSet qs, ks;            // query / key clustering (labels, perm, offs, cent)
  KStats kst;
  int32_t* R;             // [B*Hq][P][C][k1w]
  void* T;                // [B*Hq][P][C][D][Cp32] T_Ic / n_c (exact tilt: U_Ic) in the input dtype (I, d, c)
  int32_t Cp32;           // C rounded up to 32
  void* Vt;               // value columns: [nlev*B*Hkv sorted copies (+ B*Hkv input V)][D][Nv]
  int32_t Nv;             // N rounded up to 8
  void* kap;              // exact tilt: tilted key centroids [B*Hq][P][C][Cp32][D] (input dtype)
  float* lz;              // exact tilt: ln Z_Ic [B*Hq][P][C][Cp32]
  float* fb;              // exact tilt: far bias log2 Z_Ic - s log2(e) nu_I.kappa_Ic, same layout
  // spatial blocks with accumulated summaries (Plan::v4); layouts as in muse.h
  int32_t* r1;            // [B*Hq][Cq][nb][k1w] retrieved clusters of each group
  int32_t* r2;            // [B*Hq][Cq][nb][k1w][k2w] retrieved blocks
  int32_t* kb;            // [B*Hkv][Ck][nb+1] block starts inside each key cluster's run
  int32_t* qb;            // [B*Hq][Cq][nb+1] same for the query clusters
  float* pz;              // [B*Hq][Cq][Ck][nb] ln Z of each (c, beta) seen from nu_I
  float* pk;              // [B*Hq][Cq][Ck][nb][D] tilted key means
  float* pu;              // [B*Hq][Cq][Ck][nb][D] tilted value means
  void* fk;               // [B*Hq][nb][Cq][Cp32][D] far key rows of each group (input dtype)
  void* fv;               // [B*Hq][nb][Cq][D][Cp32] far values (input dtype)
  float* fbias;           // [B*Hq][nb][Cq][Cp32] far bias (base 2), -inf when empty
  float* oacc;            // causal running output [B*Hq][N][D] (fp32)
  float* lacc;            // causal running lse [B*Hq][N]
  void* O; float* lse;    // outputs
};
hipError_t launch_score_topk(const Plan& pl, const AttnBufs& b, hipStream_t st);
hipError_t launch_tilt(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st);
hipError_t launch_score_tilt(const Plan& pl, int dtype, const AttnBufs& b, bool& vt_done, hipStream_t st);
hipError_t launch_attn(const Plan& pl, int dtype, const AttnBufs& b, bool vt_done, hipStream_t st);
// Exactly tilted statistics (kap, T = tilted value means, lz, fb) and the
// retrieval sets ranked by lz.
hipError_t launch_tilt_exact(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st);

// Spatial blocks with causally accumulated summaries: block bounds, the
// exactly tilted statistics of every (query cluster, key cluster, block),
// the two-level retrieval of every group and its far items.
hipError_t launch_v4(const Plan& pl, int dtype, const AttnBufs& b, hipStream_t st);

// Backward with the forward's clustering state held fixed.
struct BwdLaunch {
  Plan pl;
  int dtype;
  AttnBufs a;             // forward state; a.T holds the recomputed T / n_c, a.O the forward output
  const void* dO;
  const float* lse;
  float* delta;           // [B*Hq][N]
  float* dq; float* dk; float* dv;   // fp32 accumulators, [heads][N][D]
  void* dT;               // per-level scratch in the input dtype, see bwd.hip
  float* G;
  float* dnu;
  float* dS;
  float* dmu;
  float* dM;
  void* dQ; void* dK; void* dV;      // outputs in the input dtype
};
hipError_t launch_bwd(const BwdLaunch& L, hipStream_t st);

}  // namespace muse

#define MUSE_KT_PRE(st) \
  do { if (muse::g_ktime_on) muse::ktime_pre(st); } while (0)
#define MUSE_KT_POST(name, st) \
  do { if (muse::g_ktime_on) muse::ktime_post(name, st); } while (0)
