/*
 * muse.h - C ABI of the MuSe (Multipole Semantic Attention) library for
 * AMD Instinct MI355X (gfx950).
 *
 * MuSe approximates softmax attention (arXiv 2509.10406, "Multipole Semantic
 * Attention: A Fast Approximation of Softmax Attention for Pretraining").
 * Passages are cited by page and section:
 *   [GIST]  gist.science page, Technical Summary, Core Mechanisms
 *   [NEWX]  newx.sg page, Abstract
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are row-major.  Attention inputs use the layout [B, H, N, D]:
 *   Q has Hq heads, K and V have Hkv heads, Hq % Hkv == 0, and query head h
 *   reads KV head floor(h * Hkv / Hq) (grouped-query attention).  The value
 *   dimension equals D.  D must be 64 or 128.
 * - dtype: MUSE_BF16 (bfloat16 storage, fp32 accumulation) or MUSE_F32.
 *   Outputs O, dQ, dK, dV use the input dtype; lse and all statistics are fp32.
 * - Every pointer argument that names a tensor is a DEVICE pointer on the
 *   current HIP device, except where a function says "host".  The caller
 *   allocates and owns all memory (inputs, outputs, state, workspace); the
 *   library never allocates, frees or synchronises.  Work is queued on
 *   `stream` (a hipStream_t; NULL is the default stream) and is asynchronous.
 * - Return value: MUSE_OK (0) or a negative error code.  All argument
 *   checks happen on the host before the first launch, so an error return
 *   means nothing was queued, except MUSE_EHIP (a launch failed; the HIP
 *   error string is available from muse_last_hip_error()).
 * - Alignment: Q, K, V, O, dO, dQ, dK, dV, X, centroids and the state and
 *   workspace buffers must be 16-byte aligned (MUSE_EINVAL otherwise); the
 *   kernels move their rows with 16-byte vector accesses.
 * - Clamping (documented, not errors): a problem with n < C points uses
 *   C_eff = n clusters; k1 is clamped to the number of non-empty key
 *   clusters of each problem.
 */
#ifndef MUSE_H
#define MUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MUSE_F32 = 0, MUSE_BF16 = 1 } muse_dtype;

enum {
  MUSE_OK = 0,
  MUSE_EINVAL = -1,       /* bad shape, dtype, null pointer or parameter */
  MUSE_EWORKSPACE = -2,   /* workspace or state buffer too small */
  MUSE_EUNSUPPORTED = -3, /* valid request this build does not handle */
  MUSE_EHIP = -4          /* a HIP launch or runtime call failed */
};

#define MUSE_MAX_CLUSTERS 256

/*
 * Hyperparameters.  The pages state that MuSe needs only hyperparameters
 * and no architectural change [NEWX]: the cluster counts, the number of
 * retrieved clusters k1 ([GIST] Retrieval-Augmented Approximation), the
 * causal flag and the local block size of the causal hierarchy [NEWX].
 *   cq, ck   clusters per query / key problem, 1..256 each ([GIST]
 *            Bidirectional Semantic Clustering: queries and keys are
 *            clustered separately).  Per-cluster arrays of the state are
 *            laid out with C = max(cq, ck) clusters per problem; the side
 *            with fewer clusters has empty clusters beyond its own count.
 *   iters    Lloyd iterations, >= 1.
 *   topk     k1, clusters per query cluster attended exactly, >= 0.
 *   block    causal local block size (>= 1); ignored when causal == 0.
 *   causal   0: acausal; 1: causal hierarchy (exact local blocks of size
 *            `block`, approximated off-diagonal blocks on ceil(log2(
 *            ceil(N/block))) dyadic levels); 2: causal spatial blocks with
 *            causally accumulated summaries ([GIST] Causal Accumulation,
 *            Retrieval-Augmented Approximation): queries and keys are
 *            clustered once per head over all N rows; a query of cluster I
 *            in block b = floor(i / block) attends exactly to the rows of
 *            its own block up to itself, to the top-`topk` key clusters by
 *            ln Z over the keys of earlier blocks and, inside each, to the
 *            keys of its top-`topk2` earlier blocks by ln Z over that
 *            block's keys; every other key of an earlier block enters
 *            through one exactly tilted far item per key cluster (its
 *            earlier keys minus the retrieved blocks).  Requires dipole == 2
 *            (MUSE_EUNSUPPORTED otherwise), at most 4096 blocks and
 *            k1w * k2w <= 256; museattn_bwd returns MUSE_EUNSUPPORTED.
 *   dipole   1: monopole + dipole summaries (first-order tilt: T_Ic =
 *            S_c + s M_c nu_I, far log-weight s q.mu_c + ln n_c; retrieval
 *            by s nu_I.mu_c + ln n_c); 0: monopole only (T_Ic = S_c);
 *            2: exact exponential tilt ([GIST] Exponential Tilting): the far
 *            item of key cluster c for a query q of query cluster I has
 *            log-weight ln Z_Ic + s (q - nu_I).kappa_Ic and value U_Ic, with
 *            Z_Ic = sum_{j in c} exp(s nu_I.k_j), kappa_Ic and U_Ic the
 *            keys' and values' means under those weights; retrieval ranks
 *            clusters by ln Z_Ic.  museattn_bwd returns MUSE_EUNSUPPORTED
 *            for 2.
 *   init_mode  0: the k-means of every problem starts from the points given
 *            by init_q / init_k (or the default points); 1: warm start, the
 *            Lloyd iterations continue from the centroids already held in
 *            `state` (q_cent, k_cent), which must come from an earlier
 *            museattn_fwd with the same shapes and cq, ck, block and causal
 *            (for example the previous training step on the same layer);
 *            init_q / init_k are then ignored.  The library cannot check
 *            where those centroids came from.
 *   scale    softmax scale s applied to q.k; <= 0 means 1/sqrt(D).
 *   topk2    k2, blocks retrieved inside each retrieved cluster (causal ==
 *            2 only; >= 1 when topk >= 1, clamped to the number of blocks;
 *            ignored otherwise).
 */
typedef struct {
  int32_t cq, ck, iters, topk, block, causal, dipole, init_mode;
  float scale;
  int32_t topk2;
} muse_cfg;

/*
 * Byte offsets of the arrays held in the `state` buffer that museattn_fwd
 * fills and museattn_bwd reads (the fixed assignments of the backward).
 * P = problems per head (1 when acausal), L = levels (1 when acausal),
 * C = max(cq, ck), k1w = max(1, min(topk, ck)), Cp32 = C rounded up to a
 * multiple of 64,
 * Nv = N rounded up to a multiple of 8.
 *   q_labels  int32 [L][B*Hq][N]      query cluster of each row per level
 *   k_labels  int32 [L][B*Hkv][N]
 *   q_perm    int32 [L][B*Hq][N]      per problem, sorted position -> row
 *   k_perm    int32 [L][B*Hkv][N]     (positions relative to the problem's
 *                                      first row, row ids absolute)
 *   q_offs    int32 [B*Hq][P][C+1]    cluster segment starts in q_perm
 *   k_offs    int32 [B*Hkv][P][C+1]
 *   q_cent    fp32  [B*Hq][P][C][D]   query-cluster centroids nu
 *   k_cent    fp32  [B*Hkv][P][C][D]  key k-means centroids
 *   mu        fp32  [B*Hkv][P][C][D]  key-cluster centroids mu
 *   S         fp32  [B*Hkv][P][C][D]  value sums
 *   M         fp32  [B*Hkv][P][D][C][D] dipoles, index (value dim, c, key dim)
 *   R         int32 [B*Hq][P][C][k1w] retrieved clusters, ascending, -1 pad
 *   Kp, Vp    dtype [L][B*Hkv][N][D]  keys / values of each key problem in
 *                                      cluster-contiguous order (slot r0 + q
 *                                      holds the row at sorted position q)
 *   mu_in     dtype [B*Hkv][P][C][D]  mu rounded to the input dtype
 * Problem p of a head: level l and segment t in level-major order (see
 * muse_plan).  Counts are k_offs[c+1] - k_offs[c].
 */
typedef struct {
  int64_t P, L, C, k1w, Cp32, Nv;
  size_t q_labels, k_labels, q_perm, k_perm, q_offs, k_offs, q_cent, k_cent, mu, S, M, R;
  size_t Kp, Vp, mu_in;
  size_t state_bytes;
  /* workspace arrays (scratch; valid after museattn_fwd until the next call) */
  size_t ws_T;      /* dtype [B*Hq][P][C][D][Cp32] T_Ic / n_c (exact tilt: U_Ic), index (I, d, c) */
  size_t ws_oacc;   /* fp32 [B*Hq][N][D] causal running output */
  size_t ws_lacc;   /* fp32 [B*Hq][N] causal running lse */
  size_t ws_Vt;     /* dtype [L*B*Hkv (+ B*Hkv when causal)][D][Nv] value columns of the sorted
                       copies (then of the input V), Nv = N rounded up to 8 */
  size_t ws_part;   /* k-means chunk partial sums */
  size_t ws_pcnt;
  size_t ws_bytes;
  /* exact tilt only (dipole == 2; zero-sized otherwise) */
  size_t ws_kap;    /* dtype [B*Hq][P][C][Cp32][D] tilted key centroids kappa_Ic */
  size_t ws_lz;     /* fp32 [B*Hq][P][C][Cp32] ln Z_Ic (-inf: empty cluster) */
  size_t ws_fb;     /* fp32 [B*Hq][P][C][Cp32] log2 Z_Ic - s log2(e) nu_I.kappa_Ic */
  /* causal == 2 only (zero-sized otherwise).  nb = ceil(N / block) blocks,
     k2w = max(1, min(topk2, nb)); group (I, b) = queries of cluster I in
     block b.  State: */
  int64_t nb, k2w;
  size_t v4_R1;     /* int32 [B*Hq][cq][nb][k1w] retrieved key clusters of each group,
                       ascending, -1 pad (all -1 for groups without queries and b = 0) */
  size_t v4_R2;     /* int32 [B*Hq][cq][nb][k1w][k2w] retrieved blocks of each retrieved
                       cluster, ascending, -1 pad */
  size_t v4_kb;     /* int32 [B*Hkv][ck][nb+1] position in k_perm of the first key of cluster c
                       in block beta (beta = nb: end of the cluster) */
  size_t v4_qb;     /* int32 [B*Hq][cq][nb+1] same for the queries in q_perm */
  /* workspace: */
  size_t ws_v4pz;   /* fp32 [B*Hq][cq][ck][nb] ln Z of the keys of (c, beta) seen from nu_I */
  size_t ws_v4pk;   /* fp32 [B*Hq][cq][ck][nb][D] their tilted key mean */
  size_t ws_v4pu;   /* fp32 [B*Hq][cq][ck][nb][D] their tilted value mean */
  size_t ws_v4kap;  /* dtype [B*Hq][nb][cq][Cp32][D] far-item key rows kappa of each group */
  size_t ws_v4T;    /* dtype [B*Hq][nb][cq][D][Cp32] far-item values U, index (d, c) */
  size_t ws_v4fb;   /* fp32 [B*Hq][nb][cq][Cp32] far-item bias log2 Z - s log2(e) nu_I.kappa,
                       -inf for an empty far item */
} muse_layout;

/*
 * Problem list of a call (host-only; no GPU needed).  Writes up to `cap`
 * rows of 6 int32 (level, t, k0, kn, q0, qn) to `out` (host memory) and the
 * number of problems per head to *count.  Acausal: one problem with keys
 * and queries = all N rows.  Causal: level l has span m = block * 2^l;
 * segment t has keys rows [2mt, 2mt + m) and queries rows
 * [2mt + m, min(2mt + 2m, N)), for every t with 2mt + m < N ([NEWX]
 * hierarchical block decomposition).
 */
int muse_plan(int64_t N, const muse_cfg* cfg, int32_t* out, int64_t cap, int64_t* count);

/*
 * Sizes and array offsets for a call with these shapes (host-only).
 * Returns MUSE_EINVAL for unsupported shapes or parameters.
 */
int muse_layout_query(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, muse_dtype dtype,
                      const muse_cfg* cfg, muse_layout* out);

/*
 * musecluster - Lloyd k-means of G independent point sets ([GIST]
 * Bidirectional Semantic Clustering: queries and keys are clustered
 * separately, each set in its own space).
 *   X          [G, n, D] points (dtype)
 *   C          clusters per set, 1..256 (clamped to n)
 *   iters      Lloyd iterations >= 1
 *   init_idx   int32 [G, C] starting point indices in [0, n), distinct per
 *              set (out-of-range values are clamped), or NULL for
 *              floor(c n / C_eff)
 *   assign     int32 [G, n] out: cluster of each point after the last
 *              assignment step (ties: lowest index)
 *   centroids  fp32 [G, C, D] out: mean of each cluster's members after the
 *              last update (empty clusters keep their previous centroid;
 *              rows >= C_eff are zero)
 *   perm       int32 [G, n] out: points in cluster-contiguous, stable order
 *   offs       int32 [G, C+1] out: segment starts in perm
 *   ws         workspace of at least muse_cluster_ws_size() bytes
 */
size_t muse_cluster_ws_size(int64_t G, int64_t n, int64_t D, muse_dtype dtype, int32_t C);
int musecluster(const void* X, muse_dtype dtype, int64_t G, int64_t n, int64_t D, int32_t C,
                int32_t iters, const int32_t* init_idx, int32_t* assign, float* centroids,
                int32_t* perm, int32_t* offs, void* ws, size_t ws_bytes, void* stream);

/*
 * musesummarize - monopole and dipole statistics of given key clusters
 * ([NEWX]: centroid approximation plus dipole correction).
 *   K, V      [G, n, D] keys and values (dtype)
 *   assign    int32 [G, n] cluster of each key, in [0, min(C, n)); values
 *             outside that range are clamped into it
 *   perm      int32 [G, n] out: stable cluster-contiguous order
 *   offs      int32 [G, C+1] out: segment starts; n_c = offs[c+1] - offs[c]
 *   mu        fp32 [G, C, D] out: mu_c = mean of the keys of c (0 if empty)
 *   S         fp32 [G, C, D] out: S_c = sum of the values of c
 *   M         fp32 [G, D, C, D] out: M[g][d][c][e] = sum_j v_jd (k_je - mu_ce)
 */
int musesummarize(const void* K, const void* V, muse_dtype dtype, int64_t G, int64_t n, int64_t D,
                  int32_t C, const int32_t* assign, int32_t* perm, int32_t* offs, float* mu,
                  float* S, float* M, void* stream);

/*
 * museattn_fwd - MuSe attention forward ([GIST] Decomposition, Hierarchical
 * Two-Stage Attention, Exponential Tilting, Retrieval-Augmented
 * Approximation; [NEWX] monopole + dipole, causal hierarchy).
 *   Q [B,Hq,N,D], K, V [B,Hkv,N,D]  inputs (dtype)
 *   init_q     int32 [B*Hq][P][cq] starting indices of the query k-means of
 *              every problem (relative to the problem's first query row) or
 *              NULL for floor(c n / C_eff)
 *   init_k     int32 [B*Hkv][P][ck] same for keys, or NULL
 *   O          [B,Hq,N,D] out (dtype)
 *   lse        fp32 [B,Hq,N] out: log of each row's softmax normaliser
 *   state      out: assignments and statistics (muse_layout), state_bytes
 *   ws         scratch, ws_bytes >= muse_layout.ws_bytes
 */
int museattn_fwd(const void* Q, const void* K, const void* V, muse_dtype dtype, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t N, int64_t D, const muse_cfg* cfg, const int32_t* init_q,
                 const int32_t* init_k, void* O, float* lse, void* state, size_t state_bytes,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * museattn_fwd_noalloc - museattn_fwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results as museattn_fwd; the workspace is a file-scope device
 * array of MUSE_NOALLOC_WS_BYTES (64 MiB) in the library, one per GPU,
 * held until the process ends.  The caller still passes inputs, outputs and
 * `state`.  The call allocates and frees nothing (per-kernel timing, when
 * switched on with muse_timing_enable, creates HIP events: leave it off).
 *   Returns MUSE_EWORKSPACE when the call's workspace (muse_layout.ws_bytes)
 *   exceeds MUSE_NOALLOC_WS_BYTES (e.g. the 8k acausal workload with 8 heads
 *   and 64 clusters needs about 20 MiB; the 64k causal workloads do not fit),
 *   MUSE_EHIP when the array's device address cannot be found, otherwise as
 *   museattn_fwd.
 * Every call on one GPU uses that GPU's single array and leaves its
 * contents behind: calls that overlap on one GPU (on different streams, or
 * from different host threads) race and must be serialised by the caller.
 */
#define MUSE_NOALLOC_WS_BYTES (64u << 20)
int museattn_fwd_noalloc(const void* Q, const void* K, const void* V, muse_dtype dtype, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t N, int64_t D, const muse_cfg* cfg,
                         const int32_t* init_q, const int32_t* init_k, void* O, float* lse, void* state,
                         size_t state_bytes, void* stream);

/*
 * museattn_bwd - gradients of museattn_fwd with the cluster assignments,
 * retrieval sets and counts held fixed (those saved in `state` by the
 * forward on the same Q, K, V and cfg); differentiates through the
 * centroids, value sums, dipoles and tilted summaries (the far-field item
 * of cluster c for query cluster I is a pseudo-key mu_c with value
 * T_Ic / n_c and log-weight ln n_c; gist.science page, Technical Summary,
 * Core Mechanisms; newx.sg page, Abstract).
 *   Q, K, V    the forward's inputs (device, dtype, [B,H,N,D] row-major)
 *   O, lse     the forward's outputs (device)
 *   dO         [B,Hq,N,D] upstream gradient (device, dtype)
 *   state      the forward's state buffer (device, read-only here)
 *   dQ         [B,Hq,N,D] out (device, dtype)
 *   dK, dV     [B,Hkv,N,D] out (device, dtype); sums over the query heads
 *              sharing a KV head
 *   ws         device scratch of ws_bytes >= muse_bwd_ws_size() bytes,
 *              owned by the caller; its contents are undefined afterwards
 *   stream     HIP stream (null = default); the call only queues work.
 * Accumulation is fp32 in a fixed order (no atomics): repeated calls give
 * bit-identical results.  Returns MUSE_EINVAL for null pointers or shapes /
 * parameters museattn_fwd rejects, MUSE_EWORKSPACE when state_bytes or
 * ws_bytes is too small, MUSE_EHIP when a launch fails.
 * muse_bwd_ws_size returns 0 for invalid arguments.
 */
size_t muse_bwd_ws_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, muse_dtype dtype,
                        const muse_cfg* cfg);
int museattn_bwd(const void* Q, const void* K, const void* V, const void* O, const float* lse,
                 const void* dO, muse_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                 int64_t D, const muse_cfg* cfg, const void* state, size_t state_bytes, void* dQ,
                 void* dK, void* dV, void* ws, size_t ws_bytes, void* stream);

/* Error text for a return code; HIP error text of the last MUSE_EHIP. */
const char* muse_strerror(int code);
const char* muse_last_hip_error(void);

/*
 * Per-kernel timing with HIP events recorded on the launch stream around
 * every kernel the library queues.  muse_timing_enable(1) starts recording,
 * muse_timing_collect() waits for the recorded events and adds their
 * durations to per-kernel totals, muse_timing_get() reads total ms and
 * launch count of entry `i` (returns MUSE_EINVAL past the last entry).
 */
int muse_timing_enable(int on);
int muse_timing_collect(void);
int muse_timing_reset(void);
int muse_timing_get(int i, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MUSE_H */
