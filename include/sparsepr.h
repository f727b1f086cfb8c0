/*
 * sparsepr.h -- C ABI of the SparsePR attention-call hot path on MI355X (gfx950).
 *
 * One call computes, per head, an approximation of softmax(Q K^T / sqrt(d)) V
 * (the attention formula of the framerc.cn post "SparsePR稀疏注意力：无训练加速
 * 视频生成与世界模型推理", section 1.2) in five stages, following the method
 * summary "Partition the Support, Reconstruct the Residual: Training-Free Sparse
 * Attention for Video Generation and World Models" (gist.science), section 2:
 *
 *   sparsepr_partition   2A  response-coupled partition (keys by k-means in the
 *                            eigen-coordinates of M_K = Q_s^T Q_s / M_s, then queries
 *                            by k-means of their logit profile on the key-group centroids)
 *   sparsepr_route       2C  group-major layout of Q/K/V; centroid-logit top-k key groups
 *                            per query group (the block selection of "Attention Sparsity
 *                            is Input-Stable ... Online QK Co-Clustering", papernotes.org);
 *                        2B  stratified probe rows
 *   sparsepr_sparse_attn 2C  variable-block-sparse attention over the routed pairs, and
 *                        2B  exact dense attention of the probe rows
 *   sparsepr_probe_fit   2B  ridge affine fit R ~ b + x B of the probe residuals, restricted
 *                            to the leading right singular subspace of the residuals
 *   sparsepr_correct     2B  fitted residual added to the unprobed rows; original order
 *
 * Conventions for every entry point
 *   - Q, K, V and O are [heads][n][d] row-major, contiguous, 16-byte aligned device
 *     buffers of the context's dtype (bf16, or fp32 holding any values: fp32 inputs
 *     are rounded to bf16, nearest-even, on entry; O is written in the same dtype).
 *   - Device work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream). Entry points return once the work is enqueued, except where
 *     noted: the probe-fit stage solves a small fp64 system on the host and waits for
 *     the probe rows (not for the sparse kernel) to do so; the partition stage does the
 *     same only with SPARSEPR_F_HOST_SOLVE.
 *   - The caller owns Q/K/V/O and keeps them alive until the stream work is done.
 *     The context owns every intermediate. Between calls it keeps only what the
 *     inspection getters read back and the partition and routing that
 *     sparsepr_reuse_route reuses.
 *   - Every function returns a sparsepr_status; nothing throws or aborts across the
 *     ABI. Arguments are validated before anything is enqueued. A HIP error returns
 *     SPARSEPR_ERR_HIP and poisons the context (destroy it). Stages must run in order
 *     partition -> route -> sparse_attn -> probe_fit -> correct, or reuse_route in place
 *     of the first two (else SPARSEPR_ERR_ORDER). A context is bound to one device, is
 *     not thread-safe, and overlapping calls on one context race.
 *   - Results are bitwise deterministic for identical inputs and parameters.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sparsepr_ctx sparsepr_ctx;

enum {
    SPARSEPR_OK = 0,
    SPARSEPR_ERR_INVALID_ARG = 1,   /* bad pointer or parameter value */
    SPARSEPR_ERR_SHAPE = 2,         /* shape outside the supported range */
    SPARSEPR_ERR_OOM = 3,           /* device or host allocation failed */
    SPARSEPR_ERR_HIP = 4,           /* HIP runtime / launch error (context poisoned) */
    SPARSEPR_ERR_ORDER = 5,         /* stage called before its prerequisite */
    SPARSEPR_ERR_NUMERIC = 6        /* a small solve failed (non-finite input) */
};

enum { SPARSEPR_BF16 = 0, SPARSEPR_F32 = 1 };

/* flags */
#define SPARSEPR_F_STAGE_TIMING 1u  /* record per-stage HIP events (sparsepr_get_stats) */
#define SPARSEPR_F_RAW_KMEANS 2u    /* comparison partitioner, not the method: keys and queries
                                       each clustered by plain Euclidean k-means of their raw
                                       rows (the independent Q/K clustering of cluster-based
                                       sparse attention), with the same seeds, rounds, routing,
                                       probes and correction; no M_K and no host round trip */
#define SPARSEPR_F_SVOO 16u         /* comparison partitioner, not the method: the online
                                       bidirectional co-clustering of "Attention Sparsity is
                                       Input-Stable ..." (papernotes.org, online co-clustering
                                       item). kmeans_iters alternating rounds: keys are assigned
                                       in the affinity space of the current query centroids
                                       (metric C_Q^T C_Q / d on raw keys), their raw means
                                       updated, then queries in the affinity space of the new key
                                       centroids (C_K^T C_K / d); seeds are the rows at the
                                       first G Weyl indices, an empty block's centroid is the zero
                                       vector. Same routing, probes and correction; no M_K and no
                                       host round trip. Not combinable with
                                       SPARSEPR_F_RAW_KMEANS (SPARSEPR_ERR_INVALID_ARG). */
#define SPARSEPR_F_HOST_SOLVE 8u    /* solve the M_K eigenproblem on the host (fp64, the partition
                                       stage then synchronises its stream once) instead of on
                                       the device; also used whenever key_rank > 64 */
#define SPARSEPR_F_SERIAL_PARTITION 32u  /* run the partition's per-head steps for all heads on the
                                       caller's stream. By default (H >= 2) the first and the
                                       second half of the heads run on two streams that the
                                       partition stage forks from and joins back into the caller's
                                       stream, so that their small launches overlap; the results
                                       are the same either way. */
#define SPARSEPR_F_FP8_QK 64u       /* an experiment, not the method's precision: the sparse
                                       kernel's logits Q K^T from Q and K rounded to FP8 E4M3
                                       (OCP 8-bit float, largest magnitude 448) after per-head
                                       power-of-two scales (the largest e with max|x| 2^e <= 448),
                                       on the fp8 matrix instruction; P V, the probe rows, the fit
                                       and the correction are unchanged. Quantization is the
                                       extension "SparsePR稀疏注意力..." (framerc.cn) section 8.4
                                       names. The workspace grows by one byte per K element. */
#define SPARSEPR_F_RAW_KEY_SCREEN 128u  /* the key k-means screens each key in raw space (x against
                                       C' = W c, depth 2 d) instead of in its coordinates x W
                                       (split into bf16 hi + lo, depth 4 r_K, formed once per
                                       call; the default when the key centroids' split
                                       coordinates fit in LDS and r_K is 16 or 32, also for the
                                       candidate lists of a large G_k). Both screens certify against the same
                                       exact scores and send the rest to the same fp64 recheck,
                                       so the labels are the same either way; for comparison. */
#define SPARSEPR_F_UNIFORM_UNITS 256u  /* the sparse kernel takes every query group in 128-row work
                                       units (4-wave blocks, two per CU). By default each group's
                                       whole 256-row chunks, and a rest of more than 128 rows, run
                                       as 256-row units (8-wave blocks that walk the group's routed
                                       key union once for up to 256 rows), beside a second launch
                                       that takes the shorter rests in 128-row units (calls of
                                       at least 2^17 query rows, H N; smaller ones always take
                                       128-row units). The
                                       rows' arithmetic, and so the output, is the same bit for
                                       bit either way; for comparison. SPARSEPR_F_FP8_QK always
                                       takes 128-row units. */
#define SPARSEPR_F_CHECK_FINITE 4u  /* count non-finite values of q and k (partition), v (route)
                                       and o (correct) on the device; read the counts with
                                       sparsepr_get_stats. The stages stay asynchronous and do not
                                       fail on them (a non-finite M_K or probe fit still returns
                                       SPARSEPR_ERR_NUMERIC where the stage solves on the host). */

typedef struct {
    int32_t heads;          /* H >= 1 */
    int32_t n;              /* tokens N, 1 .. 2^24 with n * d * 2 < 2^31 (one head's bf16 rows
                               must fit the kernels' 32-bit buffer offsets) */
    int32_t d;              /* head dim, 64 or 128 */
    int32_t dtype;          /* SPARSEPR_BF16 or SPARSEPR_F32 (Q, K, V and O) */
    int32_t n_sample;       /* M_s sampled queries for M_K, 1 .. n */
    int32_t key_rank;       /* r_K leading eigenvectors of M_K, 1 .. d */
    int32_t kv_groups;      /* G_k, 1 .. min(n, 1024) */
    int32_t q_groups;       /* G_q, 1 .. min(n, 1024) */
    int32_t kmeans_iters;   /* T >= 1 Lloyd rounds per k-means */
    int32_t probes;         /* P probe rows per head, 0 .. min(n, 4096) */
    int32_t corr_rank;      /* r, 0 .. d */
    uint32_t flags;         /* SPARSEPR_F_* */
    double density;         /* rho in (0, 1]: k = ceil(rho G_k - 1e-9) key groups per query group */
    double ridge_lambda;    /* lambda >= 0 (absolute; 0 = minimum-norm least squares) */
} sparsepr_params;

typedef struct {
    int64_t routed_pairs;      /* sum over heads and query rows of |U_i| */
    int64_t probe_pairs;       /* P * N * H */
    double  exec_density;      /* (routed_pairs + probe_pairs) / (H N^2) */
    int64_t recheck_points;    /* k-means points resolved in fp64 after an uncertified fp32 margin */
    int32_t routed_k;          /* key groups kept per query group */
    int32_t query_dims;        /* dimension the query k-means runs in: d (the logit-profile
                                  metric C_K^T C_K / d is applied in full) */
    float   stage_ms[6];       /* mean ms per call of: partition, route, sparse attention kernel,
                                  probe rows (the fit Grams run on a side stream), probe fit (the part of the
                                  host solve and upload not hidden behind the sparse kernel),
                                  correction (SPARSEPR_F_STAGE_TIMING;
                                  averaged over the calls since the previous
                                  sparsepr_get_stats, at most the last 64) */
    int32_t timed_calls;       /* calls averaged into stage_ms */
    int64_t nonfinite_inputs;  /* SPARSEPR_F_CHECK_FINITE: non-finite values in q, k, v of the last call */
    int64_t nonfinite_outputs; /* SPARSEPR_F_CHECK_FINITE: non-finite values in o of the last call */
    double  metric_gap_min;    /* min over heads of lambda_r / lambda_{r+1}, the gap after the r_K
                                  leading eigenvalues of M_K (+inf when r_K = d or lambda_{r+1} <= 0;
                                  0 with SPARSEPR_F_RAW_KMEANS, which has no M_K). Near 1 the key
                                  coordinates, and so the key labels, are not unique. */
    double  resid_gap_min;     /* min over heads of sigma_r / sigma_{r+1} of the probe residuals Y
                                  (+inf when the kept rank reaches min(P, d) or sigma_{r+1} = 0).
                                  Near 1 the correction subspace is not unique. */
} sparsepr_stats;

/* ---- parameters and lifetime (host only; sparsepr_create allocates on the current device) ---- */

/* Check a parameter set; no GPU work. Returns SPARSEPR_OK or the first violation. */
int32_t sparsepr_validate(const sparsepr_params* p);

/* k = ceil(rho G_k - 1e-9) clamped to [1, G_k]: the key groups routed per query group
 * (the width of the block lists). -status for an invalid parameter set. */
int32_t sparsepr_routed_count(const sparsepr_params* p);

/* Device bytes a context needs for these parameters (0 if invalid). */
size_t sparsepr_workspace_bytes(const sparsepr_params* p);

/* Validate and allocate a context on the current HIP device. *out is set only on success. */
int32_t sparsepr_create(const sparsepr_params* p, sparsepr_ctx** out);

/* Free the context (synchronises its device first). NULL is ignored. */
void sparsepr_destroy(sparsepr_ctx* ctx);

/* Static text for a status code. */
const char* sparsepr_status_str(int32_t status);

/* Detail of the context's last error ("" if none). With ctx NULL: why this thread's last
 * sparsepr_create or sparsepr_dense_attn_noalloc failed (the HIP call and its error
 * string, or the limit exceeded; "" after a success). */
const char* sparsepr_last_error(const sparsepr_ctx* ctx);

/* ---- the five stages (section 2 of the method summary) ---- */

/* 2A. Reads q, k. Asynchronous: M_K, its leading eigenpairs (fp64: Householder
 * tridiagonalisation, bisection, twisted-factorisation eigenvectors, inverse iteration only
 * inside clusters of near-equal eigenvalues) and both k-means run on the device.
 * With SPARSEPR_F_HOST_SOLVE, or key_rank > 64, the eigensolve runs on the host instead and
 * the stage synchronises `stream` once. The query side uses the logit-profile metric
 * C_K^T C_K / d in full.
 * Leaves key/query labels and centroids in the context. With SPARSEPR_F_RAW_KMEANS both
 * sides use the identity metric instead (no host round trip). K is then permuted into
 * group-major order on the context's side stream while the query side runs, so k must
 * stay unchanged until sparsepr_sparse_attn has run (sparsepr_dense_attn waits for this
 * permute before it rewrites the context's bf16 copy of an fp32 k). */
int32_t sparsepr_partition(sparsepr_ctx* ctx, const void* q, const void* k, void* stream);

/* 2C/2B. Reads v (k is only checked). Stable group-major permutation of V, top-k key
 * groups per query group (ties to the lower group index, empty key groups never kept),
 * probe rows.
 * V is copied into group-major fp16, scaled per head by an exact power of two (exact for
 * every bf16 value above 2^-29 of the head's largest |v|), for the sparse kernel's fp16 P.V.
 * Q is not copied: sparsepr_sparse_attn gathers its rows through the query permutation,
 * and the probe rows gather bf16 V rows through the key permutation, so q and v must stay
 * unchanged until sparsepr_sparse_attn has run (for an fp32 context the rows come from the
 * context's bf16 copies, which sparsepr_dense_attn also rewrites: do not call it in
 * between). */
int32_t sparsepr_route(sparsepr_ctx* ctx, const void* q, const void* k, const void* v,
                       void* stream);

/* 2C/2B. Exact dense + routed attention of the probe rows and the fit's fp64 Grams
 * (copied to pinned host memory), then block-sparse attention over the routed pairs
 * (unrouted blocks are never touched). Reads the q given to sparsepr_route.
 * Asynchronous: returns once both are enqueued. */
int32_t sparsepr_sparse_attn(sparsepr_ctx* ctx, void* stream);

/* 2B. fp64 fit on the host: B' = B Pi and b' = b Pi per head. Waits only for the probe
 * rows and Grams enqueued by sparsepr_sparse_attn, so the solve overlaps the sparse
 * kernel; B' and b' are uploaded on `stream`. */
int32_t sparsepr_probe_fit(sparsepr_ctx* ctx, void* stream);

/* 2B. Writes o [H][n][d] (context dtype) in the original token order: unprobed rows
 * get O_s + b' + O_s B', probe rows their exact dense output. */
int32_t sparsepr_correct(sparsepr_ctx* ctx, void* o, void* stream);

/* Reuse of the last partition and routing, an experiment and not part of the method (the
 * SparsePR summary, section 2B, says the method itself uses no temporal reuse; the framerc.cn
 * page's mask_update_stride updates the sparse mask only every few denoising steps). Takes
 * new q, k, v of the context's shape and treats them as the 2C/2B input of a new call that
 * keeps the previous call's labels, group-major permutations, block lists, probe rows and
 * work units: K and V are permuted through the kept key permutation (K on the side stream,
 * V into scaled fp16 as in sparsepr_route) and Q rows are gathered through the kept query
 * permutation. Leaves the context ready for sparsepr_sparse_attn; the same lifetime rules
 * for q, k and v as sparsepr_route apply. SPARSEPR_ERR_ORDER if no sparsepr_route (or
 * sparsepr_set_partition + sparsepr_route) has completed on this context. Asynchronous. */
int32_t sparsepr_reuse_route(sparsepr_ctx* ctx, const void* q, const void* k, const void* v,
                             void* stream);

/* ---- convenience and baseline ---- */

/* All five stages in order. */
int32_t sparsepr_attention(sparsepr_ctx* ctx, const void* q, const void* k, const void* v,
                           void* o, void* stream);

/* sparsepr_reuse_route, then the sparse attention, probe fit and correction: one call on
 * the previous call's partition and routing (the reuse experiment above). */
int32_t sparsepr_attention_reuse(sparsepr_ctx* ctx, const void* q, const void* k, const void* v,
                                 void* o, void* stream);

/* Dense softmax(Q K^T / sqrt(d)) V with this library's attention kernel (one group
 * holding every key); uses the context's shapes and workspace, no other stage state. */
int32_t sparsepr_dense_attn(sparsepr_ctx* ctx, const void* q, const void* k, const void* v,
                            void* o, void* stream);

/* The dense baseline with no allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * No context: q, k, v and o are caller-owned bf16 [heads][n][d] device buffers (16-byte
 * aligned); the same kernel, launch and results as sparsepr_dense_attn on a bf16 context.
 * The call's only scratch, its work-unit metadata, is a static device array of 65,792
 * bytes that each device holds until the process ends (its address is looked up on the
 * first call on a device). Limits: d in {64, 128}, 1 <= n <= 2,097,152 (8192 units of 256
 * rows), heads * n < 2^31, else SPARSEPR_ERR_SHAPE; null or misaligned pointers give
 * SPARSEPR_ERR_INVALID_ARG, a failed launch SPARSEPR_ERR_HIP; the detail is in
 * sparsepr_last_error(NULL). Asynchronous on `stream`. Every call on a device rewrites that
 * device's array, so calls that overlap on one device (other streams or threads) race. */
int32_t sparsepr_dense_attn_noalloc(int32_t heads, int32_t n, int32_t d, const void* q,
                                    const void* k, const void* v, void* o, void* stream);

/* ---- inspection (copy context-owned results out; NULL destinations are skipped).
 * host != 0: destinations are host memory and `stream` is synchronised before return;
 * host == 0: destinations are device memory, copies are enqueued on `stream`. ---- */

/* int32 [H][n] labels and permutations (perm[new] = old), int32 [H][G+1] offsets. */
int32_t sparsepr_get_partition(sparsepr_ctx* ctx, int32_t* key_labels, int32_t* q_labels,
                               int32_t* key_perm, int32_t* q_perm, int32_t* key_off,
                               int32_t* q_off, int32_t host, void* stream);

/* blocks int32 [H][G_q][k] ascending, -1 padded; probe rows int32 [H][P] as original
 * token indices and as group-major positions. */
int32_t sparsepr_get_routing(sparsepr_ctx* ctx, int32_t* blocks, int32_t* probe_orig,
                             int32_t* probe_pos, int32_t host, void* stream);

/* The key metric M_K = Q_s^T Q_s / M_s (fp64 [H][d][d]) and the key coordinates' map
 * W = U_r diag(sqrt(lambda_r)) (fp64 [H][d][r_K]) of the last partition (section 2A). Only
 * W W^T is defined (eigenvector signs and rotations inside a repeated eigenvalue are free).
 * Not available with SPARSEPR_F_RAW_KMEANS or SPARSEPR_F_SVOO (SPARSEPR_ERR_ORDER). */
int32_t sparsepr_get_metric(sparsepr_ctx* ctx, double* m_k, double* w, int32_t host, void* stream);

/* Raw fp64 centroids: keys [H][G_k][d], queries [H][G_q][d] (zero for an empty group). */
int32_t sparsepr_get_centroids(sparsepr_ctx* ctx, double* key_centroids, double* q_centroids,
                               int32_t host, void* stream);

/* fp32 [H][n][d] sparse output in group-major order (before correction). */
int32_t sparsepr_get_sparse_out(sparsepr_ctx* ctx, float* o_sparse, int32_t host, void* stream);

/* fp32 [H][P][d] probe sparse outputs X and residuals Y = O_dense - X. */
int32_t sparsepr_get_probes(sparsepr_ctx* ctx, float* x, float* y, int32_t host, void* stream);

/* fp64 B' [H][d][d] and b' [H][d]. */
int32_t sparsepr_get_fit(sparsepr_ctx* ctx, double* b_mat, double* b_vec, int32_t host,
                         void* stream);

/* Per-head spectral gaps of the last call (fp64 [H] each; NULL skips): lambda_r/lambda_{r+1}
 * of M_K and sigma_r/sigma_{r+1} of the probe residuals (see sparsepr_stats). Host memory
 * only (host must be 1); synchronises `stream`. */
int32_t sparsepr_get_gaps(sparsepr_ctx* ctx, double* metric_gap, double* resid_gap, int32_t host,
                          void* stream);

/* Counters of the last call and mean stage times since the previous call of this
 * function (synchronises the context's last stream). */
int32_t sparsepr_get_stats(sparsepr_ctx* ctx, sparsepr_stats* out);

/* Test hook: replace the partition with given labels (int32 [H][n] each, values in
 * [0, G); host != 0: host memory, else device memory) for the device inputs q, k;
 * the raw group centroids and the group-major permutations are recomputed, and the
 * context is then ready for sparsepr_route. Out-of-range labels: SPARSEPR_ERR_INVALID_ARG
 * (checked only for host labels). */
int32_t sparsepr_set_partition(sparsepr_ctx* ctx, const void* q, const void* k,
                               const int32_t* key_labels, const int32_t* q_labels, int32_t host,
                               void* stream);

/* ---- host-side fp64 solves used by the partition and probe-fit stages (no GPU) ---- */

/* Top-r eigenpairs of a symmetric n x n matrix a (row-major, n <= 1024): eigenvalues
 * descending into lam[r], eigenvectors as columns of vec [n][r]. */
int32_t sparsepr_host_sym_eig_top(int32_t n, const double* a, int32_t r, double* lam,
                                  double* vec);

/* Key projection W = U_r diag(sqrt(max(lambda_r, 0))) [d][r] of the metric m_k [d][d]. */
int32_t sparsepr_host_key_projection(int32_t d, const double* m_k, int32_t r, double* w);

/* Probe fit from X, Y [p][d] (fp64): B' [d][d], b' [d]. */
int32_t sparsepr_host_probe_fit(int32_t p, int32_t d, const double* x, const double* y,
                                double lambda, int32_t rank, double* b_mat, double* b_vec);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEPR_H */
