/*
 * sparsepr.h — C ABI of the SparsePR attention call on AMD Instinct MI355X (gfx950).
 *
 * SparsePR (summary page of "Partition the Support, Reconstruct the Residual:
 * Training-Free Sparse Attention for Video Generation and World Models", Taghavi,
 * Langari, Pandey; cited below as PSRR with the paragraph's topic) replaces one dense
 * self-attention call with, in one call:
 *   1. a response-coupled Q/K partition (PSRR, response-coupled partition paragraph),
 *   2. routing of (query group x key group) cells to a target execution density with
 *      the probe cost subtracted first (PSRR, execution paragraph),
 *   3. a group-major permutation of Q, K and V (PSRR, execution paragraph),
 *   4. a variable-length block-sparse attention, exact on the kept cells and
 *      renormalised over the kept K/V groups (PSRR, execution paragraph),
 *   5. probe-row residual reconstruction: exact probe rows, a coverage-weighted ridge
 *      fit and a rank-r output-subspace projection, then write-back
 *      (PSRR, probe-fit residual reconstruction paragraph).
 * Under grouped-query attention the K/V partition and the route are shared by the
 * query heads of one KV head (PSRR, execution paragraph).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers allocated and owned by the caller; the
 *    library allocates nothing and keeps no state between calls (the one exception is the
 *    fixed device array of sparsepr_attend_noalloc), so every call may be captured into a
 *    HIP graph, the first one on a device included.
 *  - `stream` is a hipStream_t (NULL = the null stream).  All work is asynchronous on
 *    it; no entry point synchronises the host.
 *  - Tensors are contiguous, row-major, 16-byte aligned.  Element type of Q/K/V and of
 *    the final output is params->dtype (bf16 or fp32).
 *  - Every argument is checked on the host before any launch.  On error a negative
 *    sparsepr_status is returned and nothing is written.  Kernel launch failures
 *    return SPARSEPR_ERR_HIP.  No C++ exception crosses this interface.
 *  - Calls that share workspace or outputs must be ordered on one stream.
 *  - Limits: 1 <= n <= 2^22, d in {64, 128}, heads_q % heads_kv == 0,
 *    heads_q / heads_kv <= 16, 1 <= groups_q, groups_k <= 64, groups <= n,
 *    groups_k <= r_q, 1 <= r_k <= 64, 1 <= n_probe <= min(64, n),
 *    1 <= rank <= min(32, n_probe, d), lambda > 0, n_probe / n < rho_exec <= 1,
 *    0 <= kmeans_iters <= 64, block == 64, ablation, probe_mode, partition_mode, budget_mode
 *    and cost_mode one of their enumerators.
 *
 * Unfused call order: partition -> route -> attend -> probe_fit -> apply.
 * Fused call order:   partition -> route -> probe_fit -> attend_apply.
 * Overlapped order:   partition -> route -> (probe_fit on a second stream, attend) -> apply,
 *                     with a separate workspace for probe_fit or none for attend (attend
 *                     uses none) and apply ordered after both.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSEPR_OK = 0,
  SPARSEPR_ERR_NULL = -1,      /* a required pointer is NULL */
  SPARSEPR_ERR_SHAPE = -2,     /* n, d, heads or groups out of range */
  SPARSEPR_ERR_DTYPE = -3,     /* dtype not bf16 / fp32 */
  SPARSEPR_ERR_ALIGN = -4,     /* a tensor pointer is not 16-byte aligned */
  SPARSEPR_ERR_WORKSPACE = -5, /* workspace smaller than sparsepr_workspace_size() */
  SPARSEPR_ERR_PARAM = -6,     /* r_k, r_q, n_probe, rank, lambda, rho_exec, iters, block;
                                  or K/V gathers deferred by the partition not yet enqueued */
  SPARSEPR_ERR_HIP = -7        /* a HIP runtime call or kernel launch failed */
} sparsepr_status;

typedef enum { SPARSEPR_BF16 = 0, SPARSEPR_FP32 = 1 } sparsepr_dtype;

/* Ablations of the residual reconstruction (PSRR, ablation paragraph, which compares the
 * method with hard drop and with the ridge fit left unprojected).  Partition and route are
 * unchanged in every variant, so a comparison isolates the reconstruction. */
typedef enum {
  SPARSEPR_ABLATE_NONE = 0,        /* the method as specified */
  SPARSEPR_ABLATE_HARD_DROP = 1,   /* no reconstruction: the output is the renormalised sparse
                                      attention.  probe_fit writes an empty fit (probe tokens
                                      and groups -1, weights 0, r_eff 0, A, B, c0, eig, o_dense,
                                      o_sparse zero) and launches nothing else; apply and
                                      attend_apply write no probe rows. */
  SPARSEPR_ABLATE_RIDGE_ONLY = 2   /* the weighted ridge correction without the rank-r
                                      projection: ybar + (o - xbar) W with W = Xt^T Z, stored as
                                      A = Xt^T [Hq, d, n_probe], B = Z [Hq, n_probe, d],
                                      r_eff = n_probe, eig zero.  A and B then hold n_probe
                                      columns / rows in place of rank. */
} sparsepr_ablation;

/* How queries and keys are grouped (PSRR, ablation paragraph: the response-coupled
 * partition against a semantic partition that clusters the activations themselves). */
typedef enum {
  SPARSEPR_PARTITION_RESPONSE = 0, /* the method: keys by response curves, queries by response
                                      directions */
  SPARSEPR_PARTITION_SEMANTIC = 1  /* keys by their raw rows, queries by their raw rows (summed
                                      in fp32 over the KV head's query heads under GQA), each
                                      quantised to [-127, 127] on one power of two per head;
                                      same k-means, permutation, centroids and route.
                                      responses_s is not written; key_centroids_int is
                                      [Hkv, G_K, d], query_features [Hkv, n, d] and
                                      query_centroids [Hkv, G_Q, d]; exponents hold the two
                                      quantisation exponents. */
} sparsepr_partition_mode;

/* How the probe rows are chosen (PSRR, ablation paragraph: stratified probes against
 * random and uniform spatiotemporal sampling). */
typedef enum {
  SPARSEPR_PROBES_RADIAL = 0,      /* the method: stratified over query groups, radial order */
  SPARSEPR_PROBES_UNIFORM = 1,     /* tokens floor((2k+1) n / (2 n_probe)), k < n_probe, of the
                                      raster order; weight 1; group = the token's query label */
  SPARSEPR_PROBES_GIVEN = 2        /* the caller's tokens, read from fit->probe_tokens
                                      [Hkv, n_probe] on entry to probe_fit (e.g. drawn at random
                                      on the host); values outside [0, n) are clamped into it;
                                      weight 1; group = the token's query label */
} sparsepr_probe_mode;

/* How the route's budget is shared (PSRR, execution paragraph: the router spends a
 * budget of pairs after subtracting the probe cost; how it is split across heads is not
 * stated). */
typedef enum {
  SPARSEPR_BUDGET_PER_HEAD = 0,    /* the method as read here: every KV head gets
                                      floor(rho_ppm n^2 / 10^6) - n_probe n pairs */
  SPARSEPR_BUDGET_GLOBAL = 1       /* one budget of H_kv times that, shared by all KV heads of
                                      the call: mandatory cells stay per head, the other cells
                                      of all heads are ranked together by mass per unit cost
                                      (ties: smaller head, then smaller a G_K + b) and the
                                      longest prefix that fits is kept.  Needs
                                      sparsepr_workspace_size's workspace in sparsepr_route. */
} sparsepr_budget_mode;

/* What a cell costs the router (PSRR, execution paragraph: cells are indivisible units). */
typedef enum {
  SPARSEPR_COST_PAIRS = 0,         /* the method as read here: n_a n_b query-key pairs */
  SPARSEPR_COST_TILES = 1          /* the pairs of the block x block tiles the cell occupies,
                                      ceil(n_a / block) block x ceil(n_b / block) block, in the
                                      ranking and in the budget; route.pairs still reports the
                                      unpadded pairs */
} sparsepr_cost_mode;

/* Problem and hyper-parameters.  Defaults on the page: r_k = 48, r_q = 64, n_probe = 64,
 * rank = 16, lambda = 0.1 (PSRR, partition and probe-fit paragraphs); rho_exec is the
 * target total execution density rho_route + n_probe / n (PSRR, execution paragraph). */
typedef struct sparsepr_params {
  int32_t heads_q;       /* query heads Hq; Q is [Hq, n, d] */
  int32_t heads_kv;      /* KV heads Hkv; K, V are [Hkv, n, d]; query head h uses KV head h / g */
  int32_t n;             /* tokens */
  int32_t d;             /* head dimension (64 or 128) */
  int32_t dtype;         /* sparsepr_dtype of Q, K, V and the output */
  int32_t groups_q;      /* query groups G_Q */
  int32_t groups_k;      /* key groups G_K */
  int32_t r_k;           /* sampled queries = key response feature width */
  int32_t r_q;           /* cap on the query feature width (features use G_K <= r_q) */
  int32_t n_probe;       /* probe rows M per query head */
  int32_t rank;          /* output-subspace rank r */
  float lambda;          /* ridge penalty */
  float rho_exec;        /* target execution density (pairs / n^2, probes included) */
  int32_t block;         /* tile height in tokens; must be 64 */
  int32_t kmeans_iters;  /* Lloyd iterations before the final assignment */
  float softmax_scale;   /* 0 -> 1 / sqrt(d) */
  int32_t ablation;      /* sparsepr_ablation (0 = the method) */
  int32_t probe_mode;    /* sparsepr_probe_mode (0 = the method) */
  int32_t partition_mode;/* sparsepr_partition_mode (0 = the method) */
  int32_t budget_mode;   /* sparsepr_budget_mode (0 = per KV head) */
  int32_t cost_mode;     /* sparsepr_cost_mode (0 = pairs) */
  int32_t defer_kv_gather;/* 1: sparsepr_partition leaves k_gm and v_gm to sparsepr_gather_kv */
} sparsepr_params;

/* Partition outputs (all caller-allocated device buffers).  g = heads_q / heads_kv.
 * perm[p] is the token at group-major position p; offsets[b] is where group b starts. */
typedef struct sparsepr_partition_t {
  float* responses_s;        /* [Hkv, r_k, n] fp32: sampled-query responses S */
  float* responses_u;        /* [Hq, n, G_K] fp32: query responses to key centroids U */
  int32_t* exponents;        /* [Hkv, 2]: power-of-two exponents e_S, e_U */
  int32_t* key_labels;       /* [Hkv, n] */
  int32_t* key_centroids_int;/* [Hkv, G_K, r_k] integer feature centroids (final) */
  int32_t* key_perm;         /* [Hkv, n] */
  int32_t* key_offsets;      /* [Hkv, G_K + 1] */
  float* key_centroids;      /* [Hkv, G_K, d] fp32 mean key vector of each group */
  int8_t* query_features;    /* [Hkv, n, G_K] integer direction features in [-127, 127] */
  int32_t* query_labels;     /* [Hkv, n] */
  int32_t* query_centroids;  /* [Hkv, G_Q, G_K] centroids used by the final assignment */
  int32_t* query_perm;       /* [Hkv, n] */
  int32_t* query_offsets;    /* [Hkv, G_Q + 1] */
  void* q_gm;                /* [Hkv, n, g, d] dtype: Q in group-major order */
  void* k_gm;                /* [Hkv, n, d] dtype: K in group-major order */
  void* v_gm;                /* [Hkv, d, n_pad] dtype, n_pad = n rounded up to 16: V in group-major
                                order (follows K), stored transposed (d-major).  Element (d, p) is at
                                d * n_pad + s(p), where s swaps bits 2 and 3 of p (within each
                                16-key group the keys are stored as 0-3, 8-11, 4-7, 12-15);
                                positions n .. n_pad - 1 are zero. */
  float* query_coord_sum;    /* optional (NULL: not written), read only when g > 1: the head-summed
                                query coordinate that the query features quantise, fp32 as the
                                kernels formed it (ascending query head order).  Response
                                partition: [Hkv, n, G_K], the sum of responses_u over the KV
                                head's query heads; semantic partition: [Hkv, n, d], the summed
                                raw query rows.  With g = 1 the features quantise responses_u (or
                                the raw rows) directly and nothing is written here. */
} sparsepr_partition_t;

/* Route outputs.  Row a of the CSR lists the kept key groups of query group a,
 * ascending. */
typedef struct sparsepr_route_t {
  int32_t* row_ptr;          /* [Hkv, G_Q + 1] */
  int32_t* cols;             /* [Hkv, G_Q * G_K] (first row_ptr[G_Q] entries used) */
  uint64_t* kept_mask;       /* [Hkv, G_Q] bit b set when cell (a, b) is kept */
  int64_t* pairs;            /* [Hkv] routed query-key pairs per query head (unpadded) */
  uint64_t* cell_mass;       /* [Hkv, G_Q, G_K] fixed-point cell masses m_ab */
} sparsepr_route_t;

/* Probe and fit outputs. */
typedef struct sparsepr_fit_t {
  int32_t* probe_tokens;     /* [Hkv, n_probe] token index of each probe row */
  int32_t* probe_groups;     /* [Hkv, n_probe] query group of each probe row */
  double* probe_weights;     /* [Hkv, n_probe] group-coverage weights (sum n_probe) */
  float* o_dense;            /* [Hq, n_probe, d] exact probe rows over all keys */
  float* o_sparse;           /* [Hq, n_probe, d] probe rows over the kept cells */
  float* A;                  /* [Hq, d, R]  W V_r (zero beyond r_eff); R = rank, or n_probe
                                with SPARSEPR_ABLATE_RIDGE_ONLY */
  float* B;                  /* [Hq, R, d]  V_r^T (zero beyond r_eff) */
  float* c0;                 /* [Hq, d]        ybar - xbar A B */
  int32_t* r_eff;            /* [Hq] eigenpairs kept (lambda_k > 1e-8 lambda_1) */
  float* eig;                /* [Hq, rank + 1] leading eigenvalues of Yt Yt^T */
} sparsepr_fit_t;

/* Bytes of scratch workspace every entry point below needs for these params. */
sparsepr_status sparsepr_workspace_size(const sparsepr_params* params, size_t* bytes);

/* Response-coupled partition (PSRR, response-coupled partition paragraph), per KV head:
 * sample r_k query rows, S = Q_s K^T * scale, quantise to integer key features, online
 * k-means over keys (V follows K), key centroids in the original space, U = Q C^T *
 * scale per query head, integer response-direction features of the head-summed U,
 * online k-means over queries (one asymmetric pass), stable group-major permutations,
 * and the gathers of Q, K and V into group-major order.
 * q: [Hq, n, d]; k, v: [Hkv, n, d] (dtype, token order). */
sparsepr_status sparsepr_partition(const sparsepr_params* params, const void* q, const void* k,
                                   const void* v, const sparsepr_partition_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* The gathers of K and V into group-major order (k_gm, and v_gm transposed) from key_perm,
 * for a partition made with defer_kv_gather = 1, which leaves them out so that they can run
 * on another stream beside the route (only the attention and the probe stage read them).
 * k, v: [Hkv, n, d] (dtype, token order); writes part->k_gm and part->v_gm. */
sparsepr_status sparsepr_gather_kv(const sparsepr_params* params, const void* k, const void* v,
                                   const sparsepr_partition_t* part, void* stream);

/* Routing to the target execution density (PSRR, execution paragraph): fixed-point cell
 * masses from the size-weighted centroid softmax of every query row (summed over the
 * KV head's query heads), budget rho_exec n^2 - n_probe n pairs per head, one mandatory
 * heaviest cell per non-empty query group, the rest by mass per unit cost until the
 * budget is spent (budget_mode and cost_mode select the variants).  Reads responses_u,
 * query_labels, query_offsets, key_offsets; the workspace is used by the global budget
 * only (it may be NULL otherwise). */
sparsepr_status sparsepr_route(const sparsepr_params* params, const sparsepr_partition_t* part,
                               const sparsepr_route_t* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Block-sparse attention over the kept cells, renormalised over the kept K/V groups
 * (PSRR, execution paragraph).  Reads q_gm, k_gm, v_gm, offsets and the CSR.  After a
 * partition made with defer_kv_gather = 1, sparsepr_gather_kv must have run (ordered before
 * this call); until it has been called the call returns SPARSEPR_ERR_PARAM (the library
 * records deferred partitions by their k_gm buffer), since k_gm and v_gm would still hold
 * an earlier call's keys and values.
 * o_gm: [Hkv, n, g, d] fp32, group-major rows; lse: [Hkv, n, g] fp32 (natural log).
 * The workspace (sparsepr_workspace_size bytes, 256-byte aligned) holds the tile schedule
 * (each head's query groups longest first, and eight counters through which the last blocks
 * of each XCD's share claim their tiles, reset by every call) in a region disjoint from the
 * one sparsepr_probe_fit uses, so the two may run concurrently on one workspace. */
sparsepr_status sparsepr_attend(const sparsepr_params* params, const sparsepr_partition_t* part,
                                const sparsepr_route_t* route, float* o_gm, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* sparsepr_attend for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same attention with
 * the same arguments and results, but no workspace.  The tile schedule that sparsepr_attend
 * keeps in the workspace lives instead in a fixed 4 MiB device array inside the library, one
 * per GPU, held until the process ends; no call allocates or frees anything.  Limit: the
 * schedule needs 4 (2 (ceil(n g / 256) + G_Q) H_kv + 64 + H_kv) bytes for bf16 (nothing for
 * fp32); larger shapes return SPARSEPR_ERR_WORKSPACE before any launch.  Every call on one GPU
 * shares that GPU's array and overwrites it, so calls that overlap on one GPU (other streams,
 * other threads, replays of several graphs at once) race and must be ordered by the caller.
 * The first call on a device looks the array's address up (no allocation, no stream work). */
sparsepr_status sparsepr_attend_noalloc(const sparsepr_params* params, const sparsepr_partition_t* part,
                                        const sparsepr_route_t* route, float* o_gm, float* lse,
                                        void* stream);

/* Probe selection, exact probe rows and the fit (PSRR, probe-fit residual reconstruction
 * paragraph): n_probe rows per KV head stratified over query groups in radial order
 * about each group centroid, their dense and sparse outputs against all keys,
 * R = O_dense - O_sparse, the group-coverage-weighted ridge fit of R on O_sparse and
 * the rank-r subspace of the probe residuals.  q: [Hq, n, d] token order.  Reads k_gm and
 * v_gm: after a partition made with defer_kv_gather = 1, sparsepr_gather_kv must have run
 * (ordered before this call; until it has been called the call returns SPARSEPR_ERR_PARAM). */
sparsepr_status sparsepr_probe_fit(const sparsepr_params* params, const void* q,
                                   const sparsepr_partition_t* part, const sparsepr_route_t* route,
                                   const sparsepr_fit_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Write-back (PSRR, execution paragraph, where write-back is one of the timed parts of the
 * call; the correction is the probe-fit paragraph's affine map projected onto the rank-r
 * output subspace): o_hat = o + c0 + (o A) B for every row, probe rows replaced by their
 * exact dense output, inverse permutation to token order, cast to dtype.
 * o_gm: [Hkv, n, g, d] fp32 from sparsepr_attend; o: [Hq, n, d] dtype, token order. */
sparsepr_status sparsepr_apply(const sparsepr_params* params, const float* o_gm,
                               const sparsepr_partition_t* part, const sparsepr_fit_t* fit, void* o,
                               void* stream);

/* Block-sparse attention with the write-back fused into its epilogue: the fused call order
 * partition -> route -> probe_fit -> attend_apply produces the same output as the unfused
 * order (up to the rounding of the correction, which is formed from bf16 operands with
 * fp32 accumulation) without the fp32 group-major intermediate.  For bf16 the correction
 * o + c0 + (o A) B runs on the matrix cores inside the attention kernel (under GQA with A and
 * B split into a bf16 high part and remainder, the g query heads of a KV head corrected in
 * turn); for fp32 O_gm is formed in the workspace and the write-back follows.
 * Reads the partition, the route and the fit; o: [Hq, n, d] dtype, token order.  After a
 * partition made with defer_kv_gather = 1, sparsepr_gather_kv must have run first (until it
 * has been called the call returns SPARSEPR_ERR_PARAM). */
sparsepr_status sparsepr_attend_apply(const sparsepr_params* params, const sparsepr_partition_t* part,
                                      const sparsepr_route_t* route, const sparsepr_fit_t* fit, void* o,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Dense softmax attention O = softmax(Q K^T * scale) V on the same tile machinery (the
 * baseline; dense formula as in the lmnt.cn SparsePR article, section 2.1).  V is first
 * transposed into the workspace (part of the call), which also holds the eight tile-claim
 * counters of the sparse schedule, reset by every call.
 * q: [Hq, n, d]; k, v: [Hkv, n, d]; o: [Hq, n, d], all dtype and token order. */
sparsepr_status sparsepr_dense_attention(const sparsepr_params* params, const void* q,
                                         const void* k, const void* v, void* o,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Residual diagnostics (PSRR, partition paragraph: how much of the hard-drop residual is
 * an affine function of the sparse output, and the energy orthogonal to it; the page
 * compares these between its partition and a semantic one).  For every query head, over
 * all n rows: R = O_dense - O_sparse (O_sparse = the renormalised sparse attention of this
 * partition and route, before any correction) and the ordinary least-squares fit
 * R ~ c + O_sparse W (a 1e-9 relative guard on the normal equations' diagonal).
 *   out: [Hq, 4] float64 device buffer (8-byte aligned): ||R||_F^2, ||R - mean R||_F^2,
 *        ||R - (c + O_sparse W)||_F^2 (affine-orthogonal energy) and the explainable
 *        fraction 1 - orthogonal / centred.
 * Needs Q, K, V of the call and the partition and route outputs; the workspace
 * (sparsepr_diagnostics_workspace_size) holds fp32 dense and sparse outputs of every row,
 * so it is large (about 8 n d Hq bytes).  Not part of the timed call. */
sparsepr_status sparsepr_diagnostics_workspace_size(const sparsepr_params* params, size_t* bytes);
sparsepr_status sparsepr_residual_diagnostics(const sparsepr_params* params, const void* q, const void* k,
                                              const void* v, const sparsepr_partition_t* part,
                                              const sparsepr_route_t* route, double* out, void* workspace,
                                              size_t workspace_bytes, void* stream);

/* Support diagnostics (PSRR, support paragraph: a single query row keeps 90 % of its
 * attention mass on few keys, while queries that share one route must keep the union of
 * their supports).  For each query head h and each set of set_size query tokens:
 *   support of a row = the fewest keys whose softmax probabilities (scale from params)
 *   reach `mass` of the row's total, taken by decreasing score, ties by lower key index;
 *   row_support[h][s][i] = its size, shared_support[h][s] = size of the union over the set.
 *   sets:  [Hq, n_sets, set_size] int32 token indices (device); an index outside [0, n)
 *          marks that row invalid: its row_support is -1 and it is left out of the union.
 *   row_support [Hq, n_sets, set_size], shared_support [Hq, n_sets]: int32 (device).
 *   1 <= set_size <= 16, n_sets >= 0 (0: nothing to do), 0 < mass <= 1.
 * Scores f are fp32 dot products of the stored Q and K values; each key's probability
 * enters the decision as the 64-bit integer floor(2^40 exp((f - f_max) scale)), formed in
 * double precision from the fp32 scores, so keys below 2^-40 of the row's largest
 * probability carry no mass.  The workspace (sparsepr_support_workspace_size) holds
 * set_size * n fp32 scores for each of up to 512 concurrent (head, set) items; when
 * Hq * n_sets <= 512 it still holds them after the call, item i = h * n_sets + s at float
 * offset i * set_size * n as [set_size][n] (rows of invalid tokens unspecified).
 * Needs only params, Q and K (no partition).  Not part of the timed call. */
sparsepr_status sparsepr_support_workspace_size(const sparsepr_params* params, int n_sets, int set_size,
                                                size_t* bytes);
sparsepr_status sparsepr_support_diagnostics(const sparsepr_params* params, const void* q, const void* k,
                                             const int32_t* sets, int n_sets, int set_size, double mass,
                                             int32_t* row_support, int32_t* shared_support, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* sparsepr_status_string(sparsepr_status status);

#ifdef __cplusplus
}
#endif
#endif /* SPARSEPR_H */
