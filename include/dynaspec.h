/*
 * dynaspec.h -- C-ABI of the MI355X (gfx950) shortlisted draft head.
 *
 * The calls follow the DynaSpec pipeline: a router scores vocabulary
 * clusters from the draft hidden state, the top clusters under a
 * position-aware budget form the shortlist, the draft logits are a gathered
 * projection over only those rows of the LM head, the drafter samples from
 * the shortlist distribution, and the target verifies over the full
 * vocabulary by rejection sampling.  Sources (pages cited by title and
 * section):
 *   [A] "DynaSpec: Context-aware Dynamic Speculative Sampling for
 *       Large-Vocabulary Language Models", arXiv abstract page, Abstract.
 *   [S] papers.lunadong.com summary of DynaSpec, sections "Problem
 *       Definition", "Pipeline Flow", "System Modules", "Novel Architectural
 *       Elements", "Modeling / Key Hyperparameters".
 *   Speculative sampling (accept with min(1, p/q), residual max(0, p - q),
 *   bonus token) is the textbook algorithm of the speculative-decoding works
 *   that [A] builds on.
 *
 * Conventions for every call:
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or retains caller memory.  It keeps
 *     no state between calls apart from a per-device cache of the
 *     compute-unit count (a read-only device attribute) and, for
 *     ds_verify_reject_noalloc alone, its per-device scratch array.
 *   - Calls only enqueue work on the given stream(s) and return; nothing
 *     synchronises with the host.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and return DS_EINVAL / DS_EDTYPE / DS_ESHAPE.  A failed launch returns
 *     DS_EHIP.  Data-dependent errors (a shortlist over capacity, a cluster
 *     id out of range) are raised on the device into a caller-owned int32
 *     flag with atomicMax, so the caller zeroes it once and checks it after
 *     its own synchronisation.
 *   - bf16 tensors are raw bf16 (16-bit) arrays; fp32 is IEEE binary32.
 *   - Identical inputs give bit-identical outputs: no floating-point
 *     atomics, fixed reduction orders.
 *   - Shortlists are ragged (CSR) arrays: sl_off holds ABSOLUTE offsets into
 *     sl_ids; sl_off[0] is the base at which a call's shortlists start, so
 *     successive calls (draft positions) can append to one buffer.
 *   - Per-group float outputs (logits, q) use the same absolute offsets:
 *     the entry (group g, head row i, shortlist index j) lives at
 *     m*sl_off[g] + i*len_g + j, with len_g = sl_off[g+1] - sl_off[g].
 *   - Workspaces ("ws") are caller-owned device buffers of at least the size
 *     the matching *_workspace_bytes() query returns.  They must be
 *     zero-filled once before first use (the kernels leave them reusable)
 *     and must not be shared by calls that may run concurrently.
 */
#ifndef DYNASPEC_H
#define DYNASPEC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DS_OK = 0,
    DS_EINVAL = 1,    /* bad argument (null pointer, non-positive size, ...) */
    DS_EDTYPE = 2,    /* unsupported dtype / activation / budget kind       */
    DS_ESHAPE = 3,    /* sizes inconsistent or beyond the supported limits  */
    DS_ECAPACITY = 4, /* (device flag) shortlist longer than the capacity   */
    DS_EHIP = 5       /* a HIP launch or runtime call failed                */
} ds_status;

typedef enum { DS_F32 = 0, DS_BF16 = 1 } ds_dtype;
typedef enum { DS_RELU = 0, DS_SILU = 1 } ds_act;
typedef enum { DS_BUDGET_CLUSTERS = 0, DS_BUDGET_TOKENS = 1 } ds_budget_kind;

/* Limits checked on the host. */
#define DS_MAX_CLUSTERS 4096    /* M: clusters are ranked in LDS            */
#define DS_MAX_GROUPS 65535     /* G (and n for selection/build)            */
#define DS_MAX_HEAD_ROWS 256    /* m: head rows sharing one shortlist       */
#define DS_MAX_TREE_NODES 1024  /* m: drafted nodes of one verified tree    */

const char *ds_status_string(ds_status s);
const char *ds_version(void);

/*
 * Router / meta-classifier [S "System Modules: Router"; "Key
 * Hyperparameters: 2-layer MLP with ReLU"; "Problem Definition": its input is
 * the draft hidden state H_{t-1}]:
 *     z_i = act(sum_k W1[i][k] h[k] + b1[i]),  scores[c] = sum_i W2[c][i] z_i + b2[c]
 * dt      DS_F32 or DS_BF16: dtype of h, W1, b1, W2, b2.
 * n       rows; row `row` of h starts at h + row*ldh elements (ldh >= d).
 * d, r, M input width, hidden width, number of clusters.  d and r must be
 *         multiples of 8 (16-byte rows for bf16, 32-byte for fp32).
 * act     DS_RELU or DS_SILU.
 * W1 [r][d], b1 [r] or NULL, W2 [M][r], b2 [M] or NULL.
 * scores  [n][M] fp32 output (accumulation in fp32, z kept in fp32).
 * ws      >= ds_router_workspace_bytes(n, r) bytes (holds z; for n >= 8 it
 *         also holds the first layer's partial sums over 256-element windows
 *         of d: a batch of bf16 inputs runs that layer on the matrix cores,
 *         still bf16 products accumulated in fp32).
 */
size_t ds_router_workspace_bytes(int n, int r);
ds_status ds_router_score(hipStream_t s, ds_dtype dt, int n, int d, int r, int M, ds_act act,
                          const void *h, int64_t ldh, const void *W1, const void *b1,
                          const void *W2, const void *b2, float *scores, void *ws,
                          size_t ws_bytes);

/*
 * Top-cluster selection under a position-aware budget [A: the shortlist is
 * the union of the best-scoring clusters; S "Key Novelty" (position-aware budget) and "Key
 * Hyperparameters" (k_c(t) decays from k_0 to k_1)].  Per row, clusters are
 * ranked by (score descending, cluster id ascending); -0.0 ties with +0.0.
 *   DS_BUDGET_CLUSTERS: the first clamp(budget[row], 1, M) clusters.
 *   DS_BUDGET_TOKENS:   the shortest prefix whose total size reaches
 *                       max(budget[row], 1) tokens (all M if none does).
 * scores [n][M] fp32 (NaN is invalid input: the result is then unspecified
 * but every index stays in range); cluster_size [M] int32 >= 0;
 * budget [n] int32.
 * Outputs: sel [n][M] int32 ranked ids (entries past n_sel[row] are -1),
 * n_sel [n] int32, sl_len [n] int32 (sum of the selected sizes).
 * Limits: 1 <= M <= DS_MAX_CLUSTERS, 1 <= n <= DS_MAX_GROUPS.
 */
ds_status ds_select_clusters(hipStream_t s, int n, int M, const float *scores,
                             const int32_t *cluster_size, ds_budget_kind kind,
                             const int32_t *budget, int32_t *sel, int32_t *n_sel,
                             int32_t *sl_len);

/*
 * Cluster index, built once per clustering (it depends only on cluster_of):
 * the vocabulary is cut into chunks of 4096 token ids, and
 * index[k][c] (k = 0..nchunks, nchunks = ceil(V/4096)) is the number of
 * members of cluster c among token ids below 4096*k, so index[nchunks][c]
 * is the size of cluster c.  int32 [(nchunks+1)][M], caller-owned, of
 * ds_cluster_index_bytes(M, V) bytes.  Entries of cluster_of outside
 * [0, M) are not counted and raise DS_EINVAL in *err_flag (may be NULL).
 * The shortlist build uses it to place every chunk's tokens directly.
 */
size_t ds_cluster_index_bytes(int M, int V);
ds_status ds_cluster_index(hipStream_t s, int M, int V, const int32_t *cluster_of,
                           int32_t *index, int32_t *err_flag);

/*
 * Shortlist = union of the selected clusters' member tokens, in ascending
 * token id [A: the shortlist is the union of the selected clusters;
 * S "Problem Definition": output V_S].
 * sel [n][M], n_sel [n] as written by ds_select_clusters; cluster_of [V]
 * int32 maps every token to its cluster; index is its cluster index
 * (ds_cluster_index of the same cluster_of).
 * sl_off [n+1] int64: sl_off[0] is READ (base offset, e.g. the end of the
 * previous call's shortlists), sl_off[1..n] are written.
 * sl_ids [capacity] int32: entries sl_off[0] .. sl_off[n]-1 are written.
 * Offsets never exceed `capacity`; entries beyond it are dropped and
 * *err_flag raised to DS_ECAPACITY.  Cluster ids in sel outside [0, M) are
 * skipped and raise DS_EINVAL (cluster_of entries outside [0, M) are skipped;
 * ds_cluster_index reports them).  err_flag may be NULL.
 * ws >= ds_build_workspace_bytes(n, V) bytes.
 */
size_t ds_build_workspace_bytes(int n, int V);
ds_status ds_build_shortlist(hipStream_t s, int n, int M, int V, const int32_t *sel,
                             const int32_t *n_sel, const int32_t *cluster_of,
                             const int32_t *index, int64_t capacity, int64_t *sl_off,
                             int32_t *sl_ids, int32_t *err_flag, void *ws, size_t ws_bytes);

/*
 * Gathered LM head [S "System Modules: Gathered LM Head" (projects hidden
 * states only onto the shortlist rows); "Novel Architectural Elements"
 * (index-select fused with the GEMM, no gathered copy of W); "Comparison to
 * Prior Work" (O(|V_S| d) instead of O(|V| d))]:
 *     logits[g][i][j] = sum_k W[S_g[j]][k] * h[g][i][k]
 * dt      dtype of W and h (fp32 accumulation, fp32 output).
 * W       [V][d], one token's row contiguous; d a multiple of 8, and a row
 *         at most 16 KB (d <= 8192 bf16, <= 4096 fp32).
 * G, m    groups (shortlists) and head rows per group (1 <= m <= 256).
 * h       row (g, i) at h + g*ldh_g + i*d elements (ldh_g >= m*d).
 * sl_off  [G+1] absolute offsets, sl_ids the token ids.
 * max_rows host-side upper bound of sl_off[G] - sl_off[0]; sizes the grid
 *         (rows past the true total are skipped on the device).
 * logits  output, entry (g, i, j) at m*sl_off[g] + i*len_g + j.
 * ws      >= ds_head_workspace_bytes(G, m, V) bytes (may be NULL when that
 *         is 0).
 * Token ids outside [0, V) give NaN.  Kernel choice: bf16 heads with
 * G >= 8 single-row groups (batched drafting) walk W once in token order on
 * the matrix cores and write only shortlisted (row, group) pairs -- this
 * path requires every shortlist to be ascending; bf16 heads with m >= 8
 * (tree drafting) run a gathered matrix-core GEMM per group (shortlists in
 * any order; ascending ones let rows shared by several groups be read from
 * HBM once); everything else streams the shortlisted rows as a GEMV.
 */
size_t ds_head_workspace_bytes(int G, int m, int V);
ds_status ds_gathered_lm_head(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int G,
                              int m, const void *h, int64_t ldh_g, const int64_t *sl_off,
                              const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                              size_t ws_bytes);
/*
 * Same as ds_gathered_lm_head; start / stop (caller-created HIP events with
 * timing enabled, either may be NULL) are stamped at the start of the first
 * and the end of the last kernel the head launches, for measuring the head's
 * own execution time inside a longer sequence.
 */
ds_status ds_gathered_lm_head_timed(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int G,
                                    int m, const void *h, int64_t ldh_g, const int64_t *sl_off,
                                    const int32_t *sl_ids, int64_t max_rows, float *logits,
                                    void *ws, size_t ws_bytes, hipEvent_t start, hipEvent_t stop);

/*
 * Static-shortlist slab [A on FR-Spec / VocabTrim: a fixed, frequency-ranked
 * shortlist; S "Comparison to Prior Work", "Evaluation Highlights" (a static
 * list of about 32K tokens)]: out[i][k] = W[ids[i]][k] for i < n, a plain
 * copy, so that a fixed list's head can run over contiguous rows (pass the
 * slab as W with ids 0..n-1) instead of gathering.
 * W [V][d] (dt), ids [n] int32, out [n][d] (dt), both 16-byte aligned;
 * d a multiple of 8.  A row whose id lies outside [0, V) is filled with quiet
 * NaN.  n = 0 enqueues nothing.
 */
ds_status ds_pack_rows(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int64_t n,
                       const int32_t *ids, void *out);

/*
 * Spherical k-means over the rows of the LM head, the offline clustering the
 * router selects from [S "Key Novelty": clusters from the semantic
 * similarity of LM-head weights; "Modeling / Key Hyperparameters":
 * spherical k-means; "Key Terms": clusters by cosine similarity].  The
 * algorithm is the published one (Dhillon and Modha, concept
 * decompositions): assign each unit row x_y = w_y / |w_y| to the unit
 * centroid of largest cosine, then replace each centroid by the normalised
 * sum of its rows.  W is [V][d] bf16, 16-byte aligned.  All three calls are
 * deterministic (no floating-point atomics).
 *
 * ds_kmeans_inv_norms: inv_norm[y] = 1 / |w_y| (fp64 sums, fp32 result; 0 for
 * an all-zero row).  d a multiple of 8, at most 8192.
 */
ds_status ds_kmeans_inv_norms(hipStream_t s, int V, int d, const void *W, float *inv_norm);
/*
 * ds_kmeans_assign: assign[y] = argmax_c w_y . C[c] (the row norm does not
 * change the argmax) over bf16 unit centroids C [M][d], ties to the lower
 * c; score[y] = that dot product (bf16 products, fp32 accumulation on the
 * matrix cores).  d a multiple of 64, at most 8192; M <= DS_MAX_CLUSTERS.
 * ws >= ds_kmeans_assign_workspace_bytes(V) bytes.  start / stop (may be
 * NULL): timing events stamped at the contraction kernel's own start and end.
 */
size_t ds_kmeans_assign_workspace_bytes(int V);
ds_status ds_kmeans_assign(hipStream_t s, int V, int d, const void *W, int M, const void *C,
                           int32_t *assign, float *score, void *ws, size_t ws_bytes,
                           hipEvent_t start, hipEvent_t stop);
/*
 * ds_kmeans_update: for every cluster c, s_c = sum over rows y with
 * assign[y] = c, in ascending y, of w_y * inv_norm[y] (fp64); C_out[c] =
 * s_c / |s_c| as fp32 and C_out_bf16[c] its bf16 rounding (nearest-even),
 * the centroids the next ds_kmeans_assign reads.  A cluster without rows
 * keeps C_prev[c].  size[c] = its row count; norm[c] = |s_c| (0 when
 * empty), whose sum is the objective sum_y x_y . C_out[assign[y]].  Labels
 * outside [0, M) are skipped and raise DS_EINVAL in *err_flag (may be
 * NULL).  d a multiple of 8, at most 8192; M <= DS_MAX_CLUSTERS.
 * C_prev, C_out [M][d] fp32; C_out_bf16 [M][d] bf16; norm [M] fp64.
 * ws >= ds_kmeans_update_workspace_bytes(V, d, M) bytes.
 */
size_t ds_kmeans_update_workspace_bytes(int V, int d, int M);
ds_status ds_kmeans_update(hipStream_t s, int V, int d, const void *W, const float *inv_norm, int M,
                           const int32_t *assign, const float *C_prev, float *C_out,
                           void *C_out_bf16, int32_t *size, double *norm, int32_t *err_flag,
                           void *ws, size_t ws_bytes);

/*
 * Draft proposal from the shortlist distribution [A; S "Pipeline Flow"].
 * Per row (g, i), q = softmax(logits / temperature) over S_g computed in
 * fp64, and token = S_g[j*] with j* the first index whose running sum of
 * exp((l_j - max)/T) exceeds u[row] * (their total) (if rounding leaves none,
 * the last index with non-zero mass).  temperature == 0 gives the argmax
 * (ties to the lowest index) with a one-hot q.  Empty rows give token -1.
 * u [G*m] fp32 in [0, 1); token [G*m] int32; q in the logits layout.
 * max_len  host-side bound on every group's shortlist length (sizes the
 *          grid; 1 <= max_len <= 2^20).  Longer rows give unspecified
 *          results (memory accesses stay in bounds).
 * ws       >= ds_sample_workspace_bytes(G, m, max_len) bytes.
 */
size_t ds_sample_workspace_bytes(int G, int m, int64_t max_len);
ds_status ds_shortlist_sample(hipStream_t s, int G, int m, const int64_t *sl_off,
                              const int32_t *sl_ids, const float *logits, float temperature,
                              const float *u, int64_t max_len, int32_t *token, float *q, void *ws,
                              size_t ws_bytes);

/*
 * ds_shortlist_sample without writing q, for temperature > 0 [same passages
 * as ds_shortlist_sample]: the same token per row, and per row its
 * statistics in place of q, qstats[row] = {M, rZ}, such that the q value
 * ds_shortlist_sample writes for logit l_j of the row is exactly
 * (float)(exp((l_j - M) / T) * rZ) evaluated as the library does (fp64
 * exponent); the verifiers' _qstats forms recompute q that way, bit for
 * bit.  Empty rows give token -1 and rZ = 0.  temperature must be > 0 (else
 * DS_EINVAL); other arguments, limits and the workspace as
 * ds_shortlist_sample.  Writes G*m tokens and G*m statistics, not the
 * sum over rows of |S_g| q values.
 */
typedef struct {
    float M;
    int32_t pad;
    double rZ;
} ds_qstats;
ds_status ds_shortlist_sample_stats(hipStream_t s, int G, int m, const int64_t *sl_off,
                                    const int32_t *sl_ids, const float *logits,
                                    float temperature, const float *u, int64_t max_len,
                                    int32_t *token, ds_qstats *qstats, void *ws,
                                    size_t ws_bytes);

/*
 * Full-vocabulary target distribution p = softmax(target logits) per row
 * (fp64 exponent and sum, fp32 output) [A: the target verifies over the full
 * vocabulary].  logits and p are [rows][V] fp32, V <= 2^20.
 * ws >= ds_softmax_workspace_bytes(rows, V) bytes.
 */
size_t ds_softmax_workspace_bytes(int rows, int V);
ds_status ds_target_softmax(hipStream_t s, int rows, int V, const float *logits, float *p,
                            void *ws, size_t ws_bytes);

/*
 * Rejection-sampling verification over the full vocabulary, which keeps the
 * emitted tokens distributed exactly as the target [A: the target checks the
 * drafts against its whole vocabulary, so the output is exact; S
 * "Pipeline Flow: Rejection Sampling Verification"].  For sequence b:
 *   for t < T: x = draft[t][b] (shortlist row t*B + b, ascending token ids,
 *   q in the sampler's layout with m = 1, q_t(x) = 0 off the shortlist);
 *   accept iff (double)u_acc[t][b] * q_t(x) < p_t(x).  At the first
 *   rejection, draw from max(0, p_t - q_t) over all V (from p_t if that has
 *   no mass) with u_fin[b] by the inverse CDF and stop; if all T are
 *   accepted, draw the bonus token from p_T with u_fin[b].
 * p [B][T+1][V] fp32 target probabilities.  Outputs n_acc [B] in [0, T] and
 * out [B][T+1] (the first n_acc+1 entries are the emitted tokens, the rest
 * -1).  Limits: 1 <= T <= 64, V <= 2^20.
 * ws >= ds_verify_workspace_bytes(B, T, V) bytes.
 */
size_t ds_verify_workspace_bytes(int B, int T, int V);
ds_status ds_verify_reject(hipStream_t s, int B, int T, int V, const int32_t *draft,
                           const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                           const float *p, const float *u_acc, const float *u_fin,
                           int32_t *n_acc, int32_t *out, void *ws, size_t ws_bytes);

/*
 * ds_verify_reject from the target's logits instead of its probabilities
 * [same passages as ds_verify_reject].  logits [B][T+1][V] fp32; every
 * p_t(y) the verification reads is the value ds_target_softmax would write
 * for that row (the same segment statistics, row normaliser and rounding),
 * so the outputs equal ds_target_softmax followed by ds_verify_reject, bit
 * for bit, without writing or reading the B*(T+1)*V probabilities.  Limits
 * as ds_verify_reject, and B*(T+1) <= 65535 (else DS_ESHAPE).
 * ws >= ds_verify_logits_workspace_bytes(B, T, V) bytes (caller-owned, no
 * state kept between calls).
 */
size_t ds_verify_logits_workspace_bytes(int B, int T, int V);
ds_status ds_verify_reject_logits(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                  const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                  const float *logits, const float *u_acc, const float *u_fin,
                                  int32_t *n_acc, int32_t *out, void *ws, size_t ws_bytes);

/*
 * ds_verify_reject_logits with q given by the draft logits and their rows'
 * statistics instead of the q array [same passages as ds_verify_reject]:
 * draft_logits in the sampler's layout (m = 1), qstats [T*B] from
 * ds_shortlist_sample_stats over them with the same temperature (> 0).
 * Every q value the verification reads is recomputed from its logit and row
 * statistics, which gives the value ds_shortlist_sample writes, so the
 * outputs equal ds_verify_reject_logits given that q, bit for bit.  Limits
 * and workspace as ds_verify_reject_logits.
 */
ds_status ds_verify_reject_logits_qstats(hipStream_t s, int B, int T, int V,
                                         const int32_t *draft, const int64_t *sl_off,
                                         const int32_t *sl_ids, const float *draft_logits,
                                         const ds_qstats *qstats, float temperature,
                                         const float *logits, const float *u_acc,
                                         const float *u_fin, int32_t *n_acc, int32_t *out,
                                         void *ws, size_t ws_bytes);

/*
 * Allocation-free ds_verify_reject, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics, limits and outputs as
 * ds_verify_reject, without the workspace: the kernels' scratch lives in a
 * static device array of DS_NOALLOC_SCRATCH_BYTES that every GPU the library
 * runs on holds until the process ends (its address is looked up once per
 * device, on that device's first call; the current device must be the
 * stream's).  The call allocates nothing.  It needs
 * ds_verify_workspace_bytes(B, T, V) <= DS_NOALLOC_SCRATCH_BYTES (about
 * B * ceil(V / 1024) <= 1040000), else DS_ESHAPE.  All calls on one GPU share
 * that GPU's array, so calls that may overlap on one GPU (other streams,
 * other threads) race and give wrong results; serialise them.
 */
#define DS_NOALLOC_SCRATCH_BYTES (8u << 20)
ds_status ds_verify_reject_noalloc(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                   const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                   const float *p, const float *u_acc, const float *u_fin,
                                   int32_t *n_acc, int32_t *out);

/*
 * Tree verification by multi-step speculative sampling, which keeps the
 * emitted tokens distributed exactly as the target (SpecInfer, "Accelerating
 * Generative Large Language Model Serving with Tree-based Speculative
 * Inference and Verification", a reference of the DySpec page; the pages
 * draft trees [tree-shaped workload] and verify over the full vocabulary
 * [A], so the tree is verified by the published tree form of the
 * rejection rule).  Per sequence b the tree has nodes 0..m: node 0 the root
 * (the last emitted token), nodes 1..m drafted, drafted node i described at
 * index i-1 of the [B][m] arrays:
 *   parent  its parent in [0, i) (any other value detaches the node);
 *   token   its token, drawn from its own proposal q_i;
 *   u_acc   its acceptance uniform in [0, 1);
 *   q_i     row i-1 of group b in the sampler's layout:
 *           q[m*sl_off[b] + (i-1)*len_b + j] over shortlist b
 *           (sl_ids[sl_off[b] .. sl_off[b+1]), ascending distinct ids;
 *           the sampler's output with G = B and m rows per group).
 * p [B][m+1][V] fp32 target probabilities at every node (row 0: the root).
 * From u = 0, the children c of u (parent == u) are tried in increasing
 * order against a residual r that starts as p_u: accept iff
 * u_acc * q_c(x_c) < r(x_c); after a rejection r <- max(0, r - q_c) / sum
 * over all V (back to p_u if that has no mass).  An accepted child becomes
 * u; when no child is accepted, one token is drawn from r with u_fin[b] by
 * the inverse CDF and the sequence stops.  The first test at a node is
 * exact (fp32 values compared in fp64); later tests and the draw use fp64
 * sums whose order differs from a sequential sum by rounding only.
 * Outputs: n_acc [B] accepted nodes (-1: the sequence's shortlist is longer
 * than max_len or has a negative length, its other outputs -1);
 * path [B][m] the accepted node numbers, then -1; out [B][m+1] the accepted
 * tokens, the final draw, then -1.
 * max_len  host-side bound on every sequence's shortlist length.
 * Limits: 1 <= m <= DS_MAX_TREE_NODES, V <= 2^20, B <= DS_MAX_GROUPS,
 * max_len <= 2^24.  Unsorted or repeated shortlist ids give unspecified
 * results (memory accesses stay in bounds).  Two kernels on stream s.
 * ws >= ds_verify_tree_workspace_bytes(B, m, V, max_len) bytes; no
 * initialisation needed.
 */
size_t ds_verify_tree_workspace_bytes(int B, int m, int V, int64_t max_len);
ds_status ds_verify_tree(hipStream_t s, int B, int m, int V, const int32_t *parent,
                         const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                         const float *q, const float *p, const float *u_acc, const float *u_fin,
                         int64_t max_len, int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                         size_t ws_bytes);

/*
 * ds_verify_tree from the target's logits instead of its probabilities
 * [same passages as ds_verify_tree].  logits [B][m+1][V] fp32; every target
 * value the walk reads is the one ds_target_softmax would write for that
 * row (the same segment statistics, row normaliser and rounding), so the
 * outputs equal ds_target_softmax followed by ds_verify_tree, bit for bit,
 * without writing or reading the B*(m+1)*V probabilities.  Limits as
 * ds_verify_tree, and B*(m+1) <= 65535 (else DS_ESHAPE).
 * ws >= ds_verify_tree_logits_workspace_bytes(B, m, V, max_len) bytes.
 */
size_t ds_verify_tree_logits_workspace_bytes(int B, int m, int V, int64_t max_len);
ds_status ds_verify_tree_logits(hipStream_t s, int B, int m, int V, const int32_t *parent,
                                const int32_t *token, const int64_t *sl_off,
                                const int32_t *sl_ids, const float *q, const float *logits,
                                const float *u_acc, const float *u_fin, int64_t max_len,
                                int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                size_t ws_bytes);

/*
 * ds_verify_tree_logits with q given by the draft logits and their rows'
 * statistics instead of the q array [same passages as ds_verify_tree]:
 * draft_logits in the sampler's layout (group b, head row = node), qstats
 * [B*m] from ds_shortlist_sample_stats over them with the same temperature
 * (> 0).  The outputs equal ds_verify_tree_logits given the q that
 * ds_shortlist_sample writes, bit for bit.  Limits and workspace as
 * ds_verify_tree_logits.
 */
ds_status ds_verify_tree_logits_qstats(hipStream_t s, int B, int m, int V,
                                       const int32_t *parent, const int32_t *token,
                                       const int64_t *sl_off, const int32_t *sl_ids,
                                       const float *draft_logits, const ds_qstats *qstats,
                                       float temperature, const float *logits,
                                       const float *u_acc, const float *u_fin, int64_t max_len,
                                       int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                       size_t ws_bytes);

/*
 * Dense LM head of the full drafter over every token, the O(|V| d)
 * projection the shortlist avoids [S "Comparison to Prior Work": EAGLE's
 * O(|V| d) head; "Modeling": the full drafter whose top-L gives the
 * router's training labels]:  logits[i][y] = sum_k W[y][k] h[i][k].
 * bf16 only (fp32 accumulation on the matrix cores); W [V][d], h [n][d]
 * contiguous rows; logits [n][V] fp32 with row stride ldl >= V.  d a
 * multiple of 64, at most 8192.  events (optional, host array of 2
 * caller-created HIP events with timing) are stamped at the kernel's own
 * start and end.
 */
ds_status ds_dense_lm_head(hipStream_t s, int V, int d, const void *W, int n, const void *h,
                           float *logits, int64_t ldl, hipEvent_t *events);

/*
 * Router training labels [S "Modeling": binary cross entropy over clusters,
 * a cluster's label positive when it holds a token in the top-L of the full
 * drafter].  Row i of logits (V fp32 values of the full drafter -- the dense
 * head over all V, e.g. ds_gathered_lm_head with the shortlist 0..V-1 --
 * row stride ldl) orders its tokens by (logit desc, id asc); the first
 * min(L, V) are its top-L; labels[i][c] = 1 iff one of them lies in cluster
 * c, else 0 (ids whose cluster is outside [0, M) mark nothing).  NaN logits
 * are invalid input.  labels [n][M] uint8.  One workgroup per row, no
 * workspace.  Limits: 1 <= M <= DS_MAX_CLUSTERS, L >= 0, V >= 1.
 */
ds_status ds_router_labels(hipStream_t s, int n, int V, int M, int L, const float *logits,
                           int64_t ldl, const int32_t *cluster_of, uint8_t *labels);

/*
 * One plain SGD step of the router on a batch [S "Modeling": supervised
 * multi-label classification, binary cross entropy over clusters; the
 * router is the 2-layer MLP of ds_router_score]:
 *   a = W1 h + b1, z = act(a), s = W2 z + b2
 *   loss = 1/(n M) sum_{i,c} [log(1 + e^s_ic) - y_ic s_ic]
 *   g_s = (sigmoid(s) - y)/(n M); dW2 = g_s^T z, db2 = sum_i g_s;
 *   g_a = (g_s W2) * act'(a) (ReLU' = 0 at 0); dW1 = g_a^T h, db1 = sum_i g_a
 *   every parameter p <- p - lr * dp (all gradients from the old values).
 * Fields: h [n][d] (row stride ldh) in h_dtype (fp32 or bf16 bits); labels
 * [n][M] uint8 (0 or 1); W1 [r][d], b1 [r], W2 [M][r], b2 [M] fp32, updated
 * in place; dW1, db1, dW2, db2 fp32 gradient outputs of the same shapes;
 * loss one double; every pointer device memory.  Arithmetic fp32 (each dot
 * product summed in ascending index order; the two forward products, the
 * gradient through act' and dW2 in up to sixteen ascending k chunks whose
 * sums are then added in chunk order), the loss summed in fp64; results are
 * reproducible bit for bit.  ws >= ds_router_train_workspace_bytes(n, r, M).
 */
typedef struct {
    int n, d, r, M;
    ds_act act;
    ds_dtype h_dtype;
    const void *h;
    int64_t ldh;
    const uint8_t *labels;
    float lr;
    float *W1, *b1, *W2, *b2;
    float *dW1, *db1, *dW2, *db2;
    double *loss;
    void *ws;
    size_t ws_bytes;
} ds_router_train_args;
size_t ds_router_train_workspace_bytes(int n, int r, int M);
ds_status ds_router_train_step(hipStream_t s, const ds_router_train_args *a);

/*
 * One chain-drafting step over T positions for B sequences, with the router
 * on its own stream, overlapped with the head [A: the router runs beside the
 * drafter on concurrent streams to hide its cost; S "Novel Architectural
 * Elements": router on a separate stream].  For each position t:
 *   router_stream: router(h[:, t]) -> select(budget[t]) -> build (appending
 *                  to the shortlist buffer) -> event
 *   head_stream:   wait(event) -> gathered head(h[:, t+1]) -> sample(u_draft[t])
 * The router of position t needs H_{t-1} = h[:, t], which a drafter
 * produces from the token sampled at position t-2; so for t >= 1
 * router_stream waits for an event recorded on head_stream right after the
 * sampler of position t-2 (at the start for t = 1), and the router,
 * selection and build of position t run while the head and sampler of
 * position t-1 work.  Rows are position-major (row t*B + b), the
 * layout ds_verify_reject reads.  With B >= 8 bf16 sequences the build also
 * writes each shortlist's 32-token tile index (first position and
 * membership mask per tile, two slots of the workspace used alternately),
 * so the head walks W once on the matrix cores without an index pass of
 * its own; the logits are those of ds_gathered_lm_head.  That head keeps
 * every compute unit busy, so kernels beside it wait for its workgroups to
 * retire: in this mode the two router layers of position t+1 run on
 * head_stream just before head t (h[:, t+1] exists then), and only the
 * selection and build of position t+1 run on router_stream beside head t.
 * When B <= 64 and the second layer's k-window partial sums of a position
 * fit 2 MB, head_stream stops at those partials and the selection adds them
 * (in window order, then b2, as ds_router_score does; the same scores are
 * written), so the layer's finishing pass leaves head_stream.  Every
 * pointer is a device pointer except max_rows, max_len, W_pos, head_events
 * and sync_events (host arrays).  On return all work is enqueued and
 * head_stream waits for everything enqueued on router_stream.
 * Required field:
 *   sync_events  host array [2T+1] of caller-created HIP events on the
 *                streams' device (hipEventDisableTiming is enough), used to
 *                order the two streams; a call records and waits on them, so
 *                two calls that may be enqueued concurrently need their own
 *                arrays.  The caller destroys them (after the enqueued work,
 *                or after ds_capture_end when the call was captured).
 * Optional fields:
 *   W_pos        host array [T] of head matrices, one per position (drafters
 *                with a separate head per position, or copies of one head on
 *                different memory); NULL means W at every position.
 *   head_events  host array [2T] of caller-created HIP events (created with
 *                timing enabled); when non-NULL, events 2t and 2t+1 are
 *                stamped at the start of the first and the end of the last
 *                head kernel of position t (the kernels' own begin and end,
 *                so hipEventElapsedTime gives the head's execution time).
 *   qstats       [T*B] row statistics; when q is NULL (temperature > 0) the
 *                sampler writes these instead of q, as
 *                ds_shortlist_sample_stats does (the same tokens), for
 *                ds_verify_reject_logits_qstats.  One of q and qstats is
 *                required.
 */
typedef struct {
    int B, T, V, d, r, M;
    ds_dtype dtype;
    ds_act act;
    ds_budget_kind budget_kind;
    float temperature;
    const void *W;              /* [V][d]                          */
    const void *W1, *b1, *W2, *b2;
    const int32_t *cluster_of;  /* [V]                             */
    const int32_t *cluster_index; /* ds_cluster_index of cluster_of */
    const int32_t *cluster_size;/* [M]                             */
    const void *h;              /* [B][T+1][d]                     */
    const int32_t *budget;      /* [T][B]                          */
    const float *u_draft;       /* [T][B]                          */
    int64_t capacity;           /* elements of sl_ids              */
    const int64_t *max_rows;    /* HOST [T]: bound on rows per position */
    const int64_t *max_len;     /* HOST [T]: bound on one row's length  */
    float *scores;              /* [T][B][M]                       */
    int32_t *sel;               /* [T][B][M]                       */
    int32_t *n_sel, *sl_len;    /* [T][B]                          */
    int64_t *sl_off;            /* [T*B+1], sl_off[0] read as base */
    int32_t *sl_ids;            /* [capacity]                      */
    float *logits;              /* [capacity]                      */
    float *q;                   /* [capacity], or NULL: qstats     */
    int32_t *token;             /* [T][B]                          */
    int32_t *err_flag;          /* 1 int32 or NULL                 */
    void *ws;                   /* ds_draft_chain_workspace_bytes  */
    size_t ws_bytes;
    const void *const *W_pos;   /* HOST [T] or NULL                */
    hipEvent_t *head_events;    /* HOST [2T] or NULL               */
    hipEvent_t *sync_events;    /* HOST [2T+1], required           */
    ds_qstats *qstats;          /* [T][B], used when q is NULL     */
} ds_draft_chain_args;

size_t ds_draft_chain_workspace_bytes(int B, int T, int V, int r, int64_t max_len);
ds_status ds_draft_chain(hipStream_t head_stream, hipStream_t router_stream,
                         const ds_draft_chain_args *a);

/*
 * HIP graph capture of any sequence of the calls above, so a whole draft
 * step (about ten launches per position) is replayed with one host call.
 * ds_capture_begin starts capturing `s` (relaxed mode); every ds_* call made
 * on `s` (and the router stream that ds_draft_chain forks from it) until
 * ds_capture_end is recorded instead of executed; ds_capture_end
 * instantiates the graph.  Replays use the pointers captured: the buffers
 * must stay allocated and every call must be valid to repeat (the library's
 * calls are: nothing is accumulated across replays).  The kernels record no
 * memset nodes.  ds_graph_destroy releases the graph (host-side objects).
 */
typedef struct ds_graph_s *ds_graph;
ds_status ds_capture_begin(hipStream_t s);
ds_status ds_capture_end(hipStream_t s, ds_graph *out);
ds_status ds_graph_launch(ds_graph g, hipStream_t s);
ds_status ds_graph_destroy(ds_graph g);

#ifdef __cplusplus
}
#endif

#endif /* DYNASPEC_H */
