/*
 * CPU oracle for the DynaSpec draft-side shortlisted LM head.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * definition that the HIP library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the
 * product path never does, and the two share no code.
 *
 * Sources (the pages are cited by title and section):
 *   [A]  "DynaSpec: Context-aware Dynamic Speculative Sampling for
 *        Large-Vocabulary Language Models", arXiv abstract page, Abstract.
 *   [S]  papers.lunadong.com summary of DynaSpec: sections "Problem
 *        Definition", "Pipeline Flow", "System Modules", "Novel
 *        Architectural Elements", "Modeling / Key Hyperparameters",
 *        "Comparison to Prior Work".
 *   Speculative sampling itself (accept with min(1, p/q), resample from the
 *   normalised residual max(0, p - q), bonus token from the last target
 *   position) is the textbook algorithm of the two speculative-decoding
 *   works that [A] builds on ("Fast Inference from Transformers via
 *   Speculative Decoding"; "Accelerating Large Language Model Decoding with
 *   Speculative Sampling").
 *
 * Arithmetic: bf16 inputs are widened to fp32 exactly and then to double;
 * every sum runs in double, in ascending index order; exp is libm's double
 * exp.  Results that the pages store as fp32 are rounded once at the end.
 *
 * Index conventions (shared with the library's C-ABI, restated here):
 *   - shortlist offsets sl_off are ABSOLUTE element offsets into sl_ids;
 *     sl_off[0] is an input (the base), build writes sl_off[1..n].
 *   - logits/q for group g, row i, entry j live at m*sl_off[g] + i*len_g + j.
 *   - verification rows are position-major: row = t*B + b.
 *
 * Parity status: every function is pinned by tests that do not retype its
 * formula (library GEMV in float64, brute force, closed forms, quadrature,
 * exact enumeration); see the oracle test module.  The pages print no
 * numeric example for any step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL 1
#define OR_ECAPACITY 4

#define TIE_REL 1e-12 /* a CDF boundary closer than this (relative) is a tie */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* element idx of an array that holds fp32 (dtype 0) or bf16 bits (dtype 1) */
static double load_elem(int dtype, const void *base, int64_t idx)
{
    if (dtype == 1)
        return bf16_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

static double activation(int act, double x)
{
    if (act == 0)
        return x > 0.0 ? x : 0.0;          /* ReLU */
    return x / (1.0 + exp(-x));             /* SiLU */
}

/*
 * Router / meta-classifier [S "System Modules: Router"; "Key
 * Hyperparameters: 2-layer MLP with ReLU"; "Problem Definition": input is the
 * draft hidden state H_{t-1}].  Two-layer MLP, one score per cluster:
 *   z_i = act(sum_k W1[i][k] h[k] + b1[i]),  s_c = sum_i W2[c][i] z_i + b2[c].
 * h row `row` starts at h + row*ldh (elements).  b1/b2 may be NULL.
 */
void oracle_router_score(int dtype, int n, int d, int r, int M, int act,
                         const void *h, int64_t ldh, const void *W1,
                         const void *b1, const void *W2, const void *b2,
                         float *scores)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)r);
    for (int row = 0; row < n; ++row) {
        for (int i = 0; i < r; ++i) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += load_elem(dtype, W1, (int64_t)i * d + k) *
                       load_elem(dtype, h, (int64_t)row * ldh + k);
            if (b1)
                acc += load_elem(dtype, b1, i);
            z[i] = activation(act, acc);
        }
        for (int c = 0; c < M; ++c) {
            double acc = 0.0;
            for (int i = 0; i < r; ++i)
                acc += load_elem(dtype, W2, (int64_t)c * r + i) * z[i];
            if (b2)
                acc += load_elem(dtype, b2, c);
            scores[(int64_t)row * M + c] = (float)acc;
        }
    }
    free(z);
}

/* ranking used by selection: score descending, then cluster id ascending */
static const float *g_rank_scores;
static int rank_cmp(const void *a, const void *b)
{
    int ia = *(const int *)a, ib = *(const int *)b;
    float sa = g_rank_scores[ia], sb = g_rank_scores[ib];
    if (sa > sb)
        return -1;
    if (sa < sb)
        return 1;
    return ia < ib ? -1 : (ia > ib ? 1 : 0);
}

/*
 * Top-cluster selection under a position-aware budget [A: the shortlist is
 * the union of the best-scoring clusters; S "Key Novelty": position-aware budget, larger
 * shortlists for early tokens; "Key Hyperparameters": k_c(t) decays from k_0
 * to k_1].  Clusters are ranked by (score desc, id asc).
 *   kind 0 (cluster budget): the first k = clamp(budget, 1, M) clusters.
 *   kind 1 (token budget):   the shortest prefix whose total size reaches the
 *                            budget (every cluster whose exclusive prefix size
 *                            is below it); budget <= 0 counts as 1.
 * Outputs: sel[row][0..n_sel) ranked ids, n_sel[row], sl_len[row] = sum of
 * the selected sizes.  NaN scores are invalid input.
 */
void oracle_select_clusters(int n, int M, const float *scores,
                            const int32_t *cluster_size, int kind,
                            const int32_t *budget, int32_t *sel,
                            int32_t *n_sel, int32_t *sl_len)
{
    int *order = (int *)malloc(sizeof(int) * (size_t)M);
    for (int row = 0; row < n; ++row) {
        const float *s = scores + (int64_t)row * M;
        for (int c = 0; c < M; ++c)
            order[c] = c;
        g_rank_scores = s;
        qsort(order, (size_t)M, sizeof(int), rank_cmp);
        int take = 0;
        int64_t total = 0;
        if (kind == 0) {
            int k = budget[row];
            if (k < 1)
                k = 1;
            if (k > M)
                k = M;
            for (take = 0; take < k; ++take)
                total += cluster_size[order[take]];
        } else {
            int64_t b = budget[row] < 1 ? 1 : budget[row];
            while (take < M && total < b)
                total += cluster_size[order[take++]];
        }
        for (int j = 0; j < M; ++j)
            sel[(int64_t)row * M + j] = j < take ? order[j] : -1;
        n_sel[row] = take;
        sl_len[row] = (int32_t)total;
    }
    free(order);
}

/*
 * Shortlist = union of the selected clusters' members [A: the shortlist is
 * the union of the selected clusters; S "Problem Definition": output V_S].
 * Listed in ascending token id.
 * sl_off[0] is read (base offset); sl_off[1..n] are written; offsets never
 * exceed `capacity` (entries past it are dropped and OR_ECAPACITY returned).
 * Cluster ids outside [0, M) are skipped and OR_EINVAL returned.
 */
int oracle_build_shortlist(int n, int M, int V, const int32_t *sel,
                           const int32_t *n_sel, const int32_t *cluster_of,
                           int64_t capacity, int64_t *sl_off, int32_t *sl_ids)
{
    int status = OR_OK;
    unsigned char *mark = (unsigned char *)malloc((size_t)(M > 0 ? M : 1));
    int64_t pos = sl_off[0];
    for (int row = 0; row < n; ++row) {
        memset(mark, 0, (size_t)M);
        int k = n_sel[row];
        if (k < 0 || k > M) {
            status = status ? status : OR_EINVAL;
            k = k < 0 ? 0 : M;
        }
        for (int j = 0; j < k; ++j) {
            int c = sel[(int64_t)row * M + j];
            if (c < 0 || c >= M) {
                status = status ? status : OR_EINVAL;
                continue;
            }
            mark[c] = 1;
        }
        for (int y = 0; y < V; ++y) {
            int c = cluster_of[y];
            if (c < 0 || c >= M) {
                status = status ? status : OR_EINVAL;
                continue;
            }
            if (!mark[c])
                continue;
            if (pos < capacity)
                sl_ids[pos] = y;
            else
                status = OR_ECAPACITY;
            ++pos;
        }
        sl_off[row + 1] = pos < capacity ? pos : capacity;
    }
    free(mark);
    return status;
}

/*
 * Gathered LM head [S "System Modules: Gathered LM Head" (projects hidden
 * states onto the shortlist rows only); "Novel Architectural Elements"
 * (index-select + GEMM); "Comparison to Prior Work" (O(|V_S| d) instead of
 * O(|V| d))]:
 *   logit[g][i][j] = sum_k W[S_g[j]][k] * h[g][i][k].
 * h row (g, i) starts at h + g*ldh_g + i*d.  Output for (g, i, j) at
 * m*sl_off[g] + i*len_g + j.  A token id outside [0, V) yields NaN.
 */
void oracle_gathered_lm_head(int dtype, int V, int d, const void *W, int G,
                             int m, const void *h, int64_t ldh_g,
                             const int64_t *sl_off, const int32_t *sl_ids,
                             float *logits)
{
    for (int g = 0; g < G; ++g) {
        int64_t len = sl_off[g + 1] - sl_off[g];
        for (int i = 0; i < m; ++i) {
            int64_t hrow = (int64_t)g * ldh_g + (int64_t)i * d;
            float *out = logits + (int64_t)m * sl_off[g] + (int64_t)i * len;
            for (int64_t j = 0; j < len; ++j) {
                int32_t y = sl_ids[sl_off[g] + j];
                if (y < 0 || y >= V) {
                    out[j] = NAN;
                    continue;
                }
                double acc = 0.0;
                for (int k = 0; k < d; ++k)
                    acc += load_elem(dtype, W, (int64_t)y * d + k) *
                           load_elem(dtype, h, hrow + k);
                out[j] = (float)acc;
            }
        }
    }
}

/*
 * Static-shortlist slab [A, on FR-Spec / VocabTrim: drafting restricted to a
 * fixed, frequency-ranked shortlist; S "Comparison to Prior Work"]: the rows
 * of a fixed list copied into one contiguous array, out[i] = W[ids[i]].  A
 * row whose id lies outside [0, V) is filled with quiet NaN (the bit pattern
 * 0x7FC0 per bf16 element, NAN per fp32 element).
 */
void oracle_pack_rows(int dtype, int V, int d, const void *W, int64_t n,
                      const int32_t *ids, void *out)
{
    const size_t e = dtype == 1 ? 2 : 4;
    for (int64_t i = 0; i < n; ++i) {
        char *dst = (char *)out + (size_t)i * d * e;
        const int32_t y = ids[i];
        if (y >= 0 && y < V) {
            memcpy(dst, (const char *)W + (size_t)y * d * e, (size_t)d * e);
        } else if (dtype == 1) {
            for (int k = 0; k < d; ++k)
                ((uint16_t *)dst)[k] = 0x7FC0;
        } else {
            for (int k = 0; k < d; ++k)
                ((float *)dst)[k] = NAN;
        }
    }
}

/*
 * Dense (full-vocabulary) head, the O(|V| d) projection the method replaces
 * [A; S "Core Problem"]: logits[row][y] = sum_k W[y][k] h_row[k].
 * Same summation as the gathered head, so the two agree bit for bit.
 */
void oracle_dense_lm_head(int dtype, int V, int d, const void *W, int n,
                          const void *h, int64_t ldh, float *logits)
{
    for (int row = 0; row < n; ++row)
        for (int y = 0; y < V; ++y) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += load_elem(dtype, W, (int64_t)y * d + k) *
                       load_elem(dtype, h, (int64_t)row * ldh + k);
            logits[(int64_t)row * V + y] = (float)acc;
        }
}

/*
 * Inverse-CDF draw over non-negative weights w[0..n): total = sum w; the
 * first j whose inclusive running sum exceeds u*total; if rounding leaves
 * none, the last j with w_j > 0 (or -1 when all are zero).  *tie is set when
 * a CDF boundary next to the threshold lies within TIE_REL*total of it.
 */
static int64_t inverse_cdf(const double *w, int64_t n, double u, int *tie,
                           double *total_out)
{
    double total = 0.0;
    for (int64_t j = 0; j < n; ++j)
        total += w[j];
    if (total_out)
        *total_out = total;
    double thr = u * total, run = 0.0, eps = TIE_REL * total;
    int64_t pick = -1, last_pos = -1;
    for (int64_t j = 0; j < n; ++j) {
        double before = run;
        run += w[j];
        if (w[j] > 0.0)
            last_pos = j;
        if (pick < 0 && run > thr) {
            pick = j;
            if (fabs(run - thr) < eps || (j > 0 && fabs(before - thr) < eps))
                *tie = 1;
        }
    }
    if (pick < 0) {
        pick = last_pos;
        *tie = 1;
    }
    return pick;
}

/*
 * Draft proposal from the shortlist distribution [A: the drafter proposes
 * from its shortlist; S "Pipeline Flow": gathered projection, then
 * sampling].  Per row (g, i): q = softmax(logits / tau) over S_g, token =
 * S_g[inverse_cdf(q, u)].  tau == 0 means argmax (ties to the lowest token
 * id) with a one-hot q.  Empty rows give token -1.  tie[row] marks draws
 * whose threshold sits within 1e-12 (relative) of a CDF boundary.
 */
void oracle_shortlist_sample(int G, int m, const int64_t *sl_off,
                             const int32_t *sl_ids, const float *logits,
                             float temperature, const float *u,
                             int32_t *token, float *q, unsigned char *tie)
{
    for (int g = 0; g < G; ++g) {
        int64_t len = sl_off[g + 1] - sl_off[g];
        double *e = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1));
        for (int i = 0; i < m; ++i) {
            int64_t row = (int64_t)g * m + i;
            const float *l = logits + (int64_t)m * sl_off[g] + (int64_t)i * len;
            float *qr = q + (int64_t)m * sl_off[g] + (int64_t)i * len;
            int t = 0;
            if (len == 0) {
                token[row] = -1;
                if (tie)
                    tie[row] = 0;
                continue;
            }
            int64_t jmax = 0;
            for (int64_t j = 1; j < len; ++j)
                if (l[j] > l[jmax])
                    jmax = j;
            int64_t pick;
            if (temperature == 0.0f) {
                pick = jmax;
                for (int64_t j = 0; j < len; ++j)
                    qr[j] = j == jmax ? 1.0f : 0.0f;
            } else {
                double mx = (double)l[jmax], Z = 0.0;
                for (int64_t j = 0; j < len; ++j)
                    e[j] = exp(((double)l[j] - mx) / (double)temperature);
                pick = inverse_cdf(e, len, (double)u[row], &t, &Z);
                for (int64_t j = 0; j < len; ++j)
                    qr[j] = (float)(e[j] / Z);
            }
            token[row] = sl_ids[sl_off[g] + pick];
            if (tie)
                tie[row] = (unsigned char)t;
        }
        free(e);
    }
}

/*
 * Full-vocabulary target distribution from target logits (softmax per row):
 * p[y] = exp(l[y] - max) / sum_y' exp(l[y'] - max), rounded to fp32.  The
 * target verifies over the full vocabulary [A; S "System Modules: Target
 * Model"].
 */
void oracle_target_softmax(int rows, int V, const float *logits, float *p)
{
    double *e = (double *)malloc(sizeof(double) * (size_t)V);
    for (int r = 0; r < rows; ++r) {
        const float *l = logits + (int64_t)r * V;
        float mx = l[0];
        for (int y = 1; y < V; ++y)
            if (l[y] > mx)
                mx = l[y];
        double Z = 0.0;
        for (int y = 0; y < V; ++y) {
            e[y] = exp((double)l[y] - (double)mx);
            Z += e[y];
        }
        for (int y = 0; y < V; ++y)
            p[(int64_t)r * V + y] = (float)(e[y] / Z);
    }
    free(e);
}

/*
 * Rejection-sampling verification over the full vocabulary, which keeps the
 * output distributed exactly as the target [A: the target checks the drafts
 * against its whole vocabulary, so the output is exact; S "Pipeline Flow:
 * Rejection Sampling Verification"; textbook speculative sampling].
 * For sequence b and positions t = 0..T-1 (draft[t][b], row t*B + b of the
 * shortlist arrays, q in the sampler's layout with m = 1):
 *   accept x iff u_acc * q_t(x) < p_t(x)   (q_t(x) = 0 off the shortlist);
 *   on the first rejection draw from max(0, p_t - q_t) over all of V (from
 *   p_t itself if that residual has no mass) with u_fin and stop;
 *   if all T are accepted draw the bonus token from p_T with u_fin.
 * out[b][0..n_acc] holds the emitted tokens, the rest is -1.
 */
void oracle_verify_reject(int B, int T, int V, const int32_t *draft,
                          const int64_t *sl_off, const int32_t *sl_ids,
                          const float *q, const float *p, const float *u_acc,
                          const float *u_fin, int32_t *n_acc, int32_t *out,
                          unsigned char *tie)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    double *qd = (double *)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        int t_flag = 0, t;
        for (int k = 0; k <= T; ++k)
            out[(int64_t)b * (T + 1) + k] = -1;
        for (t = 0; t < T; ++t) {
            int64_t row = (int64_t)t * B + b;
            const float *pt = p + ((int64_t)b * (T + 1) + t) * V;
            /* q_t as a dense vector over V */
            for (int y = 0; y < V; ++y)
                qd[y] = 0.0;
            for (int64_t j = sl_off[row]; j < sl_off[row + 1]; ++j) {
                int32_t y = sl_ids[j];
                if (y >= 0 && y < V)
                    qd[y] = (double)q[j];
            }
            int32_t x = draft[row];
            double qx = (x >= 0 && x < V) ? qd[x] : 0.0;
            double px = (x >= 0 && x < V) ? (double)pt[x] : 0.0;
            if ((double)u_acc[row] * qx < px) {
                out[(int64_t)b * (T + 1) + t] = x;
                continue;
            }
            double R;
            for (int y = 0; y < V; ++y) {
                double r = (double)pt[y] - qd[y];
                w[y] = r > 0.0 ? r : 0.0;
            }
            int64_t pick = inverse_cdf(w, V, (double)u_fin[b], &t_flag, &R);
            if (!(R > 0.0)) {
                t_flag = 0;
                for (int y = 0; y < V; ++y)
                    w[y] = (double)pt[y];
                pick = inverse_cdf(w, V, (double)u_fin[b], &t_flag, NULL);
            }
            out[(int64_t)b * (T + 1) + t] = (int32_t)pick;
            break;
        }
        if (t == T) {
            const float *pT = p + ((int64_t)b * (T + 1) + T) * V;
            for (int y = 0; y < V; ++y)
                w[y] = (double)pT[y];
            out[(int64_t)b * (T + 1) + T] =
                (int32_t)inverse_cdf(w, V, (double)u_fin[b], &t_flag, NULL);
        }
        n_acc[b] = t;
        if (tie)
            tie[b] = (unsigned char)t_flag;
    }
    free(w);
    free(qd);
}


/*
 * ---------------------------------------------------------------------------
 * Spherical k-means over the rows of the LM head [S "Key Novelty" (clusters
 * from the semantic similarity of LM-head weights), "Modeling / Key
 * Hyperparameters" (clustering algorithm: spherical k-means), "Key Terms"
 * (spherical k-means groups by cosine similarity, i.e. direction)].  The
 * algorithm is the published one (Dhillon and Modha, concept
 * decompositions): with unit rows x_y = w_y / |w_y| and unit centroids,
 * assign every row to the centroid of largest cosine, then replace every
 * centroid by the normalised sum of its rows.  W is bf16.
 * ---------------------------------------------------------------------------
 */

/* inv_norm[y] = 1 / |w_y| (fp64, rounded once); 0 for an all-zero row. */
void oracle_kmeans_inv_norms(int V, int d, const uint16_t *W, float *inv_norm)
{
    for (int y = 0; y < V; ++y) {
        double ss = 0.0;
        for (int k = 0; k < d; ++k) {
            double v = bf16_to_double(W[(int64_t)y * d + k]);
            ss += v * v;
        }
        inv_norm[y] = ss > 0.0 ? (float)(1.0 / sqrt(ss)) : 0.0f;
    }
}

/*
 * Assignment: assign[y] = argmax_c w_y . C[c] over bf16 centroids C [M][d]
 * (the row norm does not change the argmax), ties to the lower c; score[y]
 * the winning dot product (fp64, rounded to fp32).  tie[y] = 1 where the
 * runner-up is within tol of the winner, tol = d * 2^-22 * sum_k |w_yk C_ck|
 * of the winner: inside that band an fp32 accumulation in another order may
 * legitimately pick the runner-up.
 */
void oracle_kmeans_assign(int V, int d, const uint16_t *W, int M, const uint16_t *C,
                          int32_t *assign, float *score, uint8_t *tie)
{
    for (int y = 0; y < V; ++y) {
        const uint16_t *w = W + (int64_t)y * d;
        double best = -INFINITY, second = -INFINITY, mag = 0.0;
        int bc = 0;
        for (int c = 0; c < M; ++c) {
            const uint16_t *cv = C + (int64_t)c * d;
            double acc = 0.0, a = 0.0;
            for (int k = 0; k < d; ++k) {
                double p = bf16_to_double(w[k]) * bf16_to_double(cv[k]);
                acc += p;
                a += fabs(p);
            }
            if (acc > best) {
                second = best;
                best = acc;
                bc = c;
                mag = a;
            } else if (acc > second) {
                second = acc;
            }
        }
        assign[y] = bc;
        score[y] = (float)best;
        tie[y] = (uint8_t)(M > 1 && best - second <= (double)d * ldexp(1.0, -22) * mag);
    }
}

/*
 * Update: s_c = sum over rows y with assign[y] = c, in ascending y, of
 * w_y * inv_norm[y] (fp64); C_out[c] = s_c / |s_c| rounded to fp32; a
 * cluster without rows (or with s_c = 0) keeps C_prev[c].  size[c] = its row
 * count; norm[c] = |s_c|, whose sum over c is the spherical k-means
 * objective sum_y x_y . C_out[assign[y]] reached by this update.
 */
void oracle_kmeans_update(int V, int d, const uint16_t *W, const float *inv_norm, int M,
                          const int32_t *assign, const float *C_prev, float *C_out,
                          int32_t *size, double *norm)
{
    double *acc = (double *)calloc((size_t)M * d, sizeof(double));
    for (int c = 0; c < M; ++c)
        size[c] = 0;
    for (int y = 0; y < V; ++y) {
        int c = assign[y];
        if (c < 0 || c >= M)
            continue;
        size[c] += 1;
        for (int k = 0; k < d; ++k)
            acc[(int64_t)c * d + k] += bf16_to_double(W[(int64_t)y * d + k]) * (double)inv_norm[y];
    }
    for (int c = 0; c < M; ++c) {
        double ss = 0.0;
        for (int k = 0; k < d; ++k)
            ss += acc[(int64_t)c * d + k] * acc[(int64_t)c * d + k];
        double nrm = sqrt(ss);
        norm[c] = size[c] > 0 ? nrm : 0.0;
        for (int k = 0; k < d; ++k)
            C_out[(int64_t)c * d + k] = (size[c] > 0 && nrm > 0.0)
                                            ? (float)(acc[(int64_t)c * d + k] / nrm)
                                            : C_prev[(int64_t)c * d + k];
    }
    free(acc);
}


/*
 * ---------------------------------------------------------------------------
 * Tree verification.  The pages verify a drafted chain by rejection sampling
 * [A, S "Pipeline Flow"] and draft trees in the tree-shaped workload, but do
 * not define how a tree is verified.  This is the multi-step speculative
 * sampling of SpecInfer ("SpecInfer: Accelerating Generative Large Language
 * Model Serving with Tree-based Speculative Inference and Verification", a
 * reference of the DySpec page), in its general form where every child
 * carries the proposal it was drawn from: starting at the root, the children
 * of the current node u are tried in index order against a running residual
 * r, which starts as the target p_u.  Child c (token x_c drawn from q_c) is
 * accepted iff u_acc[c] * q_c(x_c) < r(x_c) (probability min(1, r/q_c));
 * after a rejection r <- max(0, r - q_c) / sum (over all V; back to p_u
 * should that have no mass).  An accepted child becomes the current node;
 * when no child is accepted (or the node has none) one token is drawn from r
 * with u_fin by the inverse CDF and the sequence stops.  The emitted tokens
 * are distributed as the target.  A tree that is a path is the chain
 * verifier above.
 *
 * Per sequence b: nodes 0..m, node 0 the root (the last emitted token, not
 * drafted), nodes 1..m drafted.  Drafted node i is described at index i-1 of
 * the [B][m] arrays: parent (in [0, i); any other value detaches the node),
 * token, u_acc, and its proposal q_i = row i-1 of group b in the sampler's
 * layout (q[m*sl_off[b] + (i-1)*len_b + j] over shortlist b).  p [B][m+1][V]
 * holds the target at every node (row 0: the root).  Outputs: n_acc[b]
 * accepted nodes, path[b][0..n_acc) their numbers (1..m), out[b][0..n_acc]
 * the emitted tokens (accepted tokens, then the final draw), the rest -1.
 * tie[b] = 1 where a decision after a rejection, or the final draw, lies
 * within 1e-12 (relative) of its threshold: there the order of the
 * residual's sums may decide.
 * ---------------------------------------------------------------------------
 */
void oracle_verify_tree(int B, int m, int V, const int32_t *parent, const int32_t *token,
                        const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                        const float *p, const float *u_acc, const float *u_fin,
                        int32_t *n_acc, int32_t *out, int32_t *path, uint8_t *tie)
{
    double *r = (double *)malloc((size_t)V * sizeof(double));
    double *qd = (double *)malloc((size_t)V * sizeof(double));
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (int64_t)b * m, *tok = token + (int64_t)b * m;
        const int64_t off = sl_off[b], len = sl_off[b + 1] - sl_off[b];
        int32_t *ob = out + (int64_t)b * (m + 1), *pb = path + (int64_t)b * m;
        for (int i = 0; i <= m; ++i)
            ob[i] = -1;
        for (int i = 0; i < m; ++i)
            pb[i] = -1;
        int t = 0;
        int u = 0, n = 0;
        for (;;) {
            const float *pu = p + ((int64_t)b * (m + 1) + u) * V;
            for (int64_t y = 0; y < V; ++y)
                r[y] = (double)pu[y];
            int accepted = -1, rejected = 0;
            for (int c = u + 1; c <= m; ++c) {
                if (par[c - 1] != u)
                    continue;
                /* the child's proposal as a dense vector over V */
                const float *qc = q + (int64_t)m * off + (int64_t)(c - 1) * len;
                for (int64_t y = 0; y < V; ++y)
                    qd[y] = 0.0;
                for (int64_t j = 0; j < len; ++j) {
                    int32_t y = sl_ids[off + j];
                    if (y >= 0 && y < V)
                        qd[y] = (double)qc[j];
                }
                const int32_t x = tok[c - 1];
                const int ok = x >= 0 && x < V;
                const double lhs = (double)u_acc[(int64_t)b * m + c - 1] * (ok ? qd[x] : 0.0);
                const double rx = ok ? r[x] : 0.0;
                if (rejected && fabs(lhs - rx) <= TIE_REL * (lhs + rx))
                    t = 1;
                if (lhs < rx) {
                    accepted = c;
                    break;
                }
                rejected = 1;
                double Z = 0.0;
                for (int64_t y = 0; y < V; ++y) {
                    r[y] = r[y] > qd[y] ? r[y] - qd[y] : 0.0;
                    Z += r[y];
                }
                for (int64_t y = 0; y < V; ++y)
                    r[y] = Z > 0.0 ? r[y] / Z : (double)pu[y];
            }
            if (accepted >= 0) {
                ob[n] = tok[accepted - 1];
                pb[n] = accepted;
                ++n;
                u = accepted;
                continue;
            }
            int dt = 0;
            const int64_t pick = inverse_cdf(r, V, (double)u_fin[b], &dt, NULL);
            if (dt)
                t = 1;
            ob[n] = (int32_t)pick;
            break;
        }
        n_acc[b] = n;
        tie[b] = (uint8_t)t;
    }
    free(r);
    free(qd);
}

/*
 * ---------------------------------------------------------------------------
 * Router training [S "Modeling": supervised multi-label classification; the
 * objective is binary cross entropy over clusters, a cluster's label being
 * positive when it holds a token from the top-L of the full drafter; the
 * trainable part of the router is its 2-layer MLP].
 * ---------------------------------------------------------------------------
 */

/* order used for the top-L: logit descending, then token id ascending */
static const float *g_topl_row;
static int topl_cmp(const void *a, const void *b)
{
    int ia = *(const int *)a, ib = *(const int *)b;
    float sa = g_topl_row[ia], sb = g_topl_row[ib];
    if (sa > sb)
        return -1;
    if (sa < sb)
        return 1;
    return ia < ib ? -1 : (ia > ib ? 1 : 0);
}

/*
 * Labels from the full drafter's logits: row i of logits (V values, row
 * stride ldl) orders the tokens by (logit desc, id asc); the first
 * min(L, V) of them are the top-L; labels[i][c] = 1 iff one of them lies in
 * cluster c (cluster_of[y] in [0, M); others are ignored), else 0.
 */
void oracle_topl_labels(int n, int V, int M, int L, const float *logits, int64_t ldl,
                        const int32_t *cluster_of, uint8_t *labels)
{
    int *idx = (int *)malloc(sizeof(int) * (size_t)V);
    for (int i = 0; i < n; ++i) {
        for (int y = 0; y < V; ++y)
            idx[y] = y;
        g_topl_row = logits + (int64_t)i * ldl;
        qsort(idx, (size_t)V, sizeof(int), topl_cmp);
        uint8_t *lab = labels + (int64_t)i * M;
        memset(lab, 0, (size_t)M);
        for (int k = 0; k < L && k < V; ++k) {
            int32_t c = cluster_of[idx[k]];
            if (c >= 0 && c < M)
                lab[c] = 1;
        }
    }
    free(idx);
}

static double sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* log(1 + e^x) without overflow */
static double softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

static double activation_grad(int act, double a)
{
    if (act == 0)
        return a > 0.0 ? 1.0 : 0.0;          /* ReLU (0 at the kink) */
    double s = sigmoid(a);                   /* SiLU: d/da a s(a) */
    return s * (1.0 + a * (1.0 - s));
}

/*
 * One plain SGD step of the router on a batch of n rows h[i] (row stride
 * ldh; fp32 or bf16 bits by dtype_h), labels y[i][c] in {0, 1}:
 *   a = W1 h + b1, z = act(a), s = W2 z + b2         (the router's forward)
 *   loss = 1/(n M) sum_{i,c} [softplus(s_ic) - y_ic s_ic]
 *        (= mean of -y log sigmoid(s) - (1 - y) log(1 - sigmoid(s)))
 *   g_s = (sigmoid(s) - y) / (n M)
 *   dW2 = g_s^T z, db2 = sum_i g_s, g_z = g_s W2, g_a = g_z * act'(a),
 *   dW1 = g_a^T h, db1 = sum_i g_a
 *   param <- param - lr * grad   (fp32 parameters, updated in place)
 * Gradients and the loss are returned in double; W1[r][d], W2[M][r].
 */
void oracle_router_train_step(int dtype_h, int n, int d, int r, int M, int act, const void *h,
                              int64_t ldh, const uint8_t *labels, float lr, float *W1,
                              float *b1, float *W2, float *b2, double *dW1, double *db1,
                              double *dW2, double *db2, double *loss)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)n * r);
    double *z = (double *)malloc(sizeof(double) * (size_t)n * r);
    double *gs = (double *)malloc(sizeof(double) * (size_t)n * M);
    double *ga = (double *)malloc(sizeof(double) * (size_t)n * r);
    const double inv = 1.0 / ((double)n * (double)M);
    double L = 0.0;
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += (double)W1[(int64_t)j * d + k] * load_elem(dtype_h, h, (int64_t)i * ldh + k);
            acc += (double)b1[j];
            a[(int64_t)i * r + j] = acc;
            z[(int64_t)i * r + j] = activation(act, acc);
        }
        for (int c = 0; c < M; ++c) {
            double s = 0.0;
            for (int j = 0; j < r; ++j)
                s += (double)W2[(int64_t)c * r + j] * z[(int64_t)i * r + j];
            s += (double)b2[c];
            const double y = labels[(int64_t)i * M + c] ? 1.0 : 0.0;
            L += softplus(s) - y * s;
            gs[(int64_t)i * M + c] = (sigmoid(s) - y) * inv;
        }
    }
    *loss = L * inv;
    for (int c = 0; c < M; ++c) {
        double bsum = 0.0;
        for (int i = 0; i < n; ++i)
            bsum += gs[(int64_t)i * M + c];
        db2[c] = bsum;
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += gs[(int64_t)i * M + c] * z[(int64_t)i * r + j];
            dW2[(int64_t)c * r + j] = acc;
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int c = 0; c < M; ++c)
                acc += gs[(int64_t)i * M + c] * (double)W2[(int64_t)c * r + j];
            ga[(int64_t)i * r + j] = acc * activation_grad(act, a[(int64_t)i * r + j]);
        }
    for (int j = 0; j < r; ++j) {
        double bsum = 0.0;
        for (int i = 0; i < n; ++i)
            bsum += ga[(int64_t)i * r + j];
        db1[j] = bsum;
        for (int k = 0; k < d; ++k) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += ga[(int64_t)i * r + j] * load_elem(dtype_h, h, (int64_t)i * ldh + k);
            dW1[(int64_t)j * d + k] = acc;
        }
    }
    /* the step, after every gradient is formed from the old parameters */
    for (int64_t e = 0; e < (int64_t)r * d; ++e)
        W1[e] = (float)((double)W1[e] - (double)lr * dW1[e]);
    for (int j = 0; j < r; ++j)
        b1[j] = (float)((double)b1[j] - (double)lr * db1[j]);
    for (int64_t e = 0; e < (int64_t)M * r; ++e)
        W2[e] = (float)((double)W2[e] - (double)lr * dW2[e]);
    for (int c = 0; c < M; ++c)
        b2[c] = (float)((double)b2[c] - (double)lr * db2[c]);
    free(a);
    free(z);
    free(gs);
    free(ga);
}
