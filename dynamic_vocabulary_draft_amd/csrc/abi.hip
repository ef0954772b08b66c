// C-ABI of the shortlisted draft head: host-side argument checks, workspace
// sizes, dispatch to the kernel families, and the two-stream chain runner.
// Nothing here allocates device memory.
#include <vector>

#include "common.h"
#include "kernels.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

ds_status hip_status(hipError_t e) { return e == hipSuccess ? DS_OK : DS_EHIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// per-thread pool of timing-free events for ds_draft_chain
struct EventPool {
    std::vector<hipEvent_t> ev;
    hipError_t ensure(size_t n)
    {
        while (ev.size() < n) {
            hipEvent_t e;
            hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
            if (r != hipSuccess)
                return r;
            ev.push_back(e);
        }
        return hipSuccess;
    }
    ~EventPool()
    {
        for (hipEvent_t e : ev)
            (void)hipEventDestroy(e);
    }
};
thread_local EventPool g_events;

ds_status check_router(ds_dtype dt, int n, int d, int r, int M, ds_act act, const void *h,
                       int64_t ldh, const void *W1, const void *b1, const void *W2,
                       const void *b2, const float *scores)
{
    if (!h || !W1 || !W2 || !scores)
        return DS_EINVAL;
    if (n <= 0 || d <= 0 || r <= 0 || M <= 0)
        return DS_EINVAL;
    if (dt != DS_F32 && dt != DS_BF16)
        return DS_EDTYPE;
    if (act != DS_RELU && act != DS_SILU)
        return DS_EDTYPE;
    if (d % 8 || r % 8 || ldh < d || ldh % 8)
        return DS_ESHAPE;
    if (!aligned16(h) || !aligned16(W1) || !aligned16(W2))
        return DS_EINVAL;
    (void)b1;
    (void)b2;
    return DS_OK;
}

ds_status check_select(int n, int M, const float *scores, const int32_t *cluster_size,
                       ds_budget_kind kind, const int32_t *budget, int32_t *sel, int32_t *n_sel,
                       int32_t *sl_len)
{
    if (!scores || !cluster_size || !budget || !sel || !n_sel || !sl_len)
        return DS_EINVAL;
    if (n <= 0 || M <= 0)
        return DS_EINVAL;
    if (kind != DS_BUDGET_CLUSTERS && kind != DS_BUDGET_TOKENS)
        return DS_EDTYPE;
    if (M > DS_MAX_CLUSTERS || n > DS_MAX_GROUPS)
        return DS_ESHAPE;
    return DS_OK;
}

ds_status check_build(int n, int M, int V, const int32_t *sel, const int32_t *n_sel,
                      const int32_t *cluster_of, int64_t capacity, int64_t *sl_off,
                      int32_t *sl_ids, void *ws, size_t ws_bytes)
{
    if (!sel || !n_sel || !cluster_of || !sl_off || !sl_ids || !ws)
        return DS_EINVAL;
    if (n <= 0 || M <= 0 || V <= 0 || capacity < 0)
        return DS_EINVAL;
    if (M > DS_MAX_CLUSTERS || n > DS_MAX_GROUPS)
        return DS_ESHAPE;
    if (!aligned16(cluster_of) || ws_bytes < ds::build_ws_bytes(n, V))
        return DS_EINVAL;
    return DS_OK;
}

ds_status check_head(ds_dtype dt, int V, int d, const void *W, int G, int m, const void *h,
                     int64_t ldh_g, const int64_t *sl_off, const int32_t *sl_ids,
                     int64_t max_rows, float *logits)
{
    if (!W || !h || !sl_off || !sl_ids || !logits)
        return DS_EINVAL;
    if (V <= 0 || d <= 0 || G <= 0 || m <= 0 || max_rows < 0)
        return DS_EINVAL;
    if (dt != DS_F32 && dt != DS_BF16)
        return DS_EDTYPE;
    if (d % 8 || ldh_g % 8 || ldh_g < (int64_t)m * d || m > DS_MAX_HEAD_ROWS || G > DS_MAX_GROUPS)
        return DS_ESHAPE;
    if ((int64_t)d * (dt == DS_BF16 ? 2 : 4) > 16 * 1024)  // <= 16 chunks of 16 B per lane
        return DS_ESHAPE;
    if (!aligned16(W) || !aligned16(h))
        return DS_EINVAL;
    return DS_OK;
}

ds_status check_sample(int G, int m, const int64_t *sl_off, const int32_t *sl_ids,
                       const float *logits, float temperature, const float *u, int32_t *token,
                       float *q)
{
    if (!sl_off || !sl_ids || !logits || !u || !token || !q)
        return DS_EINVAL;
    if (G <= 0 || m <= 0 || m > DS_MAX_HEAD_ROWS || G > DS_MAX_GROUPS)
        return DS_EINVAL;
    if (!(temperature >= 0.0f) || temperature > 3.0e38f)
        return DS_EINVAL;
    return DS_OK;
}

ds_status check_verify(int B, int T, int V, const int32_t *draft, const int64_t *sl_off,
                       const int32_t *sl_ids, const float *q, const float *p, const float *u_acc,
                       const float *u_fin, int32_t *n_acc, int32_t *out)
{
    if (!draft || !sl_off || !sl_ids || !q || !p || !u_acc || !u_fin || !n_acc || !out)
        return DS_EINVAL;
    if (B <= 0 || T <= 0 || V <= 0)
        return DS_EINVAL;
    if (T > 64 || V > (1 << 20) || B > DS_MAX_GROUPS)
        return DS_ESHAPE;
    return DS_OK;
}

}  // namespace

extern "C" {

const char *ds_status_string(ds_status s)
{
    switch (s) {
    case DS_OK: return "ok";
    case DS_EINVAL: return "invalid argument";
    case DS_EDTYPE: return "unsupported dtype, activation or budget kind";
    case DS_ESHAPE: return "inconsistent or unsupported sizes";
    case DS_ECAPACITY: return "shortlist exceeds capacity";
    case DS_EHIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

const char *ds_version(void) { return "dynaspec-mi355x 0.1 gfx950"; }

size_t ds_router_workspace_bytes(int n, int r)
{
    return n > 0 && r > 0 ? (size_t)n * (size_t)r * sizeof(float) : 0;
}

ds_status ds_router_score(hipStream_t s, ds_dtype dt, int n, int d, int r, int M, ds_act act,
                          const void *h, int64_t ldh, const void *W1, const void *b1,
                          const void *W2, const void *b2, float *scores, void *ws,
                          size_t ws_bytes)
{
    ds_status st = check_router(dt, n, d, r, M, act, h, ldh, W1, b1, W2, b2, scores);
    if (st != DS_OK)
        return st;
    if (!ws || ws_bytes < ds_router_workspace_bytes(n, r))
        return DS_EINVAL;
    return hip_status(ds::router_launch(s, dt == DS_BF16, n, d, r, M, act, h, ldh, W1, b1, W2, b2,
                                        scores, reinterpret_cast<float *>(ws)));
}

ds_status ds_select_clusters(hipStream_t s, int n, int M, const float *scores,
                             const int32_t *cluster_size, ds_budget_kind kind,
                             const int32_t *budget, int32_t *sel, int32_t *n_sel, int32_t *sl_len)
{
    ds_status st = check_select(n, M, scores, cluster_size, kind, budget, sel, n_sel, sl_len);
    if (st != DS_OK)
        return st;
    return hip_status(
        ds::select_launch(s, n, M, scores, cluster_size, kind, budget, sel, n_sel, sl_len));
}

size_t ds_build_workspace_bytes(int n, int V)
{
    return n > 0 && V > 0 ? ds::build_ws_bytes(n, V) : 0;
}

ds_status ds_build_shortlist(hipStream_t s, int n, int M, int V, const int32_t *sel,
                             const int32_t *n_sel, const int32_t *cluster_of, int64_t capacity,
                             int64_t *sl_off, int32_t *sl_ids, int32_t *err_flag, void *ws,
                             size_t ws_bytes)
{
    ds_status st = check_build(n, M, V, sel, n_sel, cluster_of, capacity, sl_off, sl_ids, ws,
                               ws_bytes);
    if (st != DS_OK)
        return st;
    return hip_status(ds::build_launch(s, n, M, V, sel, n_sel, cluster_of, capacity, sl_off,
                                       sl_ids, err_flag, ws));
}

ds_status ds_gathered_lm_head(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int G,
                              int m, const void *h, int64_t ldh_g, const int64_t *sl_off,
                              const int32_t *sl_ids, int64_t max_rows, float *logits)
{
    ds_status st = check_head(dt, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows, logits);
    if (st != DS_OK)
        return st;
    return hip_status(ds::head_launch(s, dt == DS_BF16, V, d, W, G, m, h, ldh_g, sl_off, sl_ids,
                                      max_rows, logits));
}

ds_status ds_shortlist_sample(hipStream_t s, int G, int m, const int64_t *sl_off,
                              const int32_t *sl_ids, const float *logits, float temperature,
                              const float *u, int32_t *token, float *q)
{
    ds_status st = check_sample(G, m, sl_off, sl_ids, logits, temperature, u, token, q);
    if (st != DS_OK)
        return st;
    return hip_status(ds::sample_launch(s, G, m, sl_off, sl_ids, logits, temperature, u, token, q));
}

ds_status ds_target_softmax(hipStream_t s, int rows, int V, const float *logits, float *p)
{
    if (!logits || !p || rows <= 0 || V <= 0)
        return DS_EINVAL;
    return hip_status(ds::softmax_launch(s, rows, V, logits, p));
}

ds_status ds_verify_reject(hipStream_t s, int B, int T, int V, const int32_t *draft,
                           const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                           const float *p, const float *u_acc, const float *u_fin,
                           int32_t *n_acc, int32_t *out)
{
    ds_status st = check_verify(B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out);
    if (st != DS_OK)
        return st;
    return hip_status(
        ds::verify_launch(s, B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out));
}

size_t ds_draft_chain_workspace_bytes(int B, int T, int V, int r)
{
    if (B <= 0 || T <= 0 || V <= 0 || r <= 0)
        return 0;
    return round_up(ds_router_workspace_bytes(B, r), 256) + ds::build_ws_bytes(B, V);
}

ds_status ds_draft_chain(hipStream_t hs, hipStream_t rs, const ds_draft_chain_args *a)
{
    if (!a)
        return DS_EINVAL;
    const int B = a->B, T = a->T;
    if (B <= 0 || T <= 0 || !a->max_rows || !a->budget || !a->u_draft || !a->token || !a->q)
        return DS_EINVAL;
    const size_t e = a->dtype == DS_BF16 ? 2 : 4;
    const int64_t ldh = (int64_t)(T + 1) * a->d;  // h is [B][T+1][d]
    ds_status st = check_router(a->dtype, B, a->d, a->r, a->M, a->act, a->h, ldh, a->W1, a->b1,
                                a->W2, a->b2, a->scores);
    if (st == DS_OK)
        st = check_select(B, a->M, a->scores, a->cluster_size, a->budget_kind, a->budget, a->sel,
                          a->n_sel, a->sl_len);
    if (st == DS_OK)
        st = check_head(a->dtype, a->V, a->d, a->W, B, 1, a->h, ldh, a->sl_off, a->sl_ids, 0,
                        a->logits);
    if (st != DS_OK)
        return st;
    if (!a->cluster_of || !a->sl_off || !a->sl_ids || !a->ws || a->capacity < 0 ||
        a->ws_bytes < ds_draft_chain_workspace_bytes(B, T, a->V, a->r) ||
        !aligned16(a->cluster_of))
        return DS_EINVAL;
    if (!(a->temperature >= 0.0f))
        return DS_EINVAL;
    for (int t = 0; t < T; ++t) {
        if (a->max_rows[t] < 0)
            return DS_EINVAL;
        if (a->W_pos && (!a->W_pos[t] || !aligned16(a->W_pos[t])))
            return DS_EINVAL;
        if (a->head_events && (!a->head_events[2 * t] || !a->head_events[2 * t + 1]))
            return DS_EINVAL;
    }

    float *z = reinterpret_cast<float *>(a->ws);
    void *bws = reinterpret_cast<char *>(a->ws) + round_up(ds_router_workspace_bytes(B, a->r), 256);
    if (g_events.ensure((size_t)T + 1) != hipSuccess)
        return DS_EHIP;
    hipEvent_t fork = g_events.ev[T];
    const bool bf16 = a->dtype == DS_BF16;
    const char *hb = reinterpret_cast<const char *>(a->h);
    hipError_t err = hipEventRecord(fork, hs);
    if (err == hipSuccess)
        err = hipStreamWaitEvent(rs, fork, 0);
    for (int t = 0; t < T && err == hipSuccess; ++t) {
        const int64_t rb = (int64_t)t * B;
        err = ds::router_launch(rs, bf16, B, a->d, a->r, a->M, a->act, hb + (size_t)t * a->d * e,
                                ldh, a->W1, a->b1, a->W2, a->b2, a->scores + rb * a->M, z);
        if (err == hipSuccess)
            err = ds::select_launch(rs, B, a->M, a->scores + rb * a->M, a->cluster_size,
                                    a->budget_kind, a->budget + rb, a->sel + rb * a->M,
                                    a->n_sel + rb, a->sl_len + rb);
        if (err == hipSuccess)
            err = ds::build_launch(rs, B, a->M, a->V, a->sel + rb * a->M, a->n_sel + rb,
                                   a->cluster_of, a->capacity, a->sl_off + rb, a->sl_ids,
                                   a->err_flag, bws);
        if (err == hipSuccess)
            err = hipEventRecord(g_events.ev[t], rs);
        if (err == hipSuccess)
            err = hipStreamWaitEvent(hs, g_events.ev[t], 0);
        if (err == hipSuccess && a->head_events)
            err = hipEventRecord(a->head_events[2 * t], hs);
        if (err == hipSuccess)
            err = ds::head_launch(hs, bf16, a->V, a->d, a->W_pos ? a->W_pos[t] : a->W, B, 1,
                                  hb + (size_t)(t + 1) * a->d * e, ldh, a->sl_off + rb, a->sl_ids,
                                  a->max_rows[t], a->logits);
        if (err == hipSuccess && a->head_events)
            err = hipEventRecord(a->head_events[2 * t + 1], hs);
        if (err == hipSuccess)
            err = ds::sample_launch(hs, B, 1, a->sl_off + rb, a->sl_ids, a->logits, a->temperature,
                                    a->u_draft + rb, a->token + rb, a->q);
    }
    return hip_status(err);
}

}  // extern "C"
