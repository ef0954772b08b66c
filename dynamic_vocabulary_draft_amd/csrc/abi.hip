// C-ABI of the shortlisted draft head: host-side argument checks, workspace
// sizes, dispatch to the kernel families, and the two-stream chain runner.
// Nothing here allocates device memory.
#include <cstddef>
#include <atomic>
#include <mutex>
#include <new>

#include "common.h"
#include "kernels.h"

namespace ds {

int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 256;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0)
            return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64)
        cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace ds

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

ds_status hip_status(hipError_t e) { return e == hipSuccess ? DS_OK : DS_EHIP; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

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
    if (d % 8 || r % 8 || ldh < d || ldh % 8 || d > 8192 || r > 8192)
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
                      const int32_t *cluster_of, const int32_t *index, int64_t capacity,
                      int64_t *sl_off, int32_t *sl_ids, void *ws, size_t ws_bytes)
{
    if (!sel || !n_sel || !cluster_of || !index || !sl_off || !sl_ids || !ws)
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
                       const float *logits, float temperature, const float *u, int64_t max_len,
                       int32_t *token, float *q)
{
    if (!sl_off || !sl_ids || !logits || !u || !token || !q)
        return DS_EINVAL;
    if (G <= 0 || m <= 0 || m > DS_MAX_HEAD_ROWS || G > DS_MAX_GROUPS || max_len <= 0)
        return DS_EINVAL;
    if (max_len > (1 << 20) || (int64_t)G * m > 65535)
        return DS_ESHAPE;
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
    if (T > 64 || V > (1 << 20) || B > DS_MAX_GROUPS || (int64_t)B * T > (1ll << 30))
        return DS_ESHAPE;
    return DS_OK;
}

// Scratch of ds_verify_reject_noalloc: one copy per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[DS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices];

// Device address of `scratch` on the current device (looked up on the
// device's first call, then cached).
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
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
    return n > 0 && r > 0 ? ds::router_ws_bytes(n, r) : 0;
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

size_t ds_cluster_index_bytes(int M, int V)
{
    return M > 0 && V > 0 ? ds::index_bytes(M, V) : 0;
}

ds_status ds_cluster_index(hipStream_t s, int M, int V, const int32_t *cluster_of,
                           int32_t *index, int32_t *err_flag)
{
    if (!cluster_of || !index || M <= 0 || V <= 0)
        return DS_EINVAL;
    if (M > DS_MAX_CLUSTERS)
        return DS_ESHAPE;
    return hip_status(ds::index_launch(s, M, V, cluster_of, index, err_flag));
}

size_t ds_build_workspace_bytes(int n, int V)
{
    return n > 0 && V > 0 ? ds::build_ws_bytes(n, V) : 0;
}

ds_status ds_build_shortlist(hipStream_t s, int n, int M, int V, const int32_t *sel,
                             const int32_t *n_sel, const int32_t *cluster_of,
                             const int32_t *index, int64_t capacity, int64_t *sl_off,
                             int32_t *sl_ids, int32_t *err_flag, void *ws, size_t ws_bytes)
{
    ds_status st = check_build(n, M, V, sel, n_sel, cluster_of, index, capacity, sl_off, sl_ids,
                               ws, ws_bytes);
    if (st != DS_OK)
        return st;
    return hip_status(ds::build_launch(s, n, M, V, sel, n_sel, cluster_of, index, capacity, sl_off,
                                       sl_ids, err_flag, ws));
}

size_t ds_head_workspace_bytes(int G, int m, int V)
{
    return G > 0 && m > 0 && V > 0 ? ds::head_ws_bytes(G, m, V) : 0;
}

ds_status ds_gathered_lm_head(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int G,
                              int m, const void *h, int64_t ldh_g, const int64_t *sl_off,
                              const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                              size_t ws_bytes)
{
    ds_status st = check_head(dt, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows, logits);
    if (st != DS_OK)
        return st;
    const size_t need = ds_head_workspace_bytes(G, m, V);
    if (need && (!ws || ws_bytes < need))
        return DS_EINVAL;
    return hip_status(ds::head_launch(s, dt == DS_BF16, V, d, W, G, m, h, ldh_g, sl_off, sl_ids,
                                      max_rows, logits, ws));
}

ds_status ds_gathered_lm_head_timed(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int G,
                                    int m, const void *h, int64_t ldh_g, const int64_t *sl_off,
                                    const int32_t *sl_ids, int64_t max_rows, float *logits,
                                    void *ws, size_t ws_bytes, hipEvent_t start, hipEvent_t stop)
{
    ds_status st = check_head(dt, V, d, W, G, m, h, ldh_g, sl_off, sl_ids, max_rows, logits);
    if (st != DS_OK)
        return st;
    const size_t need = ds_head_workspace_bytes(G, m, V);
    if (need && (!ws || ws_bytes < need))
        return DS_EINVAL;
    return hip_status(ds::head_launch(s, dt == DS_BF16, V, d, W, G, m, h, ldh_g, sl_off, sl_ids,
                                      max_rows, logits, ws, start, stop));
}

ds_status ds_pack_rows(hipStream_t s, ds_dtype dt, int V, int d, const void *W, int64_t n,
                       const int32_t *ids, void *out)
{
    if (n < 0 || V <= 0 || d <= 0)
        return DS_EINVAL;
    if (dt != DS_F32 && dt != DS_BF16)
        return DS_EDTYPE;
    if (d % 8)
        return DS_ESHAPE;
    if (n == 0)
        return DS_OK;
    if (!W || !ids || !out || !aligned16(W) || !aligned16(out))
        return DS_EINVAL;
    return hip_status(ds::pack_launch(s, dt == DS_BF16, V, d, W, n, ids, out));
}

ds_status ds_kmeans_inv_norms(hipStream_t s, int V, int d, const void *W, float *inv_norm)
{
    if (!W || !inv_norm || V <= 0 || d <= 0)
        return DS_EINVAL;
    if (d % 8 || d > 8192)
        return DS_ESHAPE;
    if (!aligned16(W))
        return DS_EINVAL;
    return hip_status(ds::kmeans_inv_norm_launch(s, V, d, W, inv_norm));
}

size_t ds_kmeans_assign_workspace_bytes(int V) { return V > 0 ? ds::kmeans_assign_ws_bytes(V) : 0; }

ds_status ds_kmeans_assign(hipStream_t s, int V, int d, const void *W, int M, const void *C,
                           int32_t *assign, float *score, void *ws, size_t ws_bytes,
                           hipEvent_t start, hipEvent_t stop)
{
    if (!W || !C || !assign || !score || V <= 0 || d <= 0 || M <= 0)
        return DS_EINVAL;
    if (d % 64 || d > 8192 || M > DS_MAX_CLUSTERS)
        return DS_ESHAPE;
    if (!aligned16(W) || !aligned16(C) || !ws || ws_bytes < ds_kmeans_assign_workspace_bytes(V))
        return DS_EINVAL;
    return hip_status(ds::kmeans_assign_launch(s, V, d, W, M, C, assign, score, ws, start, stop));
}

size_t ds_kmeans_update_workspace_bytes(int V, int d, int M)
{
    return V > 0 && d > 0 && M > 0 ? ds::kmeans_update_ws_bytes(V, d, M) : 0;
}

ds_status ds_kmeans_update(hipStream_t s, int V, int d, const void *W, const float *inv_norm, int M,
                           const int32_t *assign, const float *C_prev, float *C_out,
                           void *C_out_bf16, int32_t *size, double *norm, int32_t *err_flag,
                           void *ws, size_t ws_bytes)
{
    if (!W || !inv_norm || !assign || !C_prev || !C_out || !C_out_bf16 || !size || !norm)
        return DS_EINVAL;
    if (V <= 0 || d <= 0 || M <= 0)
        return DS_EINVAL;
    if (d % 8 || d > 8192 || M > DS_MAX_CLUSTERS)
        return DS_ESHAPE;
    if (!aligned16(W) || !ws || ws_bytes < ds_kmeans_update_workspace_bytes(V, d, M))
        return DS_EINVAL;
    return hip_status(ds::kmeans_update_launch(s, V, d, W, inv_norm, M, assign, C_prev, C_out,
                                               C_out_bf16, size, norm, err_flag, ws));
}

size_t ds_sample_workspace_bytes(int G, int m, int64_t max_len)
{
    return G > 0 && m > 0 && max_len > 0 ? ds::sample_ws_bytes((int64_t)G * m, max_len) : 0;
}

ds_status ds_shortlist_sample(hipStream_t s, int G, int m, const int64_t *sl_off,
                              const int32_t *sl_ids, const float *logits, float temperature,
                              const float *u, int64_t max_len, int32_t *token, float *q, void *ws,
                              size_t ws_bytes)
{
    ds_status st = check_sample(G, m, sl_off, sl_ids, logits, temperature, u, max_len, token, q);
    if (st != DS_OK)
        return st;
    if (!ws || ws_bytes < ds_sample_workspace_bytes(G, m, max_len))
        return DS_EINVAL;
    return hip_status(ds::sample_launch(s, G, m, sl_off, sl_ids, logits, temperature, u, token, q,
                                        max_len, ws));
}

static_assert(sizeof(ds_qstats) == sizeof(ds::QStats) && offsetof(ds_qstats, M) == 0 &&
                  offsetof(ds_qstats, rZ) == offsetof(ds::QStats, rZ),
              "row statistics layout");

ds_status ds_shortlist_sample_stats(hipStream_t s, int G, int m, const int64_t *sl_off,
                                    const int32_t *sl_ids, const float *logits,
                                    float temperature, const float *u, int64_t max_len,
                                    int32_t *token, ds_qstats *qstats, void *ws, size_t ws_bytes)
{
    if (!qstats || !(temperature > 0.0f))
        return DS_EINVAL;
    // check_sample wants a q pointer: the statistics take its place
    ds_status st = check_sample(G, m, sl_off, sl_ids, logits, temperature, u, max_len, token,
                                reinterpret_cast<float *>(qstats));
    if (st != DS_OK)
        return st;
    if (!ws || ws_bytes < ds_sample_workspace_bytes(G, m, max_len))
        return DS_EINVAL;
    return hip_status(ds::sample_stats_launch(s, G, m, sl_off, sl_ids, logits, temperature, u,
                                              token, reinterpret_cast<ds::QStats *>(qstats),
                                              max_len, ws));
}

size_t ds_softmax_workspace_bytes(int rows, int V)
{
    return rows > 0 && V > 0 ? ds::softmax_ws_bytes(rows, V) : 0;
}

ds_status ds_target_softmax(hipStream_t s, int rows, int V, const float *logits, float *p,
                            void *ws, size_t ws_bytes)
{
    if (!logits || !p || rows <= 0 || V <= 0)
        return DS_EINVAL;
    if (V > (1 << 20) || rows > 65535)
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_softmax_workspace_bytes(rows, V))
        return DS_EINVAL;
    return hip_status(ds::softmax_launch(s, rows, V, logits, p, ws));
}

size_t ds_verify_workspace_bytes(int B, int T, int V)
{
    return B > 0 && T > 0 && V > 0 ? ds::verify_ws_bytes(B, T, V) : 0;
}

ds_status ds_verify_reject(hipStream_t s, int B, int T, int V, const int32_t *draft,
                           const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                           const float *p, const float *u_acc, const float *u_fin,
                           int32_t *n_acc, int32_t *out, void *ws, size_t ws_bytes)
{
    ds_status st = check_verify(B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out);
    if (st != DS_OK)
        return st;
    if (!ws || ws_bytes < ds_verify_workspace_bytes(B, T, V))
        return DS_EINVAL;
    return hip_status(ds::verify_launch(s, B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin,
                                        n_acc, out, ws));
}

size_t ds_verify_logits_workspace_bytes(int B, int T, int V)
{
    return B > 0 && T > 0 && V > 0 ? ds::verify_logits_ws_bytes(B, T, V) : 0;
}

ds_status ds_verify_reject_logits(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                  const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                  const float *logits, const float *u_acc, const float *u_fin,
                                  int32_t *n_acc, int32_t *out, void *ws, size_t ws_bytes)
{
    ds_status st =
        check_verify(B, T, V, draft, sl_off, sl_ids, q, logits, u_acc, u_fin, n_acc, out);
    if (st != DS_OK)
        return st;
    if ((int64_t)B * (T + 1) > 65535)  // one statistics row per target position
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_verify_logits_workspace_bytes(B, T, V))
        return DS_EINVAL;
    return hip_status(ds::verify_logits_launch(s, B, T, V, draft, sl_off, sl_ids, q, logits,
                                               u_acc, u_fin, n_acc, out, ws));
}

ds_status ds_verify_reject_logits_qstats(hipStream_t s, int B, int T, int V,
                                         const int32_t *draft, const int64_t *sl_off,
                                         const int32_t *sl_ids, const float *draft_logits,
                                         const ds_qstats *qstats, float temperature,
                                         const float *logits, const float *u_acc,
                                         const float *u_fin, int32_t *n_acc, int32_t *out,
                                         void *ws, size_t ws_bytes)
{
    if (!qstats || !(temperature > 0.0f) || temperature > 3.0e38f)
        return DS_EINVAL;
    ds_status st = check_verify(B, T, V, draft, sl_off, sl_ids, draft_logits, logits, u_acc,
                                u_fin, n_acc, out);
    if (st != DS_OK)
        return st;
    if ((int64_t)B * (T + 1) > 65535)  // one statistics row per target position
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_verify_logits_workspace_bytes(B, T, V))
        return DS_EINVAL;
    return hip_status(ds::verify_logits_qstats_launch(
        s, B, T, V, draft, sl_off, sl_ids, draft_logits,
        reinterpret_cast<const ds::QStats *>(qstats), temperature, logits, u_acc, u_fin, n_acc,
        out, ws));
}

ds_status ds_verify_reject_noalloc(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                   const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                   const float *p, const float *u_acc, const float *u_fin,
                                   int32_t *n_acc, int32_t *out)
{
    ds_status st = check_verify(B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out);
    if (st != DS_OK)
        return st;
    if (ds::verify_ws_bytes(B, T, V) > (size_t)DS_NOALLOC_SCRATCH_BYTES)
        return DS_ESHAPE;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess)
        return DS_EHIP;
    // every scratch entry the two kernels read is written earlier in the
    // same call (chunk sums, first rejected position): nothing to clear
    return hip_status(ds::verify_launch(s, B, T, V, draft, sl_off, sl_ids, q, p, u_acc, u_fin,
                                        n_acc, out, ws));
}

size_t ds_verify_tree_workspace_bytes(int B, int m, int V, int64_t max_len)
{
    if (B <= 0 || m <= 0 || V <= 0 || max_len <= 0)
        return 0;
    return ds::verify_tree_ws_bytes(B, m, V, max_len);
}

ds_status ds_verify_tree(hipStream_t s, int B, int m, int V, const int32_t *parent,
                         const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                         const float *q, const float *p, const float *u_acc, const float *u_fin,
                         int64_t max_len, int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                         size_t ws_bytes)
{
    if (!parent || !token || !sl_off || !sl_ids || !q || !p || !u_acc || !u_fin || !n_acc ||
        !out || !path)
        return DS_EINVAL;
    if (B <= 0 || m <= 0 || V <= 0 || max_len <= 0)
        return DS_EINVAL;
    if (m > DS_MAX_TREE_NODES || V > (1 << 20) || B > DS_MAX_GROUPS || max_len > (1 << 24))
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_verify_tree_workspace_bytes(B, m, V, max_len))
        return DS_EINVAL;
    return hip_status(ds::verify_tree_launch(s, B, m, V, parent, token, sl_off, sl_ids, q, p,
                                             u_acc, u_fin, max_len, n_acc, out, path, ws));
}

size_t ds_verify_tree_logits_workspace_bytes(int B, int m, int V, int64_t max_len)
{
    if (B <= 0 || m <= 0 || V <= 0 || max_len <= 0)
        return 0;
    return ds::verify_tree_logits_ws_bytes(B, m, V, max_len);
}

ds_status ds_verify_tree_logits(hipStream_t s, int B, int m, int V, const int32_t *parent,
                                const int32_t *token, const int64_t *sl_off,
                                const int32_t *sl_ids, const float *q, const float *logits,
                                const float *u_acc, const float *u_fin, int64_t max_len,
                                int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                size_t ws_bytes)
{
    if (!parent || !token || !sl_off || !sl_ids || !q || !logits || !u_acc || !u_fin || !n_acc ||
        !out || !path)
        return DS_EINVAL;
    if (B <= 0 || m <= 0 || V <= 0 || max_len <= 0)
        return DS_EINVAL;
    if (m > DS_MAX_TREE_NODES || V > (1 << 20) || B > DS_MAX_GROUPS || max_len > (1 << 24) ||
        (int64_t)B * (m + 1) > 65535)
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_verify_tree_logits_workspace_bytes(B, m, V, max_len))
        return DS_EINVAL;
    return hip_status(ds::verify_tree_logits_launch(s, B, m, V, parent, token, sl_off, sl_ids, q,
                                                    logits, u_acc, u_fin, max_len, n_acc, out,
                                                    path, ws));
}

ds_status ds_verify_tree_logits_qstats(hipStream_t s, int B, int m, int V,
                                       const int32_t *parent, const int32_t *token,
                                       const int64_t *sl_off, const int32_t *sl_ids,
                                       const float *draft_logits, const ds_qstats *qstats,
                                       float temperature, const float *logits,
                                       const float *u_acc, const float *u_fin, int64_t max_len,
                                       int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                       size_t ws_bytes)
{
    if (!qstats || !(temperature > 0.0f) || temperature > 3.0e38f)
        return DS_EINVAL;
    if (!parent || !token || !sl_off || !sl_ids || !draft_logits || !logits || !u_acc || !u_fin ||
        !n_acc || !out || !path)
        return DS_EINVAL;
    if (B <= 0 || m <= 0 || V <= 0 || max_len <= 0)
        return DS_EINVAL;
    if (m > DS_MAX_TREE_NODES || V > (1 << 20) || B > DS_MAX_GROUPS || max_len > (1 << 24) ||
        (int64_t)B * (m + 1) > 65535)
        return DS_ESHAPE;
    if (!ws || ws_bytes < ds_verify_tree_logits_workspace_bytes(B, m, V, max_len))
        return DS_EINVAL;
    return hip_status(ds::verify_tree_logits_qstats_launch(
        s, B, m, V, parent, token, sl_off, sl_ids, draft_logits,
        reinterpret_cast<const ds::QStats *>(qstats), temperature, logits, u_acc, u_fin, max_len,
        n_acc, out, path, ws));
}

ds_status ds_dense_lm_head(hipStream_t s, int V, int d, const void *W, int n, const void *h,
                           float *logits, int64_t ldl, hipEvent_t *events)
{
    if (!W || !h || !logits || V <= 0 || d <= 0 || n <= 0 || ldl < V)
        return DS_EINVAL;
    if (d % 64 != 0 || d > 8192 || V > (1 << 30) || n > (1 << 20))
        return DS_ESHAPE;
    return hip_status(ds::dense_head_launch(s, V, d, W, n, h, logits, ldl,
                                            events ? events[0] : nullptr,
                                            events ? events[1] : nullptr));
}

ds_status ds_router_labels(hipStream_t s, int n, int V, int M, int L, const float *logits,
                           int64_t ldl, const int32_t *cluster_of, uint8_t *labels)
{
    if (!logits || !cluster_of || !labels || n <= 0 || V <= 0 || M <= 0 || L < 0 || ldl < V)
        return DS_EINVAL;
    if (M > DS_MAX_CLUSTERS || n > (1 << 30))
        return DS_ESHAPE;
    return hip_status(ds::topl_labels_launch(s, n, V, M, L, logits, ldl, cluster_of, labels));
}

size_t ds_router_train_workspace_bytes(int n, int r, int M)
{
    if (n <= 0 || r <= 0 || M <= 0)
        return 0;
    return ds::router_train_ws_bytes(n, r, M);
}

ds_status ds_router_train_step(hipStream_t s, const ds_router_train_args *a)
{
    if (!a || !a->h || !a->labels || !a->W1 || !a->b1 || !a->W2 || !a->b2 || !a->dW1 ||
        !a->db1 || !a->dW2 || !a->db2 || !a->loss || !a->ws)
        return DS_EINVAL;
    if (a->n <= 0 || a->d <= 0 || a->r <= 0 || a->M <= 0 || a->ldh < a->d)
        return DS_EINVAL;
    if (a->act != DS_RELU && a->act != DS_SILU)
        return DS_EDTYPE;
    if (a->h_dtype != DS_F32 && a->h_dtype != DS_BF16)
        return DS_EDTYPE;
    if ((int64_t)a->n * a->d > (1ll << 31) || (int64_t)a->r * a->d > (1ll << 31) ||
        (int64_t)a->n * a->M > (1ll << 31))
        return DS_ESHAPE;
    if (a->ws_bytes < ds_router_train_workspace_bytes(a->n, a->r, a->M))
        return DS_EINVAL;
    return hip_status(ds::router_train_launch(
        s, a->n, a->d, a->r, a->M, a->act, a->h_dtype == DS_BF16, a->h, a->ldh, a->labels, a->lr,
        a->W1, a->b1, a->W2, a->b2, a->dW1, a->db1, a->dW2, a->db2, a->loss, a->ws));
}

// batched chains with a one-pass second router layer: two slots (positions
// alternate) for that layer's window partials, which the selection adds up
static size_t chain_part_bytes(int B, int r)
{
    return B >= ds::kRouterMfmaMin && B <= ds::kRouterPassCols
               ? 2 * round_up(ds::router_l1_ws_bytes(r), 256)
               : 0;
}

size_t ds_draft_chain_workspace_bytes(int B, int T, int V, int r, int64_t max_len)
{
    if (B <= 0 || T <= 0 || V <= 0 || r <= 0 || max_len <= 0)
        return 0;
    // batched heads: two tile indices (positions alternate; the build of
    // position t+1 writes one while head t reads the other)
    const size_t tix = B >= ds::kUnionMinGroups ? 2 * round_up(ds::tile_index_bytes(B, V), 256) : 0;
    return round_up(ds_router_workspace_bytes(B, r), 256) +
           round_up(ds::build_ws_bytes(B, V), 256) + round_up(ds::sample_ws_bytes(B, max_len), 256) +
           tix + chain_part_bytes(B, r);
}

ds_status ds_draft_chain(hipStream_t hs, hipStream_t rs, const ds_draft_chain_args *a)
{
    if (!a)
        return DS_EINVAL;
    const int B = a->B, T = a->T;
    if (B <= 0 || T <= 0 || !a->max_rows || !a->max_len || !a->budget || !a->u_draft ||
        !a->token)
        return DS_EINVAL;
    // q, or (temperature > 0) the rows' statistics in its place
    if (!a->q && !(a->qstats && a->temperature > 0.0f))
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
    int64_t len_bound = 0;
    for (int t = 0; t < T; ++t) {
        if (a->max_len[t] <= 0 || a->max_len[t] > (1 << 20))
            return DS_ESHAPE;
        len_bound = a->max_len[t] > len_bound ? a->max_len[t] : len_bound;
    }
    if (!a->cluster_of || !a->cluster_index || !a->sl_off || !a->sl_ids || !a->ws ||
        a->capacity < 0 ||
        a->ws_bytes < ds_draft_chain_workspace_bytes(B, T, a->V, a->r, len_bound) ||
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
    if (!a->sync_events)
        return DS_EINVAL;
    for (int k = 0; k <= 2 * T; ++k)
        if (!a->sync_events[k])
            return DS_EINVAL;
    hipEvent_t *const ev = a->sync_events;

    float *z = reinterpret_cast<float *>(a->ws);
    void *bws = reinterpret_cast<char *>(a->ws) + round_up(ds_router_workspace_bytes(B, a->r), 256);
    void *sws = reinterpret_cast<char *>(bws) + round_up(ds::build_ws_bytes(B, a->V), 256);
    char *tws = reinterpret_cast<char *>(sws) + round_up(ds::sample_ws_bytes(B, len_bound), 256);
    // batched bf16 heads run on the matrix cores over the tile index that the
    // build writes alongside each shortlist (slot t % 2); build t+2 reuses a
    // slot only after sample t, hence after head t
    const bool prebuilt = ds::head_mfma_applies(a->dtype == DS_BF16, a->V, a->d, B, 1);
    const size_t tslot = round_up(ds::tile_index_bytes(B, a->V), 256);
    // events: [0, T) build of position t done, [T, 2T) h[t+1] ready (token
    // t-1 sampled) or router of t done, 2T fork
    hipEvent_t fork = ev[2 * T];
    const bool bf16 = a->dtype == DS_BF16;
    const char *hb = reinterpret_cast<const char *>(a->h);
    hipError_t err = hipEventRecord(fork, hs);
    if (err == hipSuccess)
        err = hipStreamWaitEvent(rs, fork, 0);
    // batched: the second router layer stops at its window partials (slot
    // t % 2) and the selection on router_stream adds them up, so its finish
    // leaves head_stream; slot t % 2 is rewritten by router t + 2, which
    // head_stream runs after waiting for build t
    const bool split = prebuilt && chain_part_bytes(B, a->r) > 0 &&
                       ds::router_split_applies(bf16, B, a->r, a->M);
    const size_t pslot = round_up(ds::router_l1_ws_bytes(a->r), 256);
    float *part2 = reinterpret_cast<float *>(tws + (prebuilt ? 2 * tslot : 0));
    const int nwin2 = split ? ds::router_l2_windows(a->r, a->M) : 0;
    auto router_at = [&](hipStream_t st, int t) {  // router layers of position t (reads h[:, t])
        const int64_t rb = (int64_t)t * B;
        if (split)
            return ds::router_launch_split(st, B, a->d, a->r, a->M, a->act,
                                           hb + (size_t)t * a->d * e, ldh, a->W1, a->b1, a->W2, z,
                                           part2 + (t & 1) * (pslot / sizeof(float)));
        return ds::router_launch(st, bf16, B, a->d, a->r, a->M, a->act, hb + (size_t)t * a->d * e,
                                 ldh, a->W1, a->b1, a->W2, a->b2, a->scores + rb * a->M, z);
    };
    auto select_build_at = [&](hipStream_t st, int t) {
        const int64_t rb = (int64_t)t * B;
        hipError_t r =
            split ? ds::select_partials_launch(st, B, a->M, part2 + (t & 1) * (pslot / sizeof(float)),
                                               nwin2, a->b2, a->scores + rb * a->M, a->cluster_size,
                                               a->budget_kind, a->budget + rb, a->sel + rb * a->M,
                                               a->n_sel + rb, a->sl_len + rb)
                  : ds::select_launch(st, B, a->M, a->scores + rb * a->M, a->cluster_size,
                                      a->budget_kind, a->budget + rb, a->sel + rb * a->M,
                                      a->n_sel + rb, a->sl_len + rb);
        if (r == hipSuccess)
            r = ds::build_launch(st, B, a->M, a->V, a->sel + rb * a->M, a->n_sel + rb,
                                 a->cluster_of, a->cluster_index, a->capacity, a->sl_off + rb,
                                 a->sl_ids, a->err_flag, bws,
                                 prebuilt ? reinterpret_cast<ds::TileIx *>(tws + (t & 1) * tslot)
                                          : nullptr);
        return r;
    };
    auto head_sample_at = [&](int t) {
        const int64_t rb = (int64_t)t * B;
        hipEvent_t h0 = a->head_events ? a->head_events[2 * t] : nullptr;
        hipEvent_t h1 = a->head_events ? a->head_events[2 * t + 1] : nullptr;
        const void *Wt = a->W_pos ? a->W_pos[t] : a->W;
        hipError_t r;
        if (prebuilt)
            r = ds::head_union_prebuilt_launch(
                hs, a->V, a->d, Wt, B, hb + (size_t)(t + 1) * a->d * e, ldh, a->sl_off + rb,
                reinterpret_cast<const ds::TileIx *>(tws + (t & 1) * tslot), a->logits, h0, h1);
        else
            r = ds::head_launch(hs, bf16, a->V, a->d, Wt, B, 1, hb + (size_t)(t + 1) * a->d * e,
                                ldh, a->sl_off + rb, a->sl_ids, a->max_rows[t], a->logits, nullptr,
                                h0, h1);
        if (r == hipSuccess && a->q)
            r = ds::sample_launch(hs, B, 1, a->sl_off + rb, a->sl_ids, a->logits, a->temperature,
                                  a->u_draft + rb, a->token + rb, a->q, a->max_len[t], sws);
        else if (r == hipSuccess)
            r = ds::sample_stats_launch(hs, B, 1, a->sl_off + rb, a->sl_ids, a->logits,
                                        a->temperature, a->u_draft + rb, a->token + rb,
                                        reinterpret_cast<ds::QStats *>(a->qstats) + rb,
                                        a->max_len[t], sws);
        return r;
    };
    if (!prebuilt) {
        // events: [0, T) build of position t done, [T, 2T) h[t+1] ready
        // (token t-1 sampled), 2T fork
        for (int t = 0; t < T && err == hipSuccess; ++t) {
            if (t > 0)  // h[t] (H_{t-1}) exists once token t-2 is sampled
                err = hipStreamWaitEvent(rs, ev[T + t - 1], 0);
            if (err == hipSuccess)
                err = router_at(rs, t);
            if (err == hipSuccess)
                err = select_build_at(rs, t);
            if (err == hipSuccess)
                err = hipEventRecord(ev[t], rs);
            // h[t+1] (read by head t and by router t+1) is ready once token
            // t-1 is sampled: the record follows sample t-1 directly, before
            // the head stream waits for build t, so router t+1 may run
            // alongside head t
            if (err == hipSuccess)
                err = hipEventRecord(ev[T + t], hs);
            if (err == hipSuccess)
                err = hipStreamWaitEvent(hs, ev[t], 0);
            if (err == hipSuccess)
                err = head_sample_at(t);
        }
        return hip_status(err);
    }
    // Batched matrix-core heads fill every compute unit, so router kernels
    // beside them wait for the head's workgroups to retire (measured, 32
    // sequences: the first router layer took 90-100 us beside the head, 8.5
    // us alone).  The router layers of position t+1 therefore run on the
    // head stream just before head t (h[:, t+1] exists then: token t-1 is
    // sampled), and only selection and build of t+1 run beside head t.
    // events: [0, T) build of position t done, [T, 2T) router of t done.
    if (err == hipSuccess)
        err = router_at(hs, 0);
    if (err == hipSuccess)
        err = hipEventRecord(ev[T], hs);
    for (int t = 0; t < T && err == hipSuccess; ++t) {
        err = hipStreamWaitEvent(rs, ev[T + t], 0);
        if (err == hipSuccess)
            err = select_build_at(rs, t);
        if (err == hipSuccess)
            err = hipEventRecord(ev[t], rs);
        if (err == hipSuccess && t + 1 < T) {
            err = router_at(hs, t + 1);
            if (err == hipSuccess)
                err = hipEventRecord(ev[T + t + 1], hs);
        }
        if (err == hipSuccess)
            err = hipStreamWaitEvent(hs, ev[t], 0);
        if (err == hipSuccess)
            err = head_sample_at(t);
    }
    return hip_status(err);
}

struct ds_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

ds_status ds_capture_begin(hipStream_t s)
{
    if (!s)
        return DS_EINVAL;  // the legacy default stream cannot be captured
    return hip_status(hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed));
}

ds_status ds_capture_end(hipStream_t s, ds_graph *out)
{
    if (!s || !out)
        return DS_EINVAL;
    *out = nullptr;
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(s, &g);
    if (e != hipSuccess || !g)
        return DS_EHIP;
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(g);
        return DS_EHIP;
    }
    ds_graph h = new (std::nothrow) ds_graph_s{g, x};
    if (!h) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return DS_EHIP;
    }
    *out = h;
    return DS_OK;
}

ds_status ds_graph_launch(ds_graph g, hipStream_t s)
{
    if (!g)
        return DS_EINVAL;
    return hip_status(hipGraphLaunch(g->exec, s));
}

ds_status ds_graph_destroy(ds_graph g)
{
    if (!g)
        return DS_EINVAL;
    hipError_t e1 = hipGraphExecDestroy(g->exec);
    hipError_t e2 = hipGraphDestroy(g->graph);
    delete g;
    return (e1 == hipSuccess && e2 == hipSuccess) ? DS_OK : DS_EHIP;
}

}  // extern "C"
