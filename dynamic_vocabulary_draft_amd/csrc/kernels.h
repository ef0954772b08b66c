// Internal launchers, one per kernel family (each defined next to its
// kernels).  Arguments are validated by the C-ABI layer before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds {

// workspace z: n*r floats, then (n >= kRouterMfmaMin, for bf16 routers) the
// first layer's window partial sums, router_l1_ws_bytes(r) bytes
constexpr int kRouterMfmaMin = 8;
size_t router_ws_bytes(int n, int r);
hipError_t router_launch(hipStream_t s, bool bf16, int n, int d, int r, int M, int act,
                         const void *h, int64_t ldh, const void *W1, const void *b1,
                         const void *W2, const void *b2, float *scores, float *z);
// first layer on the matrix cores (bf16, d <= 8192): z = act(W1 h + b1) via
// k-window partial sums in part (router_l1_ws_bytes(r) bytes)
size_t router_l1_ws_bytes(int r);
hipError_t router_l1_mfma_launch(hipStream_t s, int n, int d, int r, int act, const void *h,
                                 int64_t ldh, const void *W1, const void *b1, float *z, float *part);
// second layer on the matrix cores (bf16 W2, r % 8 == 0, window partials
// within router_l1_ws_bytes(r)): scores = W2 z + b2, z fp32 split exactly
// into three bf16 pieces; part as above
bool router_l2_mfma_applies(int r, int M);
hipError_t router_l2_mfma_launch(hipStream_t s, int n, int r, int M, const void *z,
                                 const void *W2, const void *b2, float *scores, float *part);
// inputs per column pass of the matrix-core router layers
constexpr int kRouterPassCols = 64;
// the second layer's k-windows (0: not on the matrix cores) and, for one
// column pass (n <= kRouterPassCols), its window partials alone:
// part[w][c][o] for window w < router_l2_windows(r, M), input c, score o
// (row stride M, window stride kRouterPassCols * M); score o of input c is
// then the sum over w in order, plus b2[o] -- what router_l2_mfma_launch's
// finish computes
int router_l2_windows(int r, int M);
hipError_t router_l2_mfma_partials(hipStream_t s, int n, int r, int M, const void *z,
                                   const void *W2, float *part);
// the router up to the second layer's window partials (bf16, kRouterMfmaMin
// <= n <= kRouterPassCols, second layer on the matrix cores): z as in
// router_launch, the partials into part2 (router_l1_ws_bytes(r) bytes
// suffice); select_partials_launch adds them up
bool router_split_applies(bool bf16, int n, int r, int M);
hipError_t router_launch_split(hipStream_t s, int n, int d, int r, int M, int act, const void *h,
                               int64_t ldh, const void *W1, const void *b1, const void *W2,
                               float *z, float *part2);

// selection from the router's second-layer window partials (nwin windows,
// layout of router_l2_mfma_partials, bias b2): every score is formed in the
// order of router_l2_mfma_launch's finish, written to scores, and selected
hipError_t select_partials_launch(hipStream_t s, int n, int M, const float *part, int nwin,
                                  const void *b2, float *scores, const int32_t *cluster_size,
                                  int kind, const int32_t *budget, int32_t *sel, int32_t *n_sel,
                                  int32_t *sl_len);
hipError_t select_launch(hipStream_t s, int n, int M, const float *scores,
                         const int32_t *cluster_size, int kind, const int32_t *budget,
                         int32_t *sel, int32_t *n_sel, int32_t *sl_len);

// build: per-cluster chunk-prefix index (built once), then compaction
constexpr int kBuildChunk = 4096;  // tokens per workgroup
size_t index_bytes(int M, int V);
hipError_t index_launch(hipStream_t s, int M, int V, const int32_t *cluster_of, int32_t *index,
                        int32_t *err_flag);
size_t build_ws_bytes(int n, int V);

// Tile index of a set of ascending shortlists, per row g and 32-token tile t
// (t = 0..nt, nt = ceil(V/32), row stride nt + 1): start = the first
// position j of S_g with S_g[j] >= 32*t, mask = the offsets y - 32*t of the
// tile's ids y < V on S_g.  The batched matrix-core head reads it.
struct TileIx {
    int32_t start;
    uint32_t mask;
};

// tix (may be null): the build also writes the tile index of the rows it
// builds for tiles 0..nt-1 (the head reads no other)
hipError_t build_launch(hipStream_t s, int n, int M, int V, const int32_t *sel,
                        const int32_t *n_sel, const int32_t *cluster_of, const int32_t *index,
                        int64_t capacity, int64_t *sl_off, int32_t *sl_ids, int32_t *err_flag,
                        void *ws, TileIx *tix = nullptr);

// gathered head: GEMV kernel (few head rows, few groups or fp32), or the
// matrix-core kernels (bf16 with >= kUnionMinGroups single-row groups, or
// >= kGatheredMinRows head rows per group)
constexpr int kUnionMinGroups = 8;
constexpr int kGatheredMinRows = 8;
size_t head_ws_bytes(int G, int m, int V);
bool head_mfma_applies(bool bf16, int V, int d, int G, int m);
// t0 / t1 (may be null): timing events stamped at the start of the first
// and the end of the last kernel of the head
hipError_t head_mfma_launch(hipStream_t s, int V, int d, const void *W, int G, int m,
                            const void *h, int64_t ldh_g, const int64_t *sl_off,
                            const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                            hipEvent_t t0, hipEvent_t t1);
// batched matrix-core head (head_mfma_applies with m = 1) over shortlists
// whose tile index tix the build already wrote: no index pass
size_t tile_index_bytes(int G, int V);
hipError_t head_union_prebuilt_launch(hipStream_t s, int V, int d, const void *W, int G,
                                      const void *h, int64_t ldh_g, const int64_t *sl_off,
                                      const TileIx *tix, float *logits, hipEvent_t t0,
                                      hipEvent_t t1);
hipError_t head_launch(hipStream_t s, bool bf16, int V, int d, const void *W, int G, int m,
                       const void *h, int64_t ldh_g, const int64_t *sl_off,
                       const int32_t *sl_ids, int64_t max_rows, float *logits, void *ws,
                       hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// spherical k-means over W's rows (bf16)
hipError_t kmeans_inv_norm_launch(hipStream_t s, int V, int d, const void *W, float *inv_norm);
size_t kmeans_assign_ws_bytes(int V);
hipError_t kmeans_assign_launch(hipStream_t s, int V, int d, const void *W, int M, const void *C,
                                int32_t *assign, float *score, void *ws, hipEvent_t t0,
                                hipEvent_t t1);
size_t kmeans_update_ws_bytes(int V, int d, int M);
hipError_t kmeans_update_launch(hipStream_t s, int V, int d, const void *W, const float *inv_norm,
                                int M, const int32_t *assign, const float *C_prev, float *C_out,
                                void *C_out_bf16, int32_t *size, double *norm, int32_t *err_flag,
                                void *ws);

// static shortlist slab: out[i] = W[ids[i]] (NaN row for ids outside [0, V))
hipError_t pack_launch(hipStream_t s, bool bf16, int V, int d, const void *W, int64_t n,
                       const int32_t *ids, void *out);

size_t sample_ws_bytes(int64_t rows, int64_t max_len);
hipError_t sample_launch(hipStream_t s, int G, int m, const int64_t *sl_off,
                         const int32_t *sl_ids, const float *logits, float temperature,
                         const float *u, int32_t *token, float *q, int64_t max_len, void *ws);
// A draft row's statistics in place of its q (temperature > 0): q_j =
// (float)(exp((l_j - M) / T) * rZ) from the row's logits l, the same
// expression and the same bits as the sampler's q (q_elem in dist.h).  An
// empty row has rZ = 0.
struct QStats {
    float M;
    int32_t pad;
    double rZ;
};
// the draw of sample_launch without writing q: one workgroup per row after
// the chunk statistics; the row's statistics go to qs[row]
hipError_t sample_stats_launch(hipStream_t s, int G, int m, const int64_t *sl_off,
                               const int32_t *sl_ids, const float *logits, float temperature,
                               const float *u, int32_t *token, QStats *qs, int64_t max_len,
                               void *ws);

size_t softmax_ws_bytes(int64_t rows, int64_t V);
hipError_t softmax_launch(hipStream_t s, int rows, int V, const float *logits, float *p, void *ws);
// the softmax's first pass alone: per 4096-element segment of every row its
// max (fp32) and sum of exp(l - max) (fp64), laid out in ws as
// [rows][nseg] sums then [rows][nseg] maxima (softmax_ws_bytes)
int64_t softmax_segments(int64_t V);
hipError_t softmax_stats_launch(hipStream_t s, int rows, int V, const float *logits, void *ws);

size_t verify_ws_bytes(int B, int T, int V);
hipError_t verify_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                         const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                         const float *p, const float *u_acc, const float *u_fin, int32_t *n_acc,
                         int32_t *out, void *ws);
// the same verification from target logits: the softmax statistics pass,
// then p computed where it is read (bit-identical to softmax_launch's p)
size_t verify_logits_ws_bytes(int B, int T, int V);
hipError_t verify_logits_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                const int64_t *sl_off, const int32_t *sl_ids, const float *q,
                                const float *logits, const float *u_acc, const float *u_fin,
                                int32_t *n_acc, int32_t *out, void *ws);
// the same with q taken from the draft logits and their rows' statistics
// (sample_stats_launch; draft row t * B + b), workspace as verify_logits
hipError_t verify_logits_qstats_launch(hipStream_t s, int B, int T, int V, const int32_t *draft,
                                       const int64_t *sl_off, const int32_t *sl_ids,
                                       const float *draft_logits, const QStats *qs,
                                       float temperature, const float *logits,
                                       const float *u_acc, const float *u_fin, int32_t *n_acc,
                                       int32_t *out, void *ws);

hipError_t dense_head_launch(hipStream_t s, int V, int d, const void *W, int n, const void *h,
                             float *logits, int64_t ldl, hipEvent_t t0 = nullptr,
                             hipEvent_t t1 = nullptr);
hipError_t topl_labels_launch(hipStream_t s, int n, int V, int M, int L, const float *logits,
                              int64_t ldl, const int32_t *cluster_of, uint8_t *labels);
size_t router_train_ws_bytes(int n, int r, int M);
hipError_t router_train_launch(hipStream_t s, int n, int d, int r, int M, int act, bool h_bf16,
                               const void *h, int64_t ldh, const uint8_t *labels, float lr,
                               float *W1, float *b1, float *W2, float *b2, float *dW1,
                               float *db1, float *dW2, float *db2, double *loss, void *ws);

size_t verify_tree_ws_bytes(int B, int m, int V, int64_t max_len);
// tree verification from target logits [B][m+1][V]: the softmax statistics
// pass, the row normalisers, then the same kernels with every target value
// taken as the softmax would write it
size_t verify_tree_logits_ws_bytes(int B, int m, int V, int64_t max_len);
hipError_t verify_tree_logits_launch(hipStream_t s, int B, int m, int V, const int32_t *parent,
                                     const int32_t *token, const int64_t *sl_off,
                                     const int32_t *sl_ids, const float *q, const float *logits,
                                     const float *u_acc, const float *u_fin, int64_t max_len,
                                     int32_t *n_acc, int32_t *out, int32_t *path, void *ws,
                                     hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// tree verification with q from the draft logits and their rows' statistics
// (sample_stats_launch; draft row b * m + node), workspace as
// verify_tree_logits
hipError_t verify_tree_logits_qstats_launch(hipStream_t s, int B, int m, int V,
                                            const int32_t *parent, const int32_t *token,
                                            const int64_t *sl_off, const int32_t *sl_ids,
                                            const float *draft_logits, const QStats *qs,
                                            float temperature, const float *logits,
                                            const float *u_acc, const float *u_fin,
                                            int64_t max_len, int32_t *n_acc, int32_t *out,
                                            int32_t *path, void *ws, hipEvent_t t0 = nullptr,
                                            hipEvent_t t1 = nullptr);
hipError_t verify_tree_launch(hipStream_t s, int B, int m, int V, const int32_t *parent,
                              const int32_t *token, const int64_t *sl_off, const int32_t *sl_ids,
                              const float *q, const float *p, const float *u_acc,
                              const float *u_fin, int64_t max_len, int32_t *n_acc, int32_t *out,
                              int32_t *path, void *ws, hipEvent_t t0 = nullptr,
                              hipEvent_t t1 = nullptr);

}  // namespace ds
