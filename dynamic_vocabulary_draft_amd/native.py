"""ctypes binding of libdynaspec.so (the C-ABI in include/dynaspec.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and sizes to the library, and
raises DynaspecError on a non-zero status.  No computation happens here, and
there is no fallback: if the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdynaspec.so")

F32, BF16 = 0, 1
RELU, SILU = 0, 1
BUDGET_CLUSTERS, BUDGET_TOKENS = 0, 1
STATUS = {0: "DS_OK", 1: "DS_EINVAL", 2: "DS_EDTYPE", 3: "DS_ESHAPE", 4: "DS_ECAPACITY",
          5: "DS_EHIP"}

_vp, _i, _i64, _f, _sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t


class DynaspecError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(code, "?"), code))
        self.code = code


class RouterTrainArgs(C.Structure):
    """Mirror of ds_router_train_args."""
    _fields_ = [("n", _i), ("d", _i), ("r", _i), ("M", _i), ("act", _i), ("h_dtype", _i),
                ("h", _vp), ("ldh", _i64), ("labels", _vp), ("lr", _f),
                ("W1", _vp), ("b1", _vp), ("W2", _vp), ("b2", _vp),
                ("dW1", _vp), ("db1", _vp), ("dW2", _vp), ("db2", _vp),
                ("loss", _vp), ("ws", _vp), ("ws_bytes", _sz)]


class ChainArgs(C.Structure):
    """Mirror of ds_draft_chain_args."""
    _fields_ = [("B", _i), ("T", _i), ("V", _i), ("d", _i), ("r", _i), ("M", _i),
                ("dtype", _i), ("act", _i), ("budget_kind", _i), ("temperature", _f),
                ("W", _vp), ("W1", _vp), ("b1", _vp), ("W2", _vp), ("b2", _vp),
                ("cluster_of", _vp), ("cluster_index", _vp), ("cluster_size", _vp), ("h", _vp),
                ("budget", _vp),
                ("u_draft", _vp), ("capacity", _i64), ("max_rows", _vp), ("max_len", _vp),
                ("scores", _vp), ("sel", _vp), ("n_sel", _vp), ("sl_len", _vp),
                ("sl_off", _vp), ("sl_ids", _vp), ("logits", _vp), ("q", _vp),
                ("token", _vp), ("err_flag", _vp), ("ws", _vp), ("ws_bytes", _sz),
                ("W_pos", _vp), ("head_events", _vp), ("sync_events", _vp),
                ("qstats", _vp)]


_SIGS = {
    "ds_status_string": (C.c_char_p, [_i]),
    "ds_version": (C.c_char_p, []),
    "ds_router_workspace_bytes": (_sz, [_i, _i]),
    "ds_router_score": (_i, [_vp, _i, _i, _i, _i, _i, _i, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                             _vp, _sz]),
    "ds_select_clusters": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp]),
    "ds_cluster_index_bytes": (_sz, [_i, _i]),
    "ds_cluster_index": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "ds_build_workspace_bytes": (_sz, [_i, _i]),
    "ds_build_shortlist": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                _sz]),
    "ds_head_workspace_bytes": (_sz, [_i, _i, _i]),
    "ds_gathered_lm_head": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _vp, _i64, _vp, _vp, _i64, _vp, _vp,
                                 _sz]),
    "ds_gathered_lm_head_timed": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _vp, _i64, _vp, _vp, _i64, _vp,
                                       _vp, _sz, _vp, _vp]),
    "ds_pack_rows": (_i, [_vp, _i, _i, _i, _vp, _i64, _vp, _vp]),
    "ds_kmeans_inv_norms": (_i, [_vp, _i, _i, _vp, _vp]),
    "ds_kmeans_assign_workspace_bytes": (_sz, [_i]),
    "ds_kmeans_assign": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "ds_kmeans_update_workspace_bytes": (_sz, [_i, _i, _i]),
    "ds_kmeans_update": (_i, [_vp, _i, _i, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _sz]),
    "ds_sample_workspace_bytes": (_sz, [_i, _i, _i64]),
    "ds_shortlist_sample": (_i, [_vp, _i, _i, _vp, _vp, _vp, _f, _vp, _i64, _vp, _vp, _vp, _sz]),
    "ds_shortlist_sample_stats": (_i, [_vp, _i, _i, _vp, _vp, _vp, _f, _vp, _i64, _vp, _vp, _vp,
                                       _sz]),
    "ds_verify_reject_logits_qstats": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _f, _vp,
                                            _vp, _vp, _vp, _vp, _vp, _sz]),
    "ds_verify_tree_logits_qstats": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp,
                                          _vp, _vp, _i64, _vp, _vp, _vp, _vp, _sz]),
    "ds_softmax_workspace_bytes": (_sz, [_i, _i]),
    "ds_target_softmax": (_i, [_vp, _i, _i, _vp, _vp, _vp, _sz]),
    "ds_verify_workspace_bytes": (_sz, [_i, _i, _i]),
    "ds_verify_reject": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _sz]),
    "ds_verify_logits_workspace_bytes": (_sz, [_i, _i, _i]),
    "ds_verify_reject_logits": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _sz]),
    "ds_verify_reject_noalloc": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp]),
    "ds_verify_tree_logits_workspace_bytes": (_sz, [_i, _i, _i, _i64]),
    "ds_verify_tree_logits": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _i64, _vp, _vp, _vp, _vp, _sz]),
    "ds_verify_tree_workspace_bytes": (_sz, [_i, _i, _i, _i64]),
    "ds_verify_tree": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                            _vp, _vp, _vp, _sz]),
    "ds_dense_lm_head": (_i, [_vp, _i, _i, _vp, _i, _vp, _vp, _i64, _vp]),
    "ds_router_labels": (_i, [_vp, _i, _i, _i, _i, _vp, _i64, _vp, _vp]),
    "ds_router_train_workspace_bytes": (_sz, [_i, _i, _i]),
    "ds_router_train_step": (_i, [_vp, C.POINTER(RouterTrainArgs)]),
    "ds_draft_chain_workspace_bytes": (_sz, [_i, _i, _i, _i, _i64]),
    "ds_draft_chain": (_i, [_vp, _vp, C.POINTER(ChainArgs)]),
    "ds_capture_begin": (_i, [_vp]),
    "ds_capture_end": (_i, [_vp, C.POINTER(_vp)]),
    "ds_graph_launch": (_i, [_vp, _vp]),
    "ds_graph_destroy": (_i, [_vp]),
}

SYMBOLS = tuple(_SIGS)


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdynaspec.so is not built (run python -m "
                          "dynamic_vocabulary_draft_amd.build); there is no fallback path")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class HipEvents:
    """HIP events created and destroyed through the HIP runtime (torch's
    Event objects only see torch's own streams, and the library takes raw
    hipEvent_t handles).  ``array(n)`` returns a ctypes array of n new
    handles; ``close()`` destroys every event made here."""

    _hip = None

    def __init__(self):
        if HipEvents._hip is None:
            hip = C.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
            hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
            hip.hipEventDestroy.argtypes = [C.c_void_p]
            HipEvents._hip = hip
        self.hip = HipEvents._hip
        self.made = []

    def array(self, n: int, timing: bool = True):
        arr = (C.c_void_p * n)()
        flags = 0 if timing else 2  # hipEventDisableTiming
        for i in range(n):
            e = C.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(C.byref(e), flags)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
            arr[i] = e.value
            self.made.append(e.value)
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        rc = self.hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(C.c_void_p(e))
        self.made = []


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _s(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("expected bf16 or fp32, got %s" % t.dtype)


def _ld(t: torch.Tensor, dim: int = 0) -> int:
    """Leading dimension (elements between consecutive indices of `dim`); a
    size-1 dimension may carry any stride, so it is taken from the shape."""
    if t.shape[dim] > 1:
        return t.stride(dim)
    n = 1
    for s in t.shape[dim + 1:]:
        n *= s
    return n


def _check(name: str, code: int) -> None:
    if code != 0:
        raise DynaspecError(name, code)


def version() -> str:
    return lib.ds_version().decode()


def router_workspace_bytes(n: int, r: int) -> int:
    return int(lib.ds_router_workspace_bytes(n, r))


def build_workspace_bytes(n: int, V: int) -> int:
    return int(lib.ds_build_workspace_bytes(n, V))


def draft_chain_workspace_bytes(B: int, T: int, V: int, r: int, max_len: int) -> int:
    return int(lib.ds_draft_chain_workspace_bytes(B, T, V, r, int(max_len)))


def sample_workspace_bytes(G: int, m: int, max_len: int) -> int:
    return int(lib.ds_sample_workspace_bytes(G, m, int(max_len)))


def softmax_workspace_bytes(rows: int, V: int) -> int:
    return int(lib.ds_softmax_workspace_bytes(rows, V))


def verify_workspace_bytes(B: int, T: int, V: int) -> int:
    return int(lib.ds_verify_workspace_bytes(B, T, V))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace of at least nbytes bytes."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def router_score(h, W1, b1, W2, b2, act, scores, ws, *, n=None, ldh=None, stream=None):
    """scores[n][M] <- router(h rows); h row i at h + i*ldh elements."""
    n = h.shape[0] if n is None else n
    ldh = _ld(h) if ldh is None else ldh
    r, d = W1.shape
    M = W2.shape[0]
    _check("ds_router_score", lib.ds_router_score(
        _s(stream), _dt(W1), n, d, r, M, act, _p(h), ldh, _p(W1), _p(b1), _p(W2), _p(b2),
        _p(scores), _p(ws), _nbytes(ws)))


def select_clusters(scores, cluster_size, kind, budget, sel, n_sel, sl_len, *, stream=None):
    n, M = scores.shape
    _check("ds_select_clusters", lib.ds_select_clusters(
        _s(stream), n, M, _p(scores), _p(cluster_size), kind, _p(budget), _p(sel), _p(n_sel),
        _p(sl_len)))


def cluster_index_bytes(M: int, V: int) -> int:
    return int(lib.ds_cluster_index_bytes(M, V))


def cluster_index(cluster_of, M, index=None, err_flag=None, *, stream=None):
    """The per-chunk prefix counts of every cluster (int32 [(nchunks+1)][M])."""
    V = cluster_of.shape[0]
    if index is None:
        index = torch.empty(cluster_index_bytes(M, V) // 4, dtype=torch.int32,
                            device=cluster_of.device)
    _check("ds_cluster_index", lib.ds_cluster_index(_s(stream), M, V, _p(cluster_of), _p(index),
                                                    _p(err_flag)))
    return index


def build_shortlist(sel, n_sel, cluster_of, index, capacity, sl_off, sl_ids, err_flag, ws, *,
                    stream=None):
    n, M = sel.shape
    _check("ds_build_shortlist", lib.ds_build_shortlist(
        _s(stream), n, M, cluster_of.shape[0], _p(sel), _p(n_sel), _p(cluster_of), _p(index),
        int(capacity), _p(sl_off), _p(sl_ids), _p(err_flag), _p(ws), _nbytes(ws)))


def head_workspace_bytes(G: int, m: int, V: int) -> int:
    return int(lib.ds_head_workspace_bytes(G, m, V))


def gathered_lm_head(W, h, sl_off, sl_ids, max_rows, logits, ws=None, *, G=None, m=None,
                     ldh_g=None, stream=None, events=None):
    """h is [G][m][d] (or pass G, m, ldh_g for a strided view).  ws: at least
    head_workspace_bytes(G, m, V) bytes (allocated here when None).  events:
    optional (start, stop) raw hipEvent_t handles stamped at the head
    kernels' own start and end (ds_gathered_lm_head_timed)."""
    V, d = W.shape
    if G is None:
        G, m = h.shape[0], h.shape[1]
        ldh_g = _ld(h)
    if ws is None:
        ws = workspace(head_workspace_bytes(G, m, V), W.device)
    args = (_s(stream), _dt(W), V, d, _p(W), G, m, _p(h), ldh_g, _p(sl_off), _p(sl_ids),
            int(max_rows), _p(logits), _p(ws), _nbytes(ws))
    if events is None:
        _check("ds_gathered_lm_head", lib.ds_gathered_lm_head(*args))
    else:
        _check("ds_gathered_lm_head_timed", lib.ds_gathered_lm_head_timed(
            *args, C.c_void_p(events[0]), C.c_void_p(events[1])))


def pack_rows(W, ids, out, *, stream=None):
    """out[i] = W[ids[i]] (NaN rows for ids outside [0, V))."""
    V, d = W.shape
    _check("ds_pack_rows", lib.ds_pack_rows(_s(stream), _dt(W), V, d, _p(W), ids.numel(),
                                            _p(ids), _p(out)))


def kmeans_inv_norms(W, inv_norm, *, stream=None):
    V, d = W.shape
    _check("ds_kmeans_inv_norms", lib.ds_kmeans_inv_norms(_s(stream), V, d, _p(W), _p(inv_norm)))


def kmeans_assign(W, Cb, assign, score, ws=None, *, stream=None, events=None):
    """W [V][d] bf16, Cb [M][d] bf16 centroids -> assign [V] int32, score [V]
    fp32.  events: optional (start, stop) raw hipEvent_t handles."""
    V, d = W.shape
    M = Cb.shape[0]
    if ws is None:
        ws = workspace(lib.ds_kmeans_assign_workspace_bytes(V), W.device)
    ev = (None, None) if events is None else (C.c_void_p(events[0]), C.c_void_p(events[1]))
    _check("ds_kmeans_assign", lib.ds_kmeans_assign(
        _s(stream), V, d, _p(W), M, _p(Cb), _p(assign), _p(score), _p(ws), _nbytes(ws), *ev))


def kmeans_update_workspace_bytes(V: int, d: int, M: int) -> int:
    return lib.ds_kmeans_update_workspace_bytes(V, d, M)


def kmeans_update(W, inv_norm, assign, C_prev, C_out, C_out_bf16, size, norm, ws=None, *,
                  err_flag=None, stream=None):
    V, d = W.shape
    M = C_prev.shape[0]
    if ws is None:
        ws = workspace(kmeans_update_workspace_bytes(V, d, M), W.device)
    _check("ds_kmeans_update", lib.ds_kmeans_update(
        _s(stream), V, d, _p(W), _p(inv_norm), M, _p(assign), _p(C_prev), _p(C_out),
        _p(C_out_bf16), _p(size), _p(norm), _p(err_flag), _p(ws), _nbytes(ws)))


def shortlist_sample(sl_off, sl_ids, logits, temperature, u, token, q, ws, *, max_len, m=1,
                     stream=None):
    G = sl_off.shape[0] - 1
    _check("ds_shortlist_sample", lib.ds_shortlist_sample(
        _s(stream), G, m, _p(sl_off), _p(sl_ids), _p(logits), float(temperature), _p(u),
        int(max_len), _p(token), _p(q), _p(ws), _nbytes(ws)))


# bytes of one row's statistics (ds_qstats: fp32 M, padding, fp64 1 / Z)
QSTATS_BYTES = 16


def qstats_buffer(rows: int, device="cuda") -> torch.Tensor:
    """Storage for `rows` ds_qstats records."""
    return torch.empty(max(rows, 1) * QSTATS_BYTES, dtype=torch.uint8, device=device)


def shortlist_sample_stats(sl_off, sl_ids, logits, temperature, u, token, qstats, ws, *,
                           max_len, m=1, stream=None):
    """ds_shortlist_sample without q: tokens and per-row statistics."""
    G = sl_off.shape[0] - 1
    _check("ds_shortlist_sample_stats", lib.ds_shortlist_sample_stats(
        _s(stream), G, m, _p(sl_off), _p(sl_ids), _p(logits), float(temperature), _p(u),
        int(max_len), _p(token), _p(qstats), _p(ws), _nbytes(ws)))


def target_softmax(logits, p, ws, *, stream=None):
    V = logits.shape[-1]
    _check("ds_target_softmax", lib.ds_target_softmax(
        _s(stream), logits.numel() // V, V, _p(logits), _p(p), _p(ws), _nbytes(ws)))


def verify_reject(draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out, ws, *, stream=None):
    T, B = draft.shape
    V = p.shape[-1]
    _check("ds_verify_reject", lib.ds_verify_reject(
        _s(stream), B, T, V, _p(draft), _p(sl_off), _p(sl_ids), _p(q), _p(p), _p(u_acc),
        _p(u_fin), _p(n_acc), _p(out), _p(ws), _nbytes(ws)))


def verify_logits_workspace_bytes(B: int, T: int, V: int) -> int:
    return int(lib.ds_verify_logits_workspace_bytes(B, T, V))


def verify_reject_logits(draft, sl_off, sl_ids, q, logits, u_acc, u_fin, n_acc, out, ws, *,
                         stream=None):
    """ds_verify_reject from target logits [B][T+1][V]."""
    T, B = draft.shape
    V = logits.shape[-1]
    _check("ds_verify_reject_logits", lib.ds_verify_reject_logits(
        _s(stream), B, T, V, _p(draft), _p(sl_off), _p(sl_ids), _p(q), _p(logits), _p(u_acc),
        _p(u_fin), _p(n_acc), _p(out), _p(ws), _nbytes(ws)))


def verify_reject_logits_qstats(draft, sl_off, sl_ids, draft_logits, qstats, temperature,
                                logits, u_acc, u_fin, n_acc, out, ws, *, stream=None):
    """verify_reject_logits with q from the draft logits and row statistics."""
    T, B = draft.shape
    V = logits.shape[-1]
    _check("ds_verify_reject_logits_qstats", lib.ds_verify_reject_logits_qstats(
        _s(stream), B, T, V, _p(draft), _p(sl_off), _p(sl_ids), _p(draft_logits), _p(qstats),
        float(temperature), _p(logits), _p(u_acc), _p(u_fin), _p(n_acc), _p(out), _p(ws),
        _nbytes(ws)))


def verify_reject_noalloc(draft, sl_off, sl_ids, q, p, u_acc, u_fin, n_acc, out, *,
                          stream=None):
    """ds_verify_reject without a workspace (the library's static scratch)."""
    T, B = draft.shape
    V = p.shape[-1]
    _check("ds_verify_reject_noalloc", lib.ds_verify_reject_noalloc(
        _s(stream), B, T, V, _p(draft), _p(sl_off), _p(sl_ids), _p(q), _p(p), _p(u_acc),
        _p(u_fin), _p(n_acc), _p(out)))


def verify_tree_workspace_bytes(B: int, m: int, V: int, max_len: int) -> int:
    return int(lib.ds_verify_tree_workspace_bytes(B, m, V, max_len))


def verify_tree(parent, token, sl_off, sl_ids, q, p, u_acc, u_fin, max_len, n_acc, out, path,
                ws, *, stream=None):
    """parent, token, u_acc [B][m] (drafted nodes 1..m); p [B][m+1][V];
    outputs n_acc [B], out [B][m+1], path [B][m]."""
    B, m = parent.shape
    V = p.shape[-1]
    _check("ds_verify_tree", lib.ds_verify_tree(
        _s(stream), B, m, V, _p(parent), _p(token), _p(sl_off), _p(sl_ids), _p(q), _p(p),
        _p(u_acc), _p(u_fin), int(max_len), _p(n_acc), _p(out), _p(path), _p(ws),
        _nbytes(ws)))


def verify_tree_logits_workspace_bytes(B: int, m: int, V: int, max_len: int) -> int:
    return int(lib.ds_verify_tree_logits_workspace_bytes(B, m, V, max_len))


def verify_tree_logits(parent, token, sl_off, sl_ids, q, logits, u_acc, u_fin, max_len, n_acc,
                       out, path, ws, *, stream=None):
    """verify_tree from target logits [B][m+1][V]."""
    B, m = parent.shape
    V = logits.shape[-1]
    _check("ds_verify_tree_logits", lib.ds_verify_tree_logits(
        _s(stream), B, m, V, _p(parent), _p(token), _p(sl_off), _p(sl_ids), _p(q), _p(logits),
        _p(u_acc), _p(u_fin), int(max_len), _p(n_acc), _p(out), _p(path), _p(ws),
        _nbytes(ws)))


def verify_tree_logits_qstats(parent, token, sl_off, sl_ids, draft_logits, qstats, temperature,
                              logits, u_acc, u_fin, max_len, n_acc, out, path, ws, *,
                              stream=None):
    """verify_tree_logits with q from the draft logits and row statistics."""
    B, m = parent.shape
    V = logits.shape[-1]
    _check("ds_verify_tree_logits_qstats", lib.ds_verify_tree_logits_qstats(
        _s(stream), B, m, V, _p(parent), _p(token), _p(sl_off), _p(sl_ids), _p(draft_logits),
        _p(qstats), float(temperature), _p(logits), _p(u_acc), _p(u_fin), int(max_len),
        _p(n_acc), _p(out), _p(path), _p(ws), _nbytes(ws)))


def dense_lm_head(W, h, logits, *, stream=None, events=None):
    """logits [n][V] (fp32, any row stride >= V) = h W^T over every token;
    W [V][d], h [n][d] bf16 with contiguous rows.  events: optional (start,
    stop) raw hipEvent_t handles stamped at the kernel's own start and end."""
    V, d = W.shape
    n = h.shape[0]
    assert h.stride(-1) == 1 and (n == 1 or h.stride(0) == d), "h rows must be contiguous"
    ev = None if events is None else (C.c_void_p * 2)(*events)
    _check("ds_dense_lm_head", lib.ds_dense_lm_head(_s(stream), V, d, _p(W), n, _p(h),
                                                    _p(logits), _ld(logits), ev))


def router_labels(logits, cluster_of, M: int, L: int, labels, *, stream=None):
    """labels [n][M] uint8 from the full drafter's logits [n][V] (fp32)."""
    n, V = logits.shape
    _check("ds_router_labels", lib.ds_router_labels(_s(stream), n, V, M, L, _p(logits),
                                                    _ld(logits), _p(cluster_of), _p(labels)))


def router_train_workspace_bytes(n: int, r: int, M: int) -> int:
    return int(lib.ds_router_train_workspace_bytes(n, r, M))


def router_train_step(h, labels, W1, b1, W2, b2, grads, loss, act: int, lr: float, ws, *,
                      stream=None):
    """One SGD step; W1, b1, W2, b2 (fp32) are updated in place; grads is a
    dict of fp32 tensors W1, b1, W2, b2; loss a 1-element float64 tensor."""
    n, d = h.shape
    r, M = W1.shape[0], W2.shape[0]
    a = RouterTrainArgs(n=n, d=d, r=r, M=M, act=act, h_dtype=_dt(h), h=_p(h), ldh=_ld(h),
                        labels=_p(labels), lr=float(lr), W1=_p(W1), b1=_p(b1), W2=_p(W2),
                        b2=_p(b2), dW1=_p(grads["W1"]), db1=_p(grads["b1"]),
                        dW2=_p(grads["W2"]), db2=_p(grads["b2"]), loss=_p(loss), ws=_p(ws),
                        ws_bytes=_nbytes(ws))
    _check("ds_router_train_step", lib.ds_router_train_step(_s(stream), C.byref(a)))


def draft_chain(args: ChainArgs, head_stream=None, router_stream=None):
    _check("ds_draft_chain", lib.ds_draft_chain(_s(head_stream), _s(router_stream),
                                                C.byref(args)))


class Graph:
    """A captured, instantiated HIP graph (see ds_capture_begin)."""

    def __init__(self, handle: C.c_void_p):
        self._h = handle

    def launch(self, stream=None) -> None:
        _check("ds_graph_launch", lib.ds_graph_launch(self._h, _s(stream)))

    def close(self) -> None:
        if self._h:
            lib.ds_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def capture(fn, stream) -> Graph:
    """Run fn() (which enqueues ds_* calls on `stream`) under graph capture
    and return the instantiated graph.  `stream` must not be the legacy
    default stream."""
    _check("ds_capture_begin", lib.ds_capture_begin(_s(stream)))
    try:
        fn()
    finally:
        h = C.c_void_p()
        code = lib.ds_capture_end(_s(stream), C.byref(h))
    _check("ds_capture_end", code)
    return Graph(h)
