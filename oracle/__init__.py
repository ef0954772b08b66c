"""CPU oracle for the shortlisted draft head (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrappers over ``dynaspec_oracle.c`` (plain single-threaded C,
fp64 accumulation).  Only the tests, the smoke check and the benchmark's CPU
baseline import this package; the HIP library never does.

Every wrapper takes and returns numpy arrays with the layouts of the library's
C-ABI: bf16 tensors are uint16 bit patterns, shortlist offsets are absolute
(``sl_off[0]`` is the base), verification rows are position-major.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dynaspec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, EINVAL, ECAPACITY = 0, 1, 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, one thread)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = C.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("expected float32 or bf16 bits (uint16), got %s" % a.dtype)


def _c(a, dt=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dt or a.dtype)


def router_score(h, W1, b1, W2, b2, act: int) -> np.ndarray:
    """scores[n][M]; h[n][d], W1[r][d], W2[M][r] (fp32 or bf16 bits)."""
    lib = _load()
    h, W1, W2 = _c(h), _c(W1), _c(W2)
    b1, b2 = _c(b1), _c(b2)
    n, d = h.shape
    r, M = W1.shape[0], W2.shape[0]
    dt = _dtype_code(W1)
    for a in (h, W2) + tuple(x for x in (b1, b2) if x is not None):
        assert _dtype_code(a) == dt
    out = np.empty((n, M), np.float32)
    lib.oracle_router_score(C.c_int(dt), C.c_int(n), C.c_int(d), C.c_int(r), C.c_int(M),
                            C.c_int(act), _p(h), C.c_int64(d), _p(W1), _p(b1), _p(W2), _p(b2),
                            _p(out))
    return out


def select_clusters(scores, cluster_size, kind: int, budget):
    """Returns (sel[n][M] ranked ids padded with -1, n_sel[n], sl_len[n])."""
    lib = _load()
    scores = _c(scores, np.float32)
    n, M = scores.shape
    cs, bud = _c(cluster_size, np.int32), _c(budget, np.int32).reshape(n)
    sel = np.empty((n, M), np.int32)
    n_sel = np.empty(n, np.int32)
    sl_len = np.empty(n, np.int32)
    lib.oracle_select_clusters(C.c_int(n), C.c_int(M), _p(scores), _p(cs), C.c_int(kind),
                               _p(bud), _p(sel), _p(n_sel), _p(sl_len))
    return sel, n_sel, sl_len


def build_shortlist(sel, n_sel, cluster_of, capacity: int | None = None, base: int = 0):
    """Returns (status, sl_off[n+1] int64, sl_ids[capacity] int32)."""
    lib = _load()
    sel = _c(sel, np.int32)
    n, M = sel.shape
    n_sel, cluster_of = _c(n_sel, np.int32), _c(cluster_of, np.int32)
    V = cluster_of.shape[0]
    if capacity is None:
        capacity = base + n * V
    sl_off = np.zeros(n + 1, np.int64)
    sl_off[0] = base
    sl_ids = np.full(max(capacity, 1), -1, np.int32)
    st = lib.oracle_build_shortlist(C.c_int(n), C.c_int(M), C.c_int(V), _p(sel), _p(n_sel),
                                    _p(cluster_of), C.c_int64(capacity), _p(sl_off), _p(sl_ids))
    return int(st), sl_off, sl_ids[:capacity]


def gathered_lm_head(W, h, sl_off, sl_ids):
    """h[G][m][d]; returns the logits buffer (length m*sl_off[G]) in the
    library's layout (group g at m*sl_off[g], [m][len_g])."""
    lib = _load()
    W, h = _c(W), _c(h)
    V, d = W.shape
    G, m, _ = h.shape
    sl_off, sl_ids = _c(sl_off, np.int64), _c(sl_ids, np.int32)
    out = np.full(int(m * sl_off[G]), np.nan, np.float32)
    lib.oracle_gathered_lm_head(C.c_int(_dtype_code(W)), C.c_int(V), C.c_int(d), _p(W),
                                C.c_int(G), C.c_int(m), _p(h), C.c_int64(m * d),
                                _p(sl_off), _p(sl_ids), _p(out))
    return out


def pack_rows(W, ids):
    """out[i] = W[ids[i]] as a new [n][d] array of W's dtype (NaN rows for
    ids outside [0, V))."""
    lib = _load()
    W = _c(W)
    V, d = W.shape
    ids = _c(ids, np.int32)
    out = np.empty((ids.shape[0], d), W.dtype)
    lib.oracle_pack_rows(C.c_int(_dtype_code(W)), C.c_int(V), C.c_int(d), _p(W),
                         C.c_int64(ids.shape[0]), _p(ids), _p(out))
    return out


def dense_lm_head(W, h):
    """logits[n][V] for h[n][d] over every row of W."""
    lib = _load()
    W, h = _c(W), _c(h)
    V, d = W.shape
    n = h.shape[0]
    out = np.empty((n, V), np.float32)
    lib.oracle_dense_lm_head(C.c_int(_dtype_code(W)), C.c_int(V), C.c_int(d), _p(W), C.c_int(n),
                             _p(h), C.c_int64(d), _p(out))
    return out


def shortlist_sample(sl_off, sl_ids, logits, u, m: int = 1, temperature: float = 1.0):
    """Returns (token[G*m], q (same layout as logits), tie[G*m] bool)."""
    lib = _load()
    sl_off, sl_ids = _c(sl_off, np.int64), _c(sl_ids, np.int32)
    logits, u = _c(logits, np.float32), _c(u, np.float32).reshape(-1)
    G = sl_off.shape[0] - 1
    assert u.shape[0] == G * m
    token = np.empty(G * m, np.int32)
    q = np.full(logits.shape[0], np.nan, np.float32)
    tie = np.zeros(G * m, np.uint8)
    lib.oracle_shortlist_sample(C.c_int(G), C.c_int(m), _p(sl_off), _p(sl_ids), _p(logits),
                                C.c_float(temperature), _p(u), _p(token), _p(q), _p(tie))
    return token, q, tie.astype(bool)


def target_softmax(logits):
    lib = _load()
    logits = _c(logits, np.float32)
    V = logits.shape[-1]
    rows = logits.size // V
    p = np.empty_like(logits)
    lib.oracle_target_softmax(C.c_int(rows), C.c_int(V), _p(logits), _p(p))
    return p


def verify_reject(draft, sl_off, sl_ids, q, p, u_acc, u_fin):
    """draft[T][B], sl_off[T*B+1] (row t*B+b), p[B][T+1][V], u_acc[T][B],
    u_fin[B].  Returns (n_acc[B], out[B][T+1], tie[B] bool)."""
    lib = _load()
    draft = _c(draft, np.int32)
    T, B = draft.shape
    p = _c(p, np.float32)
    V = p.shape[-1]
    assert p.shape == (B, T + 1, V)
    sl_off, sl_ids, q = _c(sl_off, np.int64), _c(sl_ids, np.int32), _c(q, np.float32)
    u_acc, u_fin = _c(u_acc, np.float32).reshape(T, B), _c(u_fin, np.float32).reshape(B)
    n_acc = np.empty(B, np.int32)
    out = np.empty((B, T + 1), np.int32)
    tie = np.zeros(B, np.uint8)
    lib.oracle_verify_reject(C.c_int(B), C.c_int(T), C.c_int(V), _p(draft), _p(sl_off),
                             _p(sl_ids), _p(q), _p(p), _p(u_acc), _p(u_fin), _p(n_acc),
                             _p(out), _p(tie))
    return n_acc, out, tie.astype(bool)


# ---------------------------------------------------------------------------
# spherical k-means over the LM-head rows (bf16 W)
# ---------------------------------------------------------------------------
def kmeans_inv_norms(W) -> np.ndarray:
    lib = _load()
    W = _c(W, np.uint16)
    V, d = W.shape
    out = np.empty(V, np.float32)
    lib.oracle_kmeans_inv_norms(C.c_int(V), C.c_int(d), _p(W), _p(out))
    return out


def kmeans_assign(W, Cb):
    """(assign [V] int32, score [V] fp32, tie [V] bool) for bf16 W [V][d]
    and bf16 centroids Cb [M][d]."""
    lib = _load()
    W, Cb = _c(W, np.uint16), _c(Cb, np.uint16)
    V, d = W.shape
    M = Cb.shape[0]
    assign = np.empty(V, np.int32)
    score = np.empty(V, np.float32)
    tie = np.empty(V, np.uint8)
    lib.oracle_kmeans_assign(C.c_int(V), C.c_int(d), _p(W), C.c_int(M), _p(Cb), _p(assign),
                             _p(score), _p(tie))
    return assign, score, tie.astype(bool)


def kmeans_update(W, inv_norm, assign, C_prev):
    """(C_out [M][d] fp32, size [M] int32, norm [M] fp64)."""
    lib = _load()
    W = _c(W, np.uint16)
    V, d = W.shape
    C_prev = _c(C_prev, np.float32)
    M = C_prev.shape[0]
    inv_norm, assign = _c(inv_norm, np.float32), _c(assign, np.int32)
    C_out = np.empty((M, d), np.float32)
    size = np.empty(M, np.int32)
    norm = np.empty(M, np.float64)
    lib.oracle_kmeans_update(C.c_int(V), C.c_int(d), _p(W), _p(inv_norm), C.c_int(M), _p(assign),
                             _p(C_prev), _p(C_out), _p(size), _p(norm))
    return C_out, size, norm


def verify_tree(parent, token, sl_off, sl_ids, q, p, u_acc, u_fin):
    """Tree verification (multi-step speculative sampling).  Nodes 0..m per
    sequence, node 0 the root; parent, token, u_acc [B][m] describe drafted
    nodes 1..m (index i-1 for node i); q in the sampler layout, row i-1 the
    proposal of node i; p [B][m+1][V].  Returns (n_acc [B], out [B][m+1],
    path [B][m], tie [B] bool)."""
    lib = _load()
    parent, token = _c(parent, np.int32), _c(token, np.int32)
    B, m = parent.shape
    p = _c(p, np.float32)
    V = p.shape[-1]
    assert p.shape == (B, m + 1, V)
    sl_off, sl_ids, q = _c(sl_off, np.int64), _c(sl_ids, np.int32), _c(q, np.float32)
    u_acc, u_fin = _c(u_acc, np.float32), _c(u_fin, np.float32)
    n_acc = np.empty(B, np.int32)
    out = np.empty((B, m + 1), np.int32)
    path = np.empty((B, m), np.int32)
    tie = np.empty(B, np.uint8)
    lib.oracle_verify_tree(C.c_int(B), C.c_int(m), C.c_int(V), _p(parent), _p(token), _p(sl_off),
                           _p(sl_ids), _p(q), _p(p), _p(u_acc), _p(u_fin), _p(n_acc), _p(out),
                           _p(path), _p(tie))
    return n_acc, out, path, tie.astype(bool)


def topl_labels(logits, cluster_of, M: int, L: int):
    """labels[n][M] uint8: cluster c is positive iff it holds one of the
    top-L tokens of the row (logit desc, id asc)."""
    lib = _load()
    logits = _c(logits, np.float32)
    n, V = logits.shape
    cluster_of = _c(cluster_of, np.int32)
    out = np.empty((n, M), np.uint8)
    lib.oracle_topl_labels(C.c_int(n), C.c_int(V), C.c_int(M), C.c_int(L), _p(logits),
                           C.c_int64(V), _p(cluster_of), _p(out))
    return out


def router_train_step(h, labels, W1, b1, W2, b2, act: int, lr: float):
    """One SGD step; returns (loss, grads dict (float64), new params dict
    (float32)).  h[n][d] fp32 or bf16 bits; params fp32."""
    lib = _load()
    h = _c(h)
    n, d = h.shape
    W1, b1, W2, b2 = (np.array(x, dtype=np.float32, copy=True) for x in (W1, b1, W2, b2))
    r, M = W1.shape[0], W2.shape[0]
    labels = _c(labels, np.uint8)
    g = {"W1": np.empty((r, d)), "b1": np.empty(r), "W2": np.empty((M, r)), "b2": np.empty(M)}
    loss = C.c_double()
    lib.oracle_router_train_step(C.c_int(_dtype_code(h)), C.c_int(n), C.c_int(d), C.c_int(r),
                                 C.c_int(M), C.c_int(act), _p(h), C.c_int64(d), _p(labels),
                                 C.c_float(lr), _p(W1), _p(b1), _p(W2), _p(b2), _p(g["W1"]),
                                 _p(g["b1"]), _p(g["W2"]), _p(g["b2"]), C.byref(loss))
    return loss.value, g, {"W1": W1, "b1": b1, "W2": W2, "b2": b2}
