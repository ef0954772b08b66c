"""GPU parity of router training (ds_router_labels, ds_router_train_step)
against the oracle.

Bars: labels bit-exact (integer work on identical fp32 logits; the top-L
order compares the same floats).  The training step computes in fp32 against
the oracle's fp64: loss within 1e-5 relative; every gradient tensor within
GRAD_TOL * max|ref| of the oracle; the updated parameters within
lr * GRAD_TOL * max|grad| plus one fp32 ulp.  GRAD_TOL = 5e-5 bounds fp32
sums of up to 4096 terms (sqrt(4096) * 2^-24 = 3.8e-6 typical relative
error, compounded over the forward and backward products) with margin.
Repeated steps on the same inputs are bit-identical.
"""
import numpy as np
import pytest
import torch

from dynamic_vocabulary_draft_amd import synthetic as syn
from dynamic_vocabulary_draft_amd.pipeline import to_dev

pytestmark = pytest.mark.gpu

GRAD_TOL = 5e-5


@pytest.fixture(scope="module")
def N():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocabulary_draft_amd import native
    return native


def _labels_gpu(N, logits, cluster_of, M, L):
    n = logits.shape[0]
    out = torch.full((n, M), 7, dtype=torch.uint8, device="cuda")
    N.router_labels(to_dev(logits), to_dev(cluster_of), M, L, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n,V,M,L", [(5, 5000, 100, 64), (3, 1000, 17, 1), (4, 777, 33, 780),
                                     (2, 300, 7, 0), (6, 70000, 1024, 200),
                                     (4, 3000, 50, 1024), (3, 5000, 64, 1500),
                                     (4, 128256, 1024, 64)])
def test_router_labels_bit_exact(N, oracle_lib, n, V, M, L):
    """Row 0 ties at the cut (a few thousand candidates at or above the
    bound: the LDS ranking below 2048 of them, the radix select above); row
    2 is all zeros of both signs (every key equal); L = 1024 is the largest
    L ranked in LDS, L = 1500 takes the radix select."""
    g = np.random.default_rng(V + L)
    lg = (g.standard_normal((n, V)) * 2).astype(np.float32)
    lg[0] = g.integers(0, 3, size=V).astype(np.float32)  # ties split at the L-th key
    if n > 2:
        lg[2, : V // 2] = -0.0  # signed zeros compare equal
        lg[2, V // 2:] = 0.0
    cluster_of = g.integers(0, M, size=V).astype(np.int32)
    cluster_of[:: 97] = -1
    got = _labels_gpu(N, lg, cluster_of, M, L)
    ref = oracle_lib.topl_labels(lg, cluster_of, M, L)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("V,pad,shift", [(1003, 1, 0), (4099, 5, 0), (4099, 1, 1), (4, 0, 0)])
def test_router_labels_row_stride(N, oracle_lib, V, pad, shift):
    """Rows inside a wider buffer (row stride V + pad): 16-byte loads with a
    tail of V % 4 elements when every row starts 16-byte aligned, element
    loads when the view starts one element in (shift)."""
    n, M, L = 3, 40, 64
    g = np.random.default_rng(V + pad + shift)
    lg = (g.standard_normal((n, V)) * 2).astype(np.float32)
    lg[1, -3:] = 50.0  # the largest keys sit in the tail
    cluster_of = g.integers(0, M, size=V).astype(np.int32)
    buf = torch.full((n, shift + V + pad), float("nan"), dtype=torch.float32, device="cuda")
    view = buf[:, shift:shift + V]
    view.copy_(to_dev(lg))
    out = torch.full((n, M), 7, dtype=torch.uint8, device="cuda")
    N.router_labels(view, to_dev(cluster_of), M, L, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle_lib.topl_labels(lg, cluster_of, M, L))


def test_router_labels_from_dense_head(N, oracle_lib):
    """Labels of the Llama-shaped head: the full drafter's logits come from
    the dense head (and agree with the gathered head over the whole
    vocabulary within the bf16 bar)."""
    cfg = syn.CONFIGS[1]
    wl = syn.make_workload(1, with_target=False)
    n, V, M, L = 16, cfg.V, cfg.M, 64
    W = to_dev(wl.W)
    h = to_dev(syn.make_train_hidden(cfg, n))
    sl_off = torch.tensor([0, V], dtype=torch.int64, device="cuda")
    sl_ids = torch.arange(V, dtype=torch.int32, device="cuda")
    logits = torch.empty(n * V, dtype=torch.float32, device="cuda")
    N.gathered_lm_head(W, h[None], sl_off, sl_ids, V, logits)
    dense = torch.empty(n, V, dtype=torch.float32, device="cuda")
    N.dense_lm_head(W, h, dense)
    torch.cuda.synchronize()
    assert float((dense - logits.view(n, V)).abs().max()) <= 2e-2
    lg = dense.cpu().numpy()
    got = _labels_gpu(N, lg, wl.cluster_of, M, L)
    assert np.array_equal(got, oracle_lib.topl_labels(lg, wl.cluster_of, M, L))
    assert got.sum(1).min() >= 1 and got.sum(1).max() <= L


def _train_case(n, d, r, M, seed):
    g = np.random.default_rng(seed)
    h = g.standard_normal((n, d)).astype(np.float32)
    W1 = (g.standard_normal((r, d)) / np.sqrt(d)).astype(np.float32)
    b1 = (g.standard_normal(r) * 0.1).astype(np.float32)
    W2 = (g.standard_normal((M, r)) / np.sqrt(r)).astype(np.float32)
    b2 = (g.standard_normal(M) * 0.1).astype(np.float32)
    y = (g.random((n, M)) < 0.05).astype(np.uint8)
    return h, y, W1, b1, W2, b2


def _train_gpu(N, h, y, W1, b1, W2, b2, act, lr, h_bf16):
    n, d = h.shape
    r, M = W1.shape[0], W2.shape[0]
    hd = to_dev(syn.f32_to_bf16_bits(h) if h_bf16 else h)
    P = {k: to_dev(v) for k, v in (("W1", W1), ("b1", b1), ("W2", W2), ("b2", b2))}
    G = {k: torch.full_like(v, float("nan")) for k, v in P.items()}
    loss = torch.full((1,), float("nan"), dtype=torch.float64, device="cuda")
    ws = N.workspace(N.router_train_workspace_bytes(n, r, M))
    N.router_train_step(hd, to_dev(y), P["W1"], P["b1"], P["W2"], P["b2"], G, loss, act, lr, ws)
    torch.cuda.synchronize()
    return (float(loss.item()), {k: v.cpu().numpy() for k, v in G.items()},
            {k: v.cpu().numpy() for k, v in P.items()})


_SMALL = [(37, 264, 136, 100), (8, 520, 72, 1000)]
_CASES = ([(s, a, b) for s in _SMALL for a in (syn.ACT_RELU, syn.ACT_SILU) for b in (False, True)]
          + [((256, 4096, 1024, 1024), syn.ACT_SILU, True)])  # the Llama-shaped router


@pytest.mark.parametrize("shape,act,h_bf16", _CASES)
def test_router_train_step(N, oracle_lib, shape, act, h_bf16):
    n, d, r, M = shape
    h, y, W1, b1, W2, b2 = _train_case(n, d, r, M, seed=n + d + act)
    lr = 0.5
    hin = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(h)) if h_bf16 else h
    loss_ref, g_ref, p_ref = oracle_lib.router_train_step(hin, y, W1, b1, W2, b2, act, lr)
    loss, g, p = _train_gpu(N, h, y, W1, b1, W2, b2, act, lr, h_bf16)
    assert abs(loss - loss_ref) <= 1e-5 * loss_ref
    for k in ("W1", "b1", "W2", "b2"):
        scale = float(np.abs(g_ref[k]).max())
        err = float(np.abs(g[k].astype(np.float64) - g_ref[k]).max())
        assert err <= GRAD_TOL * scale, (k, err, scale)
        ulp = np.spacing(np.abs(p_ref[k])).astype(np.float64)
        perr = np.abs(p[k].astype(np.float64) - p_ref[k].astype(np.float64))
        assert (perr <= float(np.float32(lr)) * GRAD_TOL * scale + ulp).all(), k
    # reproducible bit for bit
    loss2, g2, p2 = _train_gpu(N, h, y, W1, b1, W2, b2, act, lr, h_bf16)
    assert loss2 == loss
    for k in g:
        assert np.array_equal(g2[k], g[k]) and np.array_equal(p2[k], p[k])


@pytest.mark.parametrize("V,d,n", [(5000, 256, 37), (20011, 1024, 300), (1000, 64, 1),
                                   (3000, 192, 40)])
def test_dense_lm_head_parity(N, oracle_lib, V, d, n):
    """The dense head over all V against the oracle (bf16 bar 2e-2), on
    ragged row and column tiles and one to sixteen 64-wide slices."""
    g = np.random.default_rng(V + n)
    W = syn.f32_to_bf16_bits((g.standard_normal((V, d)) * 0.05).astype(np.float32))
    h = syn.f32_to_bf16_bits(g.standard_normal((n, d)).astype(np.float32))
    out = torch.full((n, V + 3), float("nan"), device="cuda")  # a padded row stride
    N.dense_lm_head(to_dev(W), to_dev(h), out[:, :V])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle_lib.dense_lm_head(W, h)
    assert np.abs(got[:, :V].astype(np.float64) - ref).max() <= 2e-2
    assert np.isnan(got[:, V:]).all()  # nothing written past V
