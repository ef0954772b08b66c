"""The allocation-free verifier (ds_verify_reject_noalloc) against
ds_verify_reject, through the C-ABI, on two calls in a row (the second one
smaller, so it runs over the scratch the first one left behind).

Both entry points run the same kernels; the outputs (accepted counts and
emitted tokens, integers) must be identical.  The smaller case is also
checked against the oracle.
"""
import numpy as np
import pytest
import torch

from dynamic_vocabulary_draft_amd import synthetic as syn
from dynamic_vocabulary_draft_amd.pipeline import to_dev

pytestmark = pytest.mark.gpu


def _case(V, T, B, seed):
    """Random ascending shortlists, q a softmax over each, drafts drawn from
    q, targets: half the sequences follow q (acceptances), half N(0, 3)."""
    g = np.random.default_rng(seed)
    lens = g.integers(1, max(2, V // 3), size=T * B)
    sl_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ids = np.concatenate([np.sort(g.choice(V, int(L), replace=False)) for L in lens]).astype(np.int32)
    q = np.empty(int(sl_off[-1]), np.float32)
    lg_all = (g.standard_normal(q.size) * 2).astype(np.float32)
    draft = np.empty((T, B), np.int32)
    tl = (g.standard_normal((B, T + 1, V)) * 3).astype(np.float32)
    for t in range(T):
        for b in range(B):
            r = t * B + b
            lo, hi = sl_off[r], sl_off[r + 1]
            e = np.exp(lg_all[lo:hi].astype(np.float64) - lg_all[lo:hi].max())
            q[lo:hi] = (e / e.sum()).astype(np.float32)
            draft[t, b] = ids[lo + g.choice(hi - lo, p=e / e.sum())]
            if b % 2 == 0:
                tl[b, t] = -4.0
                tl[b, t, ids[lo:hi]] = lg_all[lo:hi]
    p = np.exp(tl - tl.max(axis=-1, keepdims=True))
    p = (p / p.sum(axis=-1, keepdims=True)).astype(np.float32)
    u_acc = syn.make_uniforms(syn.CONFIGS[0], 10, (T, B), instance=seed)
    u_fin = syn.make_uniforms(syn.CONFIGS[0], 11, B, instance=seed)
    return dict(draft=draft, sl_off=sl_off, sl_ids=ids, q=q, p=p, u_acc=u_acc, u_fin=u_fin)


def _run(N, c, noalloc):
    T, B = c["draft"].shape
    V = c["p"].shape[-1]
    dv = {k: to_dev(v) for k, v in c.items()}
    n_acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    out = torch.full((B, T + 1), -7, dtype=torch.int32, device="cuda")
    args = (dv["draft"], dv["sl_off"], dv["sl_ids"], dv["q"], dv["p"], dv["u_acc"], dv["u_fin"],
            n_acc, out)
    if noalloc:
        N.verify_reject_noalloc(*args)
    else:
        N.verify_reject(*args, N.workspace(N.verify_workspace_bytes(B, T, V)))
    torch.cuda.synchronize()
    return n_acc.cpu().numpy(), out.cpu().numpy()


def test_verify_noalloc_matches_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocabulary_draft_amd import native as N
    import oracle
    oracle.build(force=False)
    # first call: the Gemma-shaped batch (64 sequences, depth 5, V = 262144);
    # second call: a smaller, ragged case on the scratch the first one left
    for (V, T, B), seed in (((262144, 5, 64), 1), ((5000, 4, 3), 2)):
        print("noalloc verify case V=%d T=%d B=%d seed=%d" % (V, T, B, seed), flush=True)
        c = _case(V, T, B, seed)
        n_ref, out_ref = _run(N, c, noalloc=False)
        n_got, out_got = _run(N, c, noalloc=True)
        assert np.array_equal(n_got, n_ref)
        assert np.array_equal(out_got, out_ref)
        assert 0 < n_ref.max() and n_ref.min() < T
        if V == 5000:
            n_o, out_o, tie = oracle.verify_reject(**c)
            assert np.array_equal(n_got, n_o)
            assert np.array_equal(out_got[~tie], out_o[~tie])
