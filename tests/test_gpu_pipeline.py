"""End-to-end parity of one speculative draft step (the launch configuration
the benchmark times) against the oracle.

Each stage is compared on the GPU's own upstream outputs (router scores ->
selection -> shortlist -> logits -> tokens -> verification), so integer
stages must match bit for bit; the router and head within the logit bar.
On small workloads the oracle also runs the whole step from scratch: a
selection may differ only where two scores ranked around the budget cut are
closer than twice the observed router error (a tie zone), and everything
downstream of matching rows must agree.  Full-size workloads check the head
on sampled entries (the oracle cannot do 10^11 fp64 MACs in seconds).
"""
import numpy as np
import pytest
import torch
from tie_checks import check_sample_ties, check_verify_ties

import oracle
from oracle import pipeline as opipe
from dynamic_vocabulary_draft_amd import synthetic as syn
from dynamic_vocabulary_draft_amd.pipeline import DraftStep, StaticStep

pytestmark = pytest.mark.gpu


def small_configs():
    c1 = syn.CONFIGS[1]
    return {
        "tiny-fp32": syn.CONFIGS[0],
        "small-bf16-b3": syn.shrink(c1, V=20000, d=264, M=100, r=136, B=3, T=4,
                                    budget=syn.linear_budget(6000, 3000, 4)),
        "small-bf16-b1-d3840": syn.shrink(c1, V=9000, d=3840, M=64, r=64, B=1, T=3,
                                          budget=syn.linear_budget(2000, 1000, 3)),
        "small-tree": syn.shrink(syn.CONFIGS[3], V=12000, d=520, M=80, r=64, B=3,
                                 budget=(3000,), tree_nodes=5),
        # batched head on the matrix cores over the build's tile index: a
        # ragged last 32-token tile and a partial last build chunk
        "small-bf16-b12": syn.shrink(c1, V=9001, d=264, M=60, r=64, B=12, T=3,
                                     budget=syn.linear_budget(3000, 1500, 3)),
        # nine fp32 sequences: GEMV router with 8+ inputs, multi-row build,
        # GEMV head over many groups, two-pass sampler and verification
        "tiny-fp32-b9": syn.shrink(syn.CONFIGS[0], B=9),
    }


def _bar(got, ref, bf16):
    err = float(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)).max()) if np.size(got) else 0.0
    bar = 2e-2 if bf16 else 1e-5 * max(1.0, float(np.abs(ref).max()) if np.size(ref) else 1.0)
    assert err <= bar, "max |d| %g > %g" % (err, bar)
    return err


def _ulp(got, ref):
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    sp = np.spacing(np.maximum(np.abs(ref), np.float32(1e-38))).astype(np.float64)
    assert (np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= sp).all()


def check_stagewise(wl, r, head_samples=None, seed=0, tau=1.0):
    """Stage-by-stage parity on the GPU's own intermediate outputs."""
    cfg = wl.cfg
    bf16 = cfg.dtype == syn.DT_BF16
    B, T, M = cfg.B, cfg.T, cfg.M
    R = wl.router
    g = np.random.default_rng(seed)
    assert int(r["err_flag"][0]) == 0
    m = cfg.tree_nodes
    npos = 1 if cfg.is_tree else T
    for t in range(npos):
        rows = slice(t * B, (t + 1) * B)
        hin = wl.h[:, 0] if cfg.is_tree else wl.h[:, t]
        sc = oracle.router_score(np.ascontiguousarray(hin), R["W1"], R["b1"], R["W2"], R["b2"],
                                 cfg.act)
        _bar(r["scores"][t], sc, bf16)
        sel, n_sel, sl_len = oracle.select_clusters(r["scores"][t], wl.cluster_size,
                                                    cfg.budget_kind, wl.budget[t])
        assert np.array_equal(r["sel"][t], sel)
        assert np.array_equal(r["n_sel"][t], n_sel) and np.array_equal(r["sl_len"][t], sl_len)
        base = int(r["sl_off"][t * B])
        st, off, ids = oracle.build_shortlist(r["sel"][t], r["n_sel"][t], wl.cluster_of, base=base)
        assert st == 0
        assert np.array_equal(r["sl_off"][t * B:(t + 1) * B + 1], off)
        lo, hi = int(off[0]), int(off[-1])
        assert np.array_equal(r["sl_ids"][lo:hi], ids[lo:hi])
        assert np.array_equal(np.diff(off), sl_len.astype(np.int64))
        # head
        hh = np.ascontiguousarray(wl.h[:, 1:] if cfg.is_tree else wl.h[:, t + 1][:, None])
        loc_off = off - lo
        loc_ids = ids[lo:hi]
        if head_samples is None:
            ref = oracle.gathered_lm_head(wl.W, hh, loc_off, loc_ids)
            _bar(r["logits"][m * lo:m * hi], ref, bf16)
        else:
            for b in range(B):
                L = int(loc_off[b + 1] - loc_off[b])
                pick = np.sort(g.choice(L, min(L, head_samples), replace=False))
                sub_ids = loc_ids[loc_off[b]:loc_off[b + 1]][pick]
                ref = oracle.gathered_lm_head(wl.W, hh[b:b + 1], np.array([0, len(pick)], np.int64),
                                              sub_ids.astype(np.int32))
                gstart = m * (lo + int(loc_off[b]))
                got = np.stack([r["logits"][gstart + i * L + pick] for i in range(m)])
                _bar(got.reshape(-1), ref, bf16)
        # sampling on the GPU's logits
        u = wl.u_draft.reshape(-1) if cfg.is_tree else wl.u_draft[t]
        tok, q, tie = oracle.shortlist_sample(loc_off, loc_ids, r["logits"][m * lo:m * hi], u, m,
                                              tau)
        got_tok = r["token"].reshape(-1) if cfg.is_tree else r["token"][t]
        assert np.array_equal(got_tok[~tie], tok[~tie])
        check_sample_ties(got_tok, tok, tie, loc_off, loc_ids, q, m)
        _ulp(r["q"][m * lo:m * hi], q)
    if "p" in r:
        _ulp(r["p"], oracle.target_softmax(wl.target_logits))
        if cfg.is_tree:
            n_acc, out, path, tie = oracle.verify_tree(wl.parent, r["token"], r["sl_off"],
                                                       r["sl_ids"], r["q"], r["p"], wl.u_acc,
                                                       wl.u_fin)
            assert np.array_equal(r["n_acc"][~tie], n_acc[~tie])
            assert np.array_equal(r["path"][~tie], path[~tie])
            assert np.array_equal(r["out"][~tie], out[~tie])
            return
        n_acc, out, tie = oracle.verify_reject(r["token"], r["sl_off"], r["sl_ids"], r["q"], r["p"],
                                               wl.u_acc, wl.u_fin)
        assert np.array_equal(r["n_acc"], n_acc)
        assert np.array_equal(r["out"][~tie], out[~tie])
        check_verify_ties(r["out"], out, n_acc, tie, r["token"], r["sl_off"], r["sl_ids"], r["q"],
                          r["p"])


def check_from_scratch(wl, r, tau=1.0):
    """The oracle's own step vs the GPU's, outside tie zones."""
    cfg = wl.cfg
    ref = opipe.run_step(wl, temperature=tau)
    B = cfg.B
    npos = 1 if cfg.is_tree else cfg.T
    router_err = max(float(np.abs(r["scores"][t] - ref["scores"][t]).max()) for t in range(npos))
    ok_rows = np.ones((npos, B), bool)
    for t in range(npos):
        for b in range(B):
            k, kg = int(ref["n_sel"][t][b]), int(r["n_sel"][t][b])
            rs, gs = ref["sel"][t][b, :k], r["sel"][t][b, :kg]
            if kg == k and np.array_equal(gs, rs):
                continue
            # the first rank where the two selections differ: the clusters
            # there must be within the router's error of each other in the
            # oracle's scores (else the GPU ranked them wrongly)
            sc = np.asarray(ref["scores"][t][b], np.float64)
            n = min(k, kg)
            diff = np.flatnonzero(rs[:n] != gs[:n])
            # equal prefixes decide the next cluster alike: a count that
            # differs after them is no ranking tie
            assert diff.size, "selection counts differ after the same ranked prefix"
            i = int(diff[0])
            c_ref, c_gpu = int(rs[i]), int(gs[i])
            assert abs(sc[c_ref] - sc[c_gpu]) < 2 * router_err + 1e-30, \
                "selection differs at rank %d outside a tie zone" % i
            ok_rows[t, b] = False
    # the excuse is for rare near-ties, not a share of the rows
    assert (~ok_rows).sum() <= max(1, ok_rows.size // 8), "too many rows in tie zones"
    if cfg.is_tree:
        tok_ok = ~ref["tie"].reshape(B, -1) & ok_rows[0][:, None]
        assert np.array_equal(r["token"][tok_ok], ref["token"].reshape(B, -1)[tok_ok])
        if "n_acc" in ref:
            seq_ok = tok_ok.all(1) & ~ref["verify_tie"]
            for k in ("n_acc", "out", "path"):
                assert np.array_equal(r[k][seq_ok], ref[k][seq_ok]), k
        return
    good = ok_rows & ~ref["tie"]
    assert np.array_equal(r["token"][good], ref["token"][good])
    if "n_acc" in ref:
        seq_ok = good.all(0) & ~ref["verify_tie"]
        assert np.array_equal(r["n_acc"][seq_ok], ref["n_acc"][seq_ok])
        assert np.array_equal(r["out"][seq_ok], ref["out"][seq_ok])


@pytest.mark.parametrize("name", list(small_configs()))
def test_step_small(oracle_lib, name):
    cfg = small_configs()[name]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    step = DraftStep(wl)
    for rep in range(2):  # reuse of the buffers and workspaces
        step.sl_off.zero_()
        step.step()
        r = step.host()
        check_stagewise(wl, r)
        check_from_scratch(wl, r)


@pytest.mark.parametrize("tau", [0.0, 0.7])
@pytest.mark.parametrize("name", ["small-bf16-b1-d3840", "small-bf16-b12", "small-tree"])
def test_step_temperature(oracle_lib, name, tau):
    """The draft chain at another temperature and at 0 (the argmax, one-hot
    q), stage by stage and against the oracle's own step."""
    cfg = small_configs()[name]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    step = DraftStep(wl, temperature=float(np.float32(tau)))
    step.step()
    r = step.host()
    check_stagewise(wl, r, tau=float(np.float32(tau)))
    check_from_scratch(wl, r, tau=float(np.float32(tau)))


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_step_full_size(oracle_lib, index):
    """Full-size workloads in the benchmark's launch configuration; the head
    is checked on 256 sampled entries per shortlist."""
    wl = syn.make_workload(index)
    step = DraftStep(wl)
    step.step()
    r = step.host()
    check_stagewise(wl, r, head_samples=256 if index != 2 else 64, seed=index)


@pytest.mark.parametrize("name", ["tiny-fp32", "small-bf16-b3", "small-tree", "small-bf16-b12",
                                  "tiny-fp32-b9"])
def test_graph_replay_matches_eager(oracle_lib, name):
    """A captured step replayed three times, with eager work and
    synchronisation between replays, reproduces the eager step bit for bit."""
    cfg = small_configs()[name]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    step = DraftStep(wl)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.step(stream)
    eager = step.host()
    check_stagewise(wl, eager)
    graph = step.capture(stream)
    keys = [k for k in eager if k != "err_flag"]
    for rep in range(3):
        with torch.cuda.stream(stream):  # eager work between replays
            for t in (step.logits, step.q):
                t.fill_(float("nan"))
            step.sl_ids.fill_(-5)
            step.token.fill_(-9)
            step.sl_off[1:].fill_(-1)
            if step.target_logits is not None:
                step.out.fill_(-3)
                step.p.fill_(-1.0)
                if step.cfg.is_tree:
                    step.path.fill_(-4)
                    step.n_acc.fill_(-6)
        torch.cuda.synchronize()
        graph.launch(stream)
        got = step.host()
        for k in keys:
            assert np.array_equal(got[k], eager[k], equal_nan=True), (rep, k)
    graph.close()


@pytest.mark.parametrize("name", ["small-bf16-b3", "small-bf16-b1-d3840"])
@pytest.mark.parametrize("packed", [False, True])
def test_static_step(oracle_lib, name, packed):
    """The static baseline (one fixed frequency-ranked list at every
    position, gathered from W or from a packed slab) against the oracle's
    static step; replayed from a graph it reproduces the eager step."""
    cfg = small_configs()[name]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    ids = syn.static_shortlist(cfg, cfg.V // 3)
    step = StaticStep(wl, ids, packed=packed)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.step(stream)
    r = step.host()
    ref = opipe.run_static_step(wl, ids)
    bf16 = cfg.dtype == syn.DT_BF16
    _bar(r["logits"], ref["logits"], bf16)
    good = ~ref["tie"]
    assert np.array_equal(r["token"][good], ref["token"][good])
    # verification on the GPU's own drafts and q
    n_acc, out, vtie = oracle.verify_reject(r["token"], r["sl_off"], r["sl_ids"], r["q"], r["p"],
                                            wl.u_acc, wl.u_fin)
    assert np.array_equal(r["n_acc"], n_acc)
    assert np.array_equal(r["out"][~vtie], out[~vtie])
    graph = step.capture(stream)
    with torch.cuda.stream(stream):
        step.token.fill_(-9)
        step.logits.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.launch(stream)
    again = step.host()
    for k in ("token", "logits", "q", "n_acc", "out"):
        assert np.array_equal(again[k], r[k], equal_nan=True), k
    graph.close()
