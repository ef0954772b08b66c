"""Draft sampling that writes each row's statistics instead of q, and the
verifiers that recompute q from the draft logits with them: the tokens and
the verification outputs must equal those of the q path bit for bit (both
sides evaluate the same expression), and q rebuilt on the host from the
statistics must match the q the sampler writes to fp32 rounding.

The q path itself is checked against the oracle in test_gpu_pipeline.py and
test_gpu_tree.py; here the reference is the library's own q path on the
same inputs."""
import numpy as np
import pytest
import torch

from dynamic_vocabulary_draft_amd import native as N
from dynamic_vocabulary_draft_amd import synthetic as syn
from dynamic_vocabulary_draft_amd.pipeline import DraftStep

pytestmark = pytest.mark.gpu


def _configs():
    c1 = syn.CONFIGS[1]
    return {
        "tiny-fp32": syn.CONFIGS[0],
        "tiny-fp32-b9": syn.shrink(syn.CONFIGS[0], B=9),
        "small-bf16-b3": syn.shrink(c1, V=20000, d=264, M=100, r=136, B=3, T=4,
                                    budget=syn.linear_budget(6000, 3000, 4)),
        "small-bf16-b12": syn.shrink(c1, V=9001, d=264, M=60, r=64, B=12, T=3,
                                     budget=syn.linear_budget(3000, 1500, 3)),
        "small-tree": syn.shrink(syn.CONFIGS[3], V=12000, d=520, M=80, r=64, B=3,
                                 budget=(3000,), tree_nodes=5),
    }


def _run(wl, mode, tau, stream=None):
    step = DraftStep(wl, temperature=tau, q_mode=mode)
    step.step(stream)
    r = step.host()
    step.close()
    return r


def _same(a, b, keys):
    for k in keys:
        if k in a or k in b:
            assert np.array_equal(a[k], b[k], equal_nan=True), k


def _q_from_stats(r, cfg, tau):
    """q of every draft row rebuilt in fp64 from the logits and the row's
    statistics (the sampler's layout: row g*m + i holds len_g entries)."""
    m = cfg.tree_nodes
    off = r["sl_off"].astype(np.int64)
    base = off[0]
    q = np.empty_like(r["logits"])
    for g in range(off.shape[0] - 1):
        lo, n = off[g] - base, off[g + 1] - off[g]
        for i in range(m):
            row = g * m + i
            seg = slice(m * lo + i * n, m * lo + (i + 1) * n)
            x = (r["logits"][seg].astype(np.float64) - np.float64(r["qstats_M"][row])) / tau
            q[seg] = (np.exp(x) * r["qstats_rZ"][row]).astype(np.float32)
    return q


KEYS = ("token", "sl_off", "sl_ids", "logits", "n_acc", "out", "path")


@pytest.mark.parametrize("tau", [1.0, 0.7, 0.1, 2.5])
@pytest.mark.parametrize("name", list(_configs()))
def test_stats_step_matches_q_step(name, tau):
    cfg = _configs()[name]
    tau = float(np.float32(tau))
    wl = syn.make_workload(cfg.index, cfg=cfg)
    dense = _run(wl, "dense", tau)
    stats = _run(wl, "stats", tau)
    _same(dense, stats, KEYS)
    q = _q_from_stats(stats, cfg, tau)
    ref = dense["q"].astype(np.float64)
    sp = np.spacing(np.maximum(np.abs(dense["q"]), np.float32(1e-38))).astype(np.float64)
    assert (np.abs(q.astype(np.float64) - ref) <= sp).all()


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_stats_step_full_size(index):
    """Full-size workloads in the benchmark's launch configuration."""
    wl = syn.make_workload(index)
    dense = _run(wl, "dense", 1.0)
    stats = _run(wl, "stats", 1.0)
    _same(dense, stats, ("token", "sl_off", "n_acc", "out", "path"))


@pytest.mark.parametrize("name", ["tiny-fp32", "small-bf16-b12", "small-tree"])
def test_stats_graph_replay_matches_eager(name):
    """A captured stats-mode step replayed three times, with eager work and
    synchronisation between the replays, reproduces the eager step."""
    cfg = _configs()[name]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    step = DraftStep(wl, q_mode="stats")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step.step(stream)
    eager = step.host()
    graph = step.capture(stream)
    for rep in range(3):
        with torch.cuda.stream(stream):
            step.logits.fill_(float("nan"))
            step.qstats.fill_(0xAB)
            step.token.fill_(-9)
            step.n_acc.fill_(-3)
            step.out.fill_(-3)
            if step.cfg.is_tree:
                step.path.fill_(-4)
        torch.cuda.synchronize()
        graph.launch(stream)
        torch.cuda.synchronize()
        got = step.host()
        _same(eager, got, KEYS + ("qstats_M", "qstats_rZ"))
    graph.close()
    step.close()


def test_sample_stats_empty_and_ragged_rows():
    """Groups of unequal length, one empty, two head rows each: the tokens
    equal the q path's, an empty group's rows get token -1 and rZ = 0."""
    g = np.random.default_rng(5)
    lens = [5000, 0, 1300, 2049]
    m = 2
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ids = np.concatenate([np.sort(g.choice(30000, n, replace=False)) for n in lens]).astype(np.int32)
    logits = (3.0 * g.standard_normal(m * off[-1])).astype(np.float32)
    u = g.random(len(lens) * m).astype(np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    d_off, d_ids, d_lg, d_u = dev(off), dev(ids), dev(logits), dev(u)
    G = len(lens)
    ws = N.workspace(N.sample_workspace_bytes(G, m, max(lens)))
    tok_q = torch.empty(G * m, dtype=torch.int32, device="cuda")
    tok_s = torch.empty(G * m, dtype=torch.int32, device="cuda")
    q = torch.empty(m * off[-1], dtype=torch.float32, device="cuda")
    qs = N.qstats_buffer(G * m)
    for tau in (1.0, 0.7):
        N.shortlist_sample(d_off, d_ids, d_lg, tau, d_u, tok_q, q, ws, max_len=max(lens), m=m)
        N.shortlist_sample_stats(d_off, d_ids, d_lg, tau, d_u, tok_s, qs, ws, max_len=max(lens),
                                 m=m)
        torch.cuda.synchronize()
        assert np.array_equal(tok_q.cpu().numpy(), tok_s.cpu().numpy())
        raw = qs.cpu().numpy()
        rZ = raw.view(np.float64)[1::2]
        assert (tok_s.cpu().numpy()[2:4] == -1).all() and (rZ[2:4] == 0.0).all()
        assert (rZ[[0, 1, 4, 5, 6, 7]] > 0.0).all()


@pytest.mark.parametrize("packed", [False, True])
def test_static_stats_step_matches_q_step(packed):
    """The static baseline with the row-statistics sampler: the same tokens
    and verification outputs as with q."""
    from dynamic_vocabulary_draft_amd.pipeline import StaticStep
    cfg = _configs()["small-bf16-b3"]
    wl = syn.make_workload(cfg.index, cfg=cfg)
    ids = syn.static_shortlist(cfg, cfg.V // 3)
    res = {}
    for mode in ("dense", "stats"):
        step = StaticStep(wl, ids, packed=packed, q_mode=mode)
        step.step()
        res[mode] = step.host()
    _same(res["dense"], res["stats"], ("token", "logits", "n_acc", "out"))
