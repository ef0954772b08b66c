"""GPU parity: every C-ABI call against the CPU oracle on identical inputs.

Bars (written in each test): cluster ids, counts, shortlist offsets and ids,
sampled and verified tokens bit-exact (tokens only outside the draws that the
oracle flags as lying within 1e-12 of a CDF boundary); logits within 2e-2
absolute for bf16 inputs and 1e-5 * max(1, max|ref|) for fp32; probabilities
within one fp32 ulp.  Sizes span several tiles and ragged tails (V not a
multiple of the 4096-token build chunk, d not a multiple of 512, M not a
power of two, empty and single-entry shortlists).
"""
import numpy as np
import pytest
import torch
from tie_checks import check_sample_ties, check_verify_ties

import oracle
from dynamic_vocabulary_draft_amd import synthetic as syn
from dynamic_vocabulary_draft_amd.pipeline import to_dev

pytestmark = pytest.mark.gpu

BF16_ATOL = 2e-2
F32_RTOL = 1e-5


@pytest.fixture(scope="module")
def N():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from dynamic_vocabulary_draft_amd import native
    return native


def _logit_bar(got, ref, bf16):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if bf16:
        err = np.abs(got - ref).max() if got.size else 0.0
        assert err <= BF16_ATOL, "max |d| = %g > %g" % (err, BF16_ATOL)
    else:
        bar = F32_RTOL * max(1.0, np.abs(ref).max() if ref.size else 1.0)
        err = np.abs(got - ref).max() if got.size else 0.0
        assert err <= bar, "max |d| = %g > %g" % (err, bar)


def _ulp_bar(got, ref):
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    spacing = np.spacing(np.maximum(np.abs(ref), np.float32(1e-38)))
    bad = np.abs(got.astype(np.float64) - ref.astype(np.float64)) > spacing.astype(np.float64)
    assert not bad.any(), "%d entries beyond one ulp" % bad.sum()


def _store(x, bf16):
    return syn.f32_to_bf16_bits(x) if bf16 else np.ascontiguousarray(x, np.float32)


def _cpu(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ----------------------------------------------------------------------------
# router_score
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bf16,act,n,d,r,M", [
    (False, syn.ACT_RELU, 4, 256, 256, 64),
    (True, syn.ACT_SILU, 7, 264, 136, 100),
    (True, syn.ACT_SILU, 1, 4096, 1024, 1024),
    (True, syn.ACT_SILU, 64, 3840, 1024, 2048),
    # batches of >= 8 bf16 inputs: first layer on the matrix cores, split over
    # 256-element windows of d (a partial last window, a ragged last row tile,
    # two column passes)
    (True, syn.ACT_SILU, 8, 264, 136, 100),
    (True, syn.ACT_SILU, 32, 4096, 1024, 1024),
    (True, syn.ACT_RELU, 70, 520, 200, 64),
    # second layer on the matrix cores: two-slice windows (M = 4096), and a
    # shape whose window partials do not fit (the vector path)
    (True, syn.ACT_SILU, 16, 512, 1024, 4096),
    (True, syn.ACT_RELU, 12, 256, 64, 4096),
])
def test_router_parity(N, oracle_lib, bf16, act, n, d, r, M):
    g = np.random.default_rng(100 + d)
    cfg = syn.shrink(syn.CONFIGS[4], dtype=syn.DT_BF16 if bf16 else syn.DT_F32, act=act, d=d, r=r,
                     M=M)
    R = syn.make_router(cfg)
    h = _store(g.standard_normal((n, 2, d)).astype(np.float32), bf16)  # rows at stride 2d
    ref = oracle_lib.router_score(np.ascontiguousarray(h[:, 0]), R["W1"], R["b1"], R["W2"], R["b2"],
                                  act)
    hd = to_dev(h)
    scores = torch.empty(n, M, dtype=torch.float32, device="cuda")
    ws = torch.zeros(N.router_workspace_bytes(n, r), dtype=torch.uint8, device="cuda")
    Rd = {k: to_dev(v) for k, v in R.items()}
    N.router_score(hd[:, 0], Rd["W1"], Rd["b1"], Rd["W2"], Rd["b2"], act, scores, ws, n=n, ldh=2 * d)
    _logit_bar(_cpu(scores), ref, bf16)


# ----------------------------------------------------------------------------
# select_clusters: bit-exact on identical scores
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 3, 64, 100, 200, 300, 1024, 2048, 4096])
@pytest.mark.parametrize("kind", [syn.BUDGET_CLUSTERS, syn.BUDGET_TOKENS])
def test_select_parity(N, oracle_lib, M, kind):
    g = np.random.default_rng(M * 7 + kind)
    n = 9
    s = g.standard_normal((n, M)).astype(np.float32)
    s[:3] = g.integers(-2, 3, size=(3, M)).astype(np.float32)  # heavy ties
    s[0][s[0] == 0] = -0.0
    size = (syn.zipf_cluster_sizes(max(M * 40, M), M, 1.1) if M > 1
            else np.array([7], np.int32))
    total = int(size.sum())
    if kind == syn.BUDGET_CLUSTERS:
        budget = np.array([0, 1, 2, M, M + 5, -3, max(1, M // 2), 3, 8], np.int32)
    else:
        budget = np.array([0, 1, total, total + 9, -4, total // 3, total // 5, 17, 5000],
                          np.int32)
    ref = oracle_lib.select_clusters(s, size, kind, budget)
    sel = torch.empty(n, M, dtype=torch.int32, device="cuda")
    n_sel = torch.empty(n, dtype=torch.int32, device="cuda")
    sl_len = torch.empty(n, dtype=torch.int32, device="cuda")
    N.select_clusters(to_dev(s), to_dev(size), kind, to_dev(budget), sel, n_sel, sl_len)
    assert np.array_equal(_cpu(n_sel), ref[1])
    assert np.array_equal(_cpu(sl_len), ref[2])
    assert np.array_equal(_cpu(sel), ref[0])


@pytest.mark.parametrize("M", [100, 1024, 3000])
def test_select_zero_sizes_and_ties(N, oracle_lib, M):
    """Token budgets over clusters of which a third are empty, with tied
    scores: the cut falls where the running size first reaches the budget,
    empty clusters ranked before it are taken and those after it are not."""
    g = np.random.default_rng(M + 11)
    n = 12
    s = g.integers(-3, 4, size=(n, M)).astype(np.float32)
    s[n // 2:] = g.standard_normal((n - n // 2, M)).astype(np.float32)
    size = g.integers(0, 60, size=M).astype(np.int32)
    size[g.random(M) < 0.33] = 0
    total = int(size.sum())
    budget = np.array([0, 1, 2, 59, 60, 61, total // 7, total // 2, total - 1, total, total + 1,
                       3], np.int32)
    for kind in (syn.BUDGET_TOKENS, syn.BUDGET_CLUSTERS):
        ref = oracle_lib.select_clusters(s, size, kind, budget)
        sel = torch.empty(n, M, dtype=torch.int32, device="cuda")
        n_sel = torch.empty(n, dtype=torch.int32, device="cuda")
        sl_len = torch.empty(n, dtype=torch.int32, device="cuda")
        N.select_clusters(to_dev(s), to_dev(size), kind, to_dev(budget), sel, n_sel, sl_len)
        assert np.array_equal(_cpu(n_sel), ref[1])
        assert np.array_equal(_cpu(sl_len), ref[2])
        assert np.array_equal(_cpu(sel), ref[0])


# ----------------------------------------------------------------------------
# build_shortlist: bit-exact
# ----------------------------------------------------------------------------
def _clusters(V, M, seed):
    g = np.random.default_rng(seed)
    size = syn.zipf_cluster_sizes(V, M, 1.1)
    cluster_of = np.empty(V, np.int32)
    cluster_of[g.permutation(V)] = np.repeat(np.arange(M, dtype=np.int32), size)
    return cluster_of, size


@pytest.mark.parametrize("V,M", [(13, 3), (4096, 64), (20000, 100), (262144, 2048)])
def test_cluster_index_is_chunk_prefix_counts(N, V, M):
    cluster_of, size = _clusters(V, M, V + 3)
    idx = N.cluster_index(to_dev(cluster_of), M)
    nch = (V + 4095) // 4096
    got = _cpu(idx).reshape(nch + 1, M)
    hist = np.stack([np.bincount(cluster_of[k * 4096:(k + 1) * 4096], minlength=M)
                     for k in range(nch)])
    ref = np.concatenate([np.zeros((1, M), np.int64), np.cumsum(hist, axis=0)])
    assert np.array_equal(got, ref)
    assert np.array_equal(got[-1], size)


@pytest.mark.parametrize("V,M,n", [(13, 3, 2), (4096, 64, 3), (20000, 100, 5), (20000, 100, 1),
                                   (128256, 1024, 4), (128256, 1024, 1), (262144, 2048, 2)])
def test_build_parity(N, oracle_lib, V, M, n):
    cluster_of, size = _clusters(V, M, V)
    g = np.random.default_rng(V + 1)
    s = g.standard_normal((n, M)).astype(np.float32)
    budget = g.integers(1, max(2, V // 3), size=n).astype(np.int32)
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, syn.BUDGET_TOKENS, budget)
    base = 17
    cap = base + int(sl_len.sum())
    st, off_ref, ids_ref = oracle_lib.build_shortlist(sel, n_sel, cluster_of, capacity=cap,
                                                      base=base)
    assert st == 0
    sl_off = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    sl_off[0] = base
    sl_ids = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(N.build_workspace_bytes(n, V), dtype=torch.uint8, device="cuda")
    cdev = to_dev(cluster_of)
    index = N.cluster_index(cdev, M, err_flag=flag)
    for _ in range(2):  # the workspace is reusable call after call
        N.build_shortlist(to_dev(sel), to_dev(n_sel), cdev, index, cap, sl_off, sl_ids, flag, ws)
        assert int(_cpu(flag)[0]) == 0
        assert np.array_equal(_cpu(sl_off), off_ref)
        assert np.array_equal(_cpu(sl_ids)[base:], ids_ref[base:])
        assert (_cpu(sl_ids)[:base] == -7).all()


@pytest.mark.parametrize("n", [1, 3])
def test_build_capacity_and_invalid_ids(N, oracle_lib, n):
    V, M = 9000, 40
    cluster_of, size = _clusters(V, M, 5)
    g = np.random.default_rng(6)
    sel, n_sel, sl_len = oracle_lib.select_clusters(g.standard_normal((n, M)).astype(np.float32),
                                                    size, syn.BUDGET_TOKENS,
                                                    np.full(n, 3000, np.int32))
    ws = torch.zeros(N.build_workspace_bytes(n, V), dtype=torch.uint8, device="cuda")
    cap = int(sl_len.sum()) - 100
    st, off_ref, ids_ref = oracle_lib.build_shortlist(sel, n_sel, cluster_of, capacity=cap)
    assert st == oracle.ECAPACITY
    sl_off = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    sl_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    cdev = to_dev(cluster_of)
    index = N.cluster_index(cdev, M, err_flag=flag)
    assert int(_cpu(flag)[0]) == 0
    N.build_shortlist(to_dev(sel), to_dev(n_sel), cdev, index, cap, sl_off, sl_ids, flag, ws)
    assert int(_cpu(flag)[0]) == oracle.ECAPACITY
    assert np.array_equal(_cpu(sl_off), off_ref)
    assert np.array_equal(_cpu(sl_ids), ids_ref)
    # out-of-range cluster ids: in the map (reported by the index) and in the
    # selection (reported by the build) are skipped like the oracle does
    bad_map = cluster_of.copy()
    bad_map[[5, 700, 8999]] = [-1, M, 10 ** 6]
    bad_sel = sel.copy()
    bad_sel[0, 0] = M + 3
    st, off_ref, ids_ref = oracle_lib.build_shortlist(bad_sel, n_sel, bad_map)
    assert st == oracle.EINVAL
    cap2 = n * V
    sl_ids2 = torch.empty(cap2, dtype=torch.int32, device="cuda")
    flag.zero_()
    bdev = to_dev(bad_map)
    index2 = N.cluster_index(bdev, M, err_flag=flag)
    assert int(_cpu(flag)[0]) == oracle.EINVAL
    flag.zero_()
    N.build_shortlist(to_dev(bad_sel), to_dev(n_sel), bdev, index2, cap2, sl_off, sl_ids2, flag,
                      ws)
    assert int(_cpu(flag)[0]) == oracle.EINVAL
    got_off = _cpu(sl_off)
    assert np.array_equal(got_off, off_ref)
    assert np.array_equal(_cpu(sl_ids2)[: got_off[-1]], ids_ref[: off_ref[-1]])


# ----------------------------------------------------------------------------
# gathered_lm_head
# ----------------------------------------------------------------------------
def _random_shortlists(g, V, lens, base=0):
    sl_off = np.concatenate([[base], base + np.cumsum(lens)]).astype(np.int64)
    ids = [np.sort(g.choice(V, L, replace=False)) for L in lens]
    sl_ids = np.full(base + sum(lens), -1, np.int32)
    if sum(lens):
        sl_ids[base:] = np.concatenate(ids)
    return sl_off, sl_ids


@pytest.mark.parametrize("bf16,d", [(False, 256), (True, 264), (True, 3840), (True, 4096),
                                    (False, 1032)])
@pytest.mark.parametrize("G,m", [(1, 1), (3, 1), (4, 3), (2, 64), (16, 1), (64, 1), (70, 1),
                                 (3, 8), (2, 100)])
def test_head_parity(N, oracle_lib, bf16, d, G, m):
    """GEMV path (fp32, or few single-row groups), union matrix-core path
    (bf16, >= 8 single-row groups; 70 groups take two column passes) and
    gathered matrix-core path (bf16, >= 8 head rows; 100 rows take two)."""
    V = 5000
    g = np.random.default_rng(d * 31 + G * 7 + m)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16 if bf16 else syn.DT_F32)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), bf16)
    lens = [int(x) for x in g.integers(0, 700, size=G)]
    lens[0] = max(lens[0], 1)
    if G > 2:
        lens[1] = 0  # an empty group
    base = 5
    sl_off, sl_ids = _random_shortlists(g, V, lens, base)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off - base, sl_ids[base:])
    Wd, hd = to_dev(W), to_dev(h)
    total = int(sl_off[-1] - base)
    for max_rows in (total, max(1, total // 5)):  # any bound gives the same result
        logits = torch.full((m * int(sl_off[-1]),), float("nan"), device="cuda")
        N.gathered_lm_head(Wd, hd, to_dev(sl_off), to_dev(sl_ids), max_rows, logits)
        got = _cpu(logits)[m * base:]
        assert not np.isnan(got).any()
        _logit_bar(got, ref, bf16)


@pytest.mark.parametrize("drop", [0, 37])
def test_head_union_dense_shortlists(N, oracle_lib, drop):
    """Batched path with shortlists covering (nearly) all of V: every 32-token
    tile is full or nearly so, and runs of one tile's entries cross the
    boundaries between the waves that index them."""
    V, d, G = 4999, 264, 9
    g = np.random.default_rng(4242 + drop)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, 1, d)).astype(np.float32), True)
    ids = []
    for k in range(G):
        keep = np.ones(V, bool)
        if drop:
            keep[g.choice(V, drop * (k + 1), replace=False)] = False
        ids.append(np.nonzero(keep)[0].astype(np.int32))
    sl_off = np.concatenate([[0], np.cumsum([len(x) for x in ids])]).astype(np.int64)
    sl_ids = np.concatenate(ids)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids), int(sl_off[-1]), logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("G", [9, 40])
def test_head_union_persistent_grid(N, oracle_lib, G):
    """Batched head over more tiles than resident workgroups: each workgroup
    of the persistent grid strides over about two tiles (128-row tiles for
    up to 32 groups, 256-row tiles above), with a ragged last tile; every
    logit is checked."""
    V, d = 70001, 264
    g = np.random.default_rng(7000 + G)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, 1, d)).astype(np.float32), True)
    lens = [int(x) for x in g.integers(V // 5, V // 2, size=G)]
    sl_off, sl_ids = _random_shortlists(g, V, lens)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids), int(sl_off[-1]),
                       logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("G", [4096, 4100])
def test_head_tree_many_groups(N, oracle_lib, G):
    """Tree head (8 head rows per group) with thousands of short shortlists,
    some empty: up to 4096 groups the workgroups share one list of every
    group's tiles (prefix built in LDS), above it each group keeps its own
    workgroups."""
    V, d, m = 5000, 264, 8
    g = np.random.default_rng(4000 + G)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), True)
    lens = [int(x) for x in g.integers(0, 5, size=G)]
    lens[-1] = 300  # one group spanning two 256-entry tiles
    sl_off, sl_ids = _random_shortlists(g, V, lens)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((m * int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids), int(sl_off[-1]),
                       logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("G,m,lo,hi", [(8, 64, 10000, 30000), (20, 8, 55000, 60000)])
def test_head_tree_tile_orders(N, oracle_lib, G, m, lo, hi):
    """Tree head over long ragged shortlists on the persistent tile list:
    eight groups of 40 to 120 tiles with 64 head rows each, and twenty
    groups of 8 head rows with over 4096 tiles in all (more tiles than
    workgroups many times over)."""
    V, d = 60000, 264
    g = np.random.default_rng(G * 1000 + m)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), True)
    lens = [int(x) for x in g.integers(lo, hi, size=G)]
    sl_off, sl_ids = _random_shortlists(g, V, lens)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((m * int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids), max(lens), logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("G,m,d", [(8, 64, 264), (8, 100, 264), (5, 8, 4096), (1, 64, 264),
                                   (8, 32, 520)])
def test_head_tree_shared_rows(N, oracle_lib, G, m, d):
    """Tree head over trees whose shortlists overlap heavily: a block of
    tokens on every tree, blocks shared by pairs of neighbouring trees, and
    scattered tokens of each tree alone; one pass of up to 64 head rows or
    two (100 rows), one or two 32-row column blocks, d of one and several
    phases.  Every logit is checked against the oracle."""
    V = 20000
    g = np.random.default_rng(G * 100 + m + d)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), True)
    perm = g.permutation(V)
    common = perm[:1500]
    pairs = [perm[1500 + 700 * k: 2200 + 700 * k] for k in range(G)]
    rest = perm[1500 + 700 * G:]
    ids = []
    for k in range(G):
        own = g.choice(rest, 900 + 137 * k, replace=False)
        sel = [common, pairs[k], pairs[(k + 1) % G], own]
        ids.append(np.unique(np.concatenate(sel)).astype(np.int32))
    sl_off = np.concatenate([[0], np.cumsum([len(x) for x in ids])]).astype(np.int64)
    sl_ids = np.concatenate(ids)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((m * int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids),
                       int(max(len(x) for x in ids)), logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("kind", ["identical", "unsorted", "descending", "one_long"])
def test_head_tree_merge_edges(N, oracle_lib, kind):
    """Edge cases of the tree head's tile list merged by token id: every
    group with the same shortlist (every tile's first id tied across the
    groups: ties go to the lower group), shortlists not in ascending order
    (the merge does not apply and the tile-index order runs instead), and
    one long group among short ones.  Every logit is checked."""
    V, d, G, m = 30000, 264, 8, 16
    g = np.random.default_rng({"identical": 1, "unsorted": 2, "descending": 3, "one_long": 4}[kind])
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), True)
    if kind == "identical":
        one = np.sort(g.choice(V, 3000, replace=False)).astype(np.int32)
        ids = [one] * G
    elif kind == "one_long":
        ids = [np.sort(g.choice(V, 300 if k else 20000, replace=False)).astype(np.int32)
               for k in range(G)]
    else:
        ids = [np.sort(g.choice(V, 2000 + 300 * k, replace=False)).astype(np.int32)
               for k in range(G)]
        ids = [x[g.permutation(len(x))] if kind == "unsorted" else x[::-1].copy() for x in ids]
    sl_off = np.concatenate([[0], np.cumsum([len(x) for x in ids])]).astype(np.int64)
    sl_ids = np.concatenate(ids)
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    logits = torch.full((m * int(sl_off[-1]),), float("nan"), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids),
                       int(max(len(x) for x in ids)), logits)
    got = _cpu(logits)
    assert not np.isnan(got).any()
    _logit_bar(got, ref, True)


@pytest.mark.parametrize("G,m", [(3, 1), (16, 1), (3, 8)])
def test_head_invalid_ids_are_nan(N, oracle_lib, G, m):
    """Ids outside [0, V) give NaN on every kernel path (GEMV, union, gathered);
    the valid entries of the same ascending shortlists are unaffected.  The
    ids >= V include ones inside the last 32-token tile."""
    V, d, bf16 = 5000, 264, True
    g = np.random.default_rng(900 + G * 10 + m)
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=50, dtype=syn.DT_BF16)
    cluster_of, _ = _clusters(V, 50, 3)
    W = syn.make_lm_head(cfg, cluster_of)
    h = _store(g.standard_normal((G, m, d)).astype(np.float32), bf16)
    lens = [int(x) for x in g.integers(50, 400, size=G)]
    sl_off, sl_ids = _random_shortlists(g, V, lens)
    bad = np.zeros(sl_ids.shape[0], bool)
    for k in range(G):
        a, b = int(sl_off[k]), int(sl_off[k + 1])
        if k % 2 == 0:
            sl_ids[a:a + 2] = [-7, -1]
            bad[a:a + 2] = True
        sl_ids[b - 3:b] = [V, V + 3, 2 ** 31 - 1]
        bad[b - 3:b] = True
        sl_ids[a:b] = np.sort(sl_ids[a:b])
    ref = oracle_lib.gathered_lm_head(W, h, sl_off, np.where(bad, 0, sl_ids).astype(np.int32))
    logits = torch.zeros(m * int(sl_off[-1]), device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h), to_dev(sl_off), to_dev(sl_ids), int(sl_off[-1]),
                       logits)
    got = _cpu(logits)
    bad_m = np.zeros(got.shape[0], bool)
    for k in range(G):
        a, b = int(sl_off[k]), int(sl_off[k + 1])
        for i in range(m):
            bad_m[m * a + i * (b - a): m * a + (i + 1) * (b - a)] = bad[a:b]
    assert np.isnan(got[bad_m]).all()
    assert not np.isnan(got[~bad_m]).any()
    _logit_bar(got[~bad_m], ref[~bad_m], bf16)


def test_head_full_vocabulary_is_dense(N, oracle_lib):
    """With the whole vocabulary as shortlist the head is the dense LM head."""
    cfg = syn.CONFIGS[0]
    cluster_of, _ = syn.make_clusters(cfg)
    W = syn.make_lm_head(cfg, cluster_of)
    h = syn.make_hidden(cfg)[0, :3]
    dense = oracle_lib.dense_lm_head(W, h)
    logits = torch.empty(3 * cfg.V, device="cuda")
    N.gathered_lm_head(to_dev(W), to_dev(h[None]), to_dev(np.array([0, cfg.V], np.int64)),
                       to_dev(np.arange(cfg.V, dtype=np.int32)), cfg.V, logits)
    _logit_bar(_cpu(logits).reshape(3, cfg.V), dense, False)


# ----------------------------------------------------------------------------
# static-shortlist slab
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bf16,d", [(True, 264), (False, 1032), (True, 4096)])
def test_pack_rows_bit_exact(N, oracle_lib, bf16, d):
    V, n = 3000, 2500
    g = np.random.default_rng(d)
    W = g.standard_normal((V, d)).astype(np.float32)
    W = syn.f32_to_bf16_bits(W) if bf16 else W
    ids = g.integers(0, V, size=n).astype(np.int32)
    ids[[0, 7, n - 1]] = [-1, V, 2 ** 31 - 1]
    ref = oracle_lib.pack_rows(W, ids)
    Wd = to_dev(W)
    out = torch.empty((n, d), dtype=Wd.dtype, device="cuda")
    N.pack_rows(Wd, to_dev(ids), out)
    got = _cpu(out.view(torch.int16) if bf16 else out.view(torch.int32))
    want = ref.view(np.int16) if bf16 else ref.view(np.int32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("G", [1, 16])
def test_packed_head_equals_gathered_head_gpu(N, oracle_lib, G):
    """Head over a packed slab (ids 0..L-1) == gathered head over the list,
    bit for bit, on the GEMV (1 group) and union (16 groups) paths."""
    cfg = syn.shrink(syn.CONFIGS[1], V=6000, d=264, M=40)
    cluster_of, _ = _clusters(6000, 40, 5)
    W = syn.make_lm_head(cfg, cluster_of)
    ids = syn.static_shortlist(cfg, 1500)
    L = ids.shape[0]
    h = _store(np.random.default_rng(G).standard_normal((G, 1, 264)).astype(np.float32), True)
    off = (np.arange(G + 1) * L).astype(np.int64)
    Wd = to_dev(W)
    slab = torch.empty((L, 264), dtype=Wd.dtype, device="cuda")
    N.pack_rows(Wd, to_dev(ids), slab)
    a = torch.empty(G * L, device="cuda")
    b = torch.empty(G * L, device="cuda")
    N.gathered_lm_head(Wd, to_dev(h), to_dev(off), to_dev(np.tile(ids, G)), G * L, a)
    N.gathered_lm_head(slab, to_dev(h), to_dev(off), to_dev(np.tile(np.arange(L, dtype=np.int32), G)),
                       G * L, b)
    assert torch.equal(a, b)
    _logit_bar(_cpu(a), oracle_lib.gathered_lm_head(W, h, off, np.tile(ids, G)), True)


# ----------------------------------------------------------------------------
# shortlist_sample
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("lens,m", [([1, 5, 255, 256, 257, 1000], 1), ([27000, 3], 1),
                                    ([600000], 1), ([300, 1, 40], 4)])
@pytest.mark.parametrize("tau", [1.0, float(np.float32(0.7)), 0.0])
def test_sample_parity(N, oracle_lib, lens, m, tau):
    g = np.random.default_rng(sum(lens) + m)
    G = len(lens)
    sl_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sl_ids = np.concatenate([np.sort(g.choice(10 ** 6, L, replace=False)) for L in lens]).astype(np.int32)
    logits = (g.standard_normal(m * int(sl_off[-1])) * 3).astype(np.float32)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, G * m, instance=G)
    u[0] = 0.0
    tok_ref, q_ref, tie = oracle_lib.shortlist_sample(sl_off, sl_ids, logits, u, m, tau)
    token = torch.empty(G * m, dtype=torch.int32, device="cuda")
    q = torch.empty(logits.shape[0], dtype=torch.float32, device="cuda")
    ws = N.workspace(N.sample_workspace_bytes(G, m, max(lens)))
    N.shortlist_sample(to_dev(sl_off), to_dev(sl_ids), to_dev(logits), tau, to_dev(u), token, q, ws,
                       max_len=max(lens), m=m)
    got = _cpu(token)
    assert np.array_equal(got[~tie], tok_ref[~tie])
    check_sample_ties(got, tok_ref, tie, sl_off, sl_ids, q_ref, m)
    _ulp_bar(_cpu(q), q_ref)


def test_sample_many_rows_bit_exact(N, oracle_lib):
    """20k draws over one 5000-entry shortlist: the tokens match the oracle."""
    L, R = 5000, 20000
    g = np.random.default_rng(77)
    lg = (g.standard_normal(L) * 2).astype(np.float32)
    sl_off = (np.arange(R + 1) * L).astype(np.int64)
    ids = np.tile(np.arange(L, dtype=np.int32), R)
    logits = np.tile(lg, R)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, R, instance=5)
    tok_ref, q_ref, tie = oracle_lib.shortlist_sample(sl_off, ids, logits, u)
    token = torch.empty(R, dtype=torch.int32, device="cuda")
    q = torch.empty(L * R, dtype=torch.float32, device="cuda")
    ws = N.workspace(N.sample_workspace_bytes(R, 1, L))
    N.shortlist_sample(to_dev(sl_off), to_dev(ids), to_dev(logits), 1.0, to_dev(u), token, q, ws,
                       max_len=L)
    got = _cpu(token)
    assert np.array_equal(got[~tie], tok_ref[~tie])
    check_sample_ties(got, tok_ref, tie, sl_off, ids, q_ref)
    assert tie.sum() <= 2


@pytest.mark.parametrize("rows,maxlen", [(800, 12000), (150, 70000)])
@pytest.mark.parametrize("tau", [1.0, float(np.float32(0.7)), 0.0])
def test_sample_multi_chunk_workgroups(N, oracle_lib, rows, maxlen, tau):
    """Ragged rows in large launches: 800 short rows (one chunk per
    workgroup), 150 rows up to 70000 entries (four chunks per workgroup),
    shorter rows ending inside a workgroup."""
    g = np.random.default_rng(rows + int(tau * 10))
    lens = g.integers(1, maxlen, size=rows)
    lens[:3] = [1, 1024, maxlen]
    sl_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sl_ids = np.concatenate([np.sort(g.choice(10 ** 6, L, replace=False)) for L in lens])
    sl_ids = sl_ids.astype(np.int32)
    logits = (g.standard_normal(int(sl_off[-1])) * 3).astype(np.float32)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, rows, instance=rows)
    tok_ref, q_ref, tie = oracle_lib.shortlist_sample(sl_off, sl_ids, logits, u, 1, tau)
    token = torch.empty(rows, dtype=torch.int32, device="cuda")
    q = torch.empty(logits.shape[0], dtype=torch.float32, device="cuda")
    ws = N.workspace(N.sample_workspace_bytes(rows, 1, int(lens.max())))
    N.shortlist_sample(to_dev(sl_off), to_dev(sl_ids), to_dev(logits), tau, to_dev(u), token, q,
                       ws, max_len=int(lens.max()))
    got = _cpu(token)
    assert np.array_equal(got[~tie], tok_ref[~tie])
    check_sample_ties(got, tok_ref, tie, sl_off, sl_ids, q_ref)
    _ulp_bar(_cpu(q), q_ref)


# ----------------------------------------------------------------------------
# target_softmax and verify_reject
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("rows,V", [(3, 1000), (5, 128256), (2, 262144), (40, 128256),
                                    (70, 128256), (9, 151936)])
def test_target_softmax_parity(N, oracle_lib, rows, V):
    """One segment (V = 1000) and many, the last one partial."""
    g = np.random.default_rng(V)
    lg = (g.standard_normal((rows, V)) * 3).astype(np.float32)
    p = torch.empty(rows, V, device="cuda")
    N.target_softmax(to_dev(lg), p, N.workspace(N.softmax_workspace_bytes(rows, V)))
    _ulp_bar(_cpu(p), oracle_lib.target_softmax(lg))


def test_target_softmax_extreme_logits(N, oracle_lib):
    """-inf logits (two whole 4096-element segments, every third entry), a
    spread that takes exp through its whole range to underflow and to
    subnormal p, a single huge logit, a constant row, a large negative
    offset; V = 10001 leaves rows unaligned for 16-byte accesses."""
    rows, V = 7, 10001
    g = np.random.default_rng(11)
    lg = (g.standard_normal((rows, V)) * 40).astype(np.float32)
    lg[0, :8192] = -np.inf
    lg[1, ::3] = -np.inf
    lg[2] = g.permutation(np.linspace(0.0, -1100.0, V)).astype(np.float32)  # every exponent
    lg[3, 5000] = 3.0e38
    lg[4] = 7.0
    lg[5] = (g.standard_normal(V) * 3 - 1.0e4).astype(np.float32)
    ref = oracle_lib.target_softmax(lg)
    assert (ref[2] == 0).sum() > V // 2 and ((ref[2] > 0) & (ref[2] < 1.2e-38)).sum() > 50
    p = torch.full((rows, V), float("nan"), device="cuda")
    N.target_softmax(to_dev(lg), p, N.workspace(N.softmax_workspace_bytes(rows, V)))
    got = _cpu(p)
    _ulp_bar(got, ref)
    assert (got[0, :8192] == 0).all() and (got[1, ::3] == 0).all() and got[3, 5000] == 1.0


def _verify_case(oracle_lib, V, T, B, mode, seed):
    """Shortlists from random cluster selections, drafts sampled from q,
    target probabilities per mode; everything computed on the host."""
    g = np.random.default_rng(seed)
    M = max(2, V // 64)
    cluster_of, size = _clusters(V, M, seed)
    s = g.standard_normal((T * B, M)).astype(np.float32)
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, syn.BUDGET_TOKENS,
                                                    np.full(T * B, max(1, V // 4), np.int32))
    st, sl_off, sl_ids = oracle_lib.build_shortlist(sel, n_sel, cluster_of)
    n = int(sl_off[-1])
    sl_ids = sl_ids[:n]
    lg = (g.standard_normal(n) * 2).astype(np.float32)
    u_d = syn.make_uniforms(syn.CONFIGS[0], 9, T * B, instance=seed)
    draft, q, _ = oracle_lib.shortlist_sample(sl_off, sl_ids, lg, u_d)
    if mode == "correlated":  # target logits = draft logits on the shortlist + N(0, 0.5)
        tl = np.full((B, T + 1, V), -4.0, np.float32)
        for t in range(T):
            for b in range(B):
                r = t * B + b
                tl[b, t, sl_ids[sl_off[r]:sl_off[r + 1]]] = lg[sl_off[r]:sl_off[r + 1]]
        tl += (g.standard_normal(tl.shape) * 0.5).astype(np.float32)
    else:
        tl = (g.standard_normal((B, T + 1, V)) * 3).astype(np.float32)
    p = oracle_lib.target_softmax(tl)
    u_acc = syn.make_uniforms(syn.CONFIGS[0], 10, (T, B), instance=seed)
    if mode == "accept_all":
        u_acc[:] = 0.0
    elif mode == "reject_all":
        u_acc[:] = np.float32(1 - 2 ** -24)
    u_fin = syn.make_uniforms(syn.CONFIGS[0], 11, B, instance=seed)
    return dict(draft=draft.reshape(T, B), sl_off=sl_off, sl_ids=sl_ids, q=q, p=p, u_acc=u_acc,
                u_fin=u_fin), tl


@pytest.mark.parametrize("V,T,B", [(8, 3, 64), (5000, 4, 16), (128256, 6, 4), (262144, 5, 3)])
@pytest.mark.parametrize("mode", ["random", "accept_all", "reject_all", "correlated"])
def test_verify_parity(N, oracle_lib, V, T, B, mode):
    c, _ = _verify_case(oracle_lib, V, T, B, mode, seed=V + T + B)
    n_ref, out_ref, tie = oracle_lib.verify_reject(**c)
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, T + 1, dtype=torch.int32, device="cuda")
    dv = {k: to_dev(v) for k, v in c.items()}
    N.verify_reject(dv["draft"], dv["sl_off"], dv["sl_ids"], dv["q"], dv["p"], dv["u_acc"],
                    dv["u_fin"], n_acc, out, N.workspace(N.verify_workspace_bytes(B, T, V)))
    assert np.array_equal(_cpu(n_acc), n_ref)  # accept decisions are exact
    got = _cpu(out)
    assert np.array_equal(got[~tie], out_ref[~tie])
    check_verify_ties(got, out_ref, n_ref, tie, c["draft"], c["sl_off"], c["sl_ids"], c["q"],
                      c["p"])
    if mode == "accept_all":
        assert (n_ref == T).all()
    if mode == "correlated":
        assert n_ref.mean() > 0.5


def test_verify_residual_without_mass(N, oracle_lib):
    """Rejections whose residual max(0, p - q) has no mass draw from p_t
    itself: p_0 = q_0 / 2 on the shortlist (sequences 0-2) rejects for
    u = 0.9 and leaves no residual; an all-zero p_0 (sequence 3) has nothing
    to draw (-1)."""
    V, T, B = 5000, 3, 4
    c, _ = _verify_case(oracle_lib, V, T, B, "random", seed=77)
    p = c["p"].copy()
    for b in range(B):
        p[b, 0] = 0.0
        if b < 3:
            lo, hi = c["sl_off"][b], c["sl_off"][b + 1]
            p[b, 0, c["sl_ids"][lo:hi]] = 0.5 * c["q"][lo:hi]
    c["p"] = p
    c["u_acc"] = c["u_acc"].copy()
    c["u_acc"][0] = 0.9
    n_ref, out_ref, tie = oracle_lib.verify_reject(**c)
    assert (n_ref == 0).all() and out_ref[3, 0] == -1 and (out_ref[:3, 0] >= 0).all()
    n_acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, T + 1, dtype=torch.int32, device="cuda")
    dv = {k: to_dev(v) for k, v in c.items()}
    N.verify_reject(dv["draft"], dv["sl_off"], dv["sl_ids"], dv["q"], dv["p"], dv["u_acc"],
                    dv["u_fin"], n_acc, out, N.workspace(N.verify_workspace_bytes(B, T, V)))
    assert np.array_equal(_cpu(n_acc), n_ref)
    got = _cpu(out)
    assert np.array_equal(got[~tie], out_ref[~tie])
    check_verify_ties(got, out_ref, n_ref, tie, c["draft"], c["sl_off"], c["sl_ids"], c["q"],
                      c["p"])


@pytest.mark.parametrize("V,T,B", [(8, 3, 64), (5000, 4, 16), (128256, 6, 4), (262144, 5, 3),
                                   (10001, 64, 3), (32000, 3, 200)])
@pytest.mark.parametrize("mode", ["random", "reject_all", "correlated"])
def test_verify_logits_parity(N, oracle_lib, V, T, B, mode):
    """Verification from target logits: the same outputs as the target
    softmax followed by verification over its probabilities (bit for bit,
    every entry: the same p values are computed), and the oracle's
    verification over those probabilities (exact outside the tie zone)."""
    c, tl = _verify_case(oracle_lib, V, T, B, mode, seed=V + 7 * T + B)
    dv = {k: to_dev(v) for k, v in c.items()}
    lg = to_dev(tl)
    p = torch.empty(B, T + 1, V, device="cuda")
    N.target_softmax(lg, p, N.workspace(N.softmax_workspace_bytes(B * (T + 1), V)))
    outs = []
    for fused in (False, True):
        n_acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, T + 1), -7, dtype=torch.int32, device="cuda")
        if fused:
            N.verify_reject_logits(dv["draft"], dv["sl_off"], dv["sl_ids"], dv["q"], lg,
                                   dv["u_acc"], dv["u_fin"], n_acc, out,
                                   N.workspace(N.verify_logits_workspace_bytes(B, T, V)))
        else:
            N.verify_reject(dv["draft"], dv["sl_off"], dv["sl_ids"], dv["q"], p, dv["u_acc"],
                            dv["u_fin"], n_acc, out,
                            N.workspace(N.verify_workspace_bytes(B, T, V)))
        outs.append((_cpu(n_acc), _cpu(out)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    c["p"] = _cpu(p)
    n_ref, out_ref, tie = oracle_lib.verify_reject(**c)
    assert np.array_equal(outs[1][0], n_ref)
    assert np.array_equal(outs[1][1][~tie], out_ref[~tie])
    check_verify_ties(outs[1][1], out_ref, n_ref, tie, c["draft"], c["sl_off"], c["sl_ids"],
                      c["q"], c["p"])


# ----------------------------------------------------------------------------
# spherical k-means over the LM-head rows
# ----------------------------------------------------------------------------
def _km_head(V, d, M, seed):
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=M)
    cluster_of, _ = syn.make_clusters(cfg)
    return cfg, cluster_of, syn.make_lm_head(cfg, cluster_of)


def _bf16_rne(x32):
    return syn.f32_to_bf16_bits(np.asarray(x32, np.float32))


@pytest.mark.parametrize("V,d", [(3001, 64), (5000, 3840)])
def test_kmeans_inv_norms(N, oracle_lib, V, d):
    cfg, _, W = _km_head(V, d, 16, 0)
    W[3] = 0
    out = torch.empty(V, device="cuda")
    N.kmeans_inv_norms(to_dev(W), out)
    _ulp_bar(_cpu(out), oracle_lib.kmeans_inv_norms(W))


@pytest.mark.parametrize("V,d,M", [(3001, 64, 200), (4000, 256, 128), (2500, 3840, 37),
                                   (1000, 128, 1), (6000, 512, 700), (2000, 192, 300)])
def test_kmeans_assign(N, oracle_lib, V, d, M):
    """Ragged row and centroid tiles (several centroid tiles too), one and
    many 64-wide slices; rows are compared outside the band where fp32
    accumulation order may decide."""
    cfg, _, W = _km_head(V, d, max(M, 2), 1)
    g = np.random.default_rng(V + M)
    Cf = g.standard_normal((M, d)).astype(np.float32)
    Cf /= np.linalg.norm(Cf, axis=1, keepdims=True)
    Cb = _bf16_rne(Cf)
    if M > 4:
        Cb[M - 1] = Cb[2]  # an exact duplicate: the lower id must win
    ref, sref, tie = oracle_lib.kmeans_assign(W, Cb)
    a = torch.empty(V, dtype=torch.int32, device="cuda")
    sc = torch.empty(V, device="cuda")
    N.kmeans_assign(to_dev(W), to_dev(Cb), a, sc)
    got = _cpu(a)
    assert np.array_equal(got[~tie], ref[~tie])
    assert ((got >= 0) & (got < M)).all()
    if M > 4:
        assert not (got == M - 1).any()
    bound = d * 2.0 ** -22 * np.abs(sref).max() + 1e-6
    assert np.abs(_cpu(sc)[~tie] - sref[~tie]).max() <= bound * 50


def _km_update_gpu(N, W, inv, lab, Cp, M, err=None):
    V, d = W.shape
    out = torch.empty(M, d, device="cuda")
    outb = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
    size = torch.empty(M, dtype=torch.int32, device="cuda")
    norm = torch.empty(M, dtype=torch.float64, device="cuda")
    N.kmeans_update(to_dev(W), inv, to_dev(lab), to_dev(Cp), out, outb, size, norm, err_flag=err)
    return _cpu(out), _cpu(outb.view(torch.int16)).view(np.uint16), _cpu(size), _cpu(norm)


@pytest.mark.parametrize("V,d,M", [(3001, 64, 20), (9000, 264, 300), (20000, 2056, 64)])
def test_kmeans_update(N, oracle_lib, V, d, M):
    """Clusters from empty to many member ranges (128 rows each),
    several scatter chunks, d with a partial 2048-element group."""
    cfg, cluster_of, W = _km_head(V, d, M, 2)
    inv_h = oracle_lib.kmeans_inv_norms(W)
    lab = syn.kmeans_init_assign(cfg, cluster_of, 0.3)
    lab[lab == 5] = 6  # cluster 5 empty
    if V > 10000:
        lab[: V // 2] = 1  # one cluster of 10000 rows: ten member ranges
    Cp = np.random.default_rng(7).standard_normal((M, d)).astype(np.float32)
    inv = to_dev(inv_h)
    out, outb, size, norm = _km_update_gpu(N, W, inv, lab, Cp, M)
    ref, rsize, rnorm = oracle_lib.kmeans_update(W, inv_h, lab, Cp)
    assert np.array_equal(size, rsize)
    _ulp_bar(out, ref)
    assert np.array_equal(out[5], Cp[5])
    assert np.array_equal(outb, _bf16_rne(out))
    assert np.allclose(norm, rnorm, rtol=1e-12, atol=0)


def test_kmeans_update_invalid_labels(N, oracle_lib):
    cfg, cluster_of, W = _km_head(3000, 64, 20, 3)
    inv_h = oracle_lib.kmeans_inv_norms(W)
    lab = cluster_of.astype(np.int32).copy()
    lab[[4, 99]] = [-1, 20]
    Cp = np.zeros((20, 64), np.float32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, _, size, _ = _km_update_gpu(N, W, to_dev(inv_h), lab, Cp, 20, err=flag)
    assert int(_cpu(flag)[0]) == oracle.EINVAL
    ref, rsize, _ = oracle_lib.kmeans_update(W, inv_h, lab, Cp)
    assert np.array_equal(size, rsize)
    _ulp_bar(out, ref)


def test_kmeans_iterations_recover_planted(N, oracle_lib):
    """Several GPU iterations checked stage by stage against the oracle on the
    GPU's own inputs; from a 30%-noisy start they recover the planted
    partition and the objective does not decrease."""
    V, d, M = 6000, 256, 40
    cfg, cluster_of, W = _km_head(V, d, M, 4)
    Wd = to_dev(W)
    inv = torch.empty(V, device="cuda")
    N.kmeans_inv_norms(Wd, inv)
    inv_h = _cpu(inv)
    lab = syn.kmeans_init_assign(cfg, cluster_of, 0.3)
    Cp = np.zeros((M, d), np.float32)
    objs = []
    a = torch.empty(V, dtype=torch.int32, device="cuda")
    sc = torch.empty(V, device="cuda")
    for it in range(3):
        out, outb, size, norm = _km_update_gpu(N, W, inv, lab, Cp, M)
        ref, _, _ = oracle_lib.kmeans_update(W, inv_h, lab, Cp)
        _ulp_bar(out, ref)
        objs.append(float(norm.sum()))
        N.kmeans_assign(Wd, to_dev(outb), a, sc)
        lab = _cpu(a)
        rl, _, tie = oracle_lib.kmeans_assign(W, outb)
        assert np.array_equal(lab[~tie], rl[~tie])
        Cp = out
    assert np.array_equal(lab, cluster_of)
    assert all(b >= a_ * (1 - 1e-6) for a_, b in zip(objs, objs[1:]))
