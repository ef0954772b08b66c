"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests retypes the oracle's formula: each compares it with a
library routine in float64 (numpy/BLAS matmul, scipy softmax, numpy
cumsum/searchsorted), a brute-force Python enumeration, a closed form, a
stratified quadrature, or the exact distribution that speculative sampling
must reproduce (the target's), chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from dynamic_vocabulary_draft_amd import synthetic as syn

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return syn.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _small_cfg(dtype=syn.DT_F32, act=syn.ACT_RELU):
    return syn.shrink(syn.CONFIGS[0], dtype=dtype, act=act)


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [syn.DT_F32, syn.DT_BF16])
@pytest.mark.parametrize("act", [syn.ACT_RELU, syn.ACT_SILU])
def test_router_matches_float64_blas(oracle_lib, dtype, act):
    cfg = _small_cfg(dtype, act)
    R = syn.make_router(cfg)
    h = syn.make_hidden(cfg)[0]  # [T+1][d]
    got = oracle_lib.router_score(h, R["W1"], R["b1"], R["W2"], R["b2"], act)
    pre = _f64(h) @ _f64(R["W1"]).T + _f64(R["b1"])
    z = np.maximum(pre, 0) if act == syn.ACT_RELU else pre * scipy.special.expit(pre)
    ref = z @ _f64(R["W2"]).T + _f64(R["b2"])
    bound = np.abs(z) @ np.abs(_f64(R["W2"])).T
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -23, atol=1e-12 * bound.max() + 1e-30)


def test_router_hand_example(oracle_lib):
    # h=[1,2]; W1=[[1,0],[0,-1]], b1=[.5,0] -> pre=[1.5,-2]
    h = np.array([[1, 2]], np.float32)
    W1 = np.array([[1, 0], [0, -1]], np.float32)
    b1 = np.array([0.5, 0], np.float32)
    W2 = np.array([[2, 1], [1, 1]], np.float32)
    b2 = np.array([0, -1], np.float32)
    relu = oracle_lib.router_score(h, W1, b1, W2, b2, syn.ACT_RELU)
    assert relu.tolist() == [[3.0, 0.5]]
    silu = oracle_lib.router_score(h, W1, b1, W2, b2, syn.ACT_SILU)
    z = [1.5 / (1 + math.exp(-1.5)), -2 / (1 + math.exp(2))]
    exp = [2 * z[0] + z[1], z[0] + z[1] - 1]
    np.testing.assert_allclose(silu[0], exp, rtol=1e-7)
    # no biases == zero biases
    nob = oracle_lib.router_score(h, W1, None, W2, None, syn.ACT_RELU)
    zb = oracle_lib.router_score(h, W1, np.zeros(2, np.float32), W2, np.zeros(2, np.float32),
                                 syn.ACT_RELU)
    assert np.array_equal(nob, zb)


# ----------------------------------------------------------------------------
# select_clusters
# ----------------------------------------------------------------------------
def _brute_select(s, size, kind, budget):
    order = sorted(range(len(s)), key=lambda c: (-float(s[c]), c))
    if kind == syn.BUDGET_CLUSTERS:
        k = min(max(int(budget), 1), len(s))
        chosen = order[:k]
    else:
        b = max(int(budget), 1)
        chosen, tot = [], 0
        for c in order:
            if tot >= b:
                break
            chosen.append(c)
            tot += int(size[c])
    return chosen, sum(int(size[c]) for c in chosen)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", [syn.BUDGET_CLUSTERS, syn.BUDGET_TOKENS])
def test_select_matches_brute_force(oracle_lib, seed, kind):
    g = np.random.default_rng(seed)
    M = int(g.integers(1, 300))
    n = 5
    # integer-valued scores make many ties; -0.0 and +0.0 must tie too
    s = g.integers(-3, 4, size=(n, M)).astype(np.float32)
    s[s == 0] = np.where(g.random((s == 0).sum()) < 0.5, -0.0, 0.0)
    size = g.integers(1, 50, size=M).astype(np.int32)
    if kind == syn.BUDGET_CLUSTERS:
        budget = g.integers(-2, M + 3, size=n).astype(np.int32)
    else:
        budget = g.integers(-5, int(size.sum()) + 10, size=n).astype(np.int32)
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, kind, budget)
    for row in range(n):
        chosen, tot = _brute_select(s[row], size, kind, budget[row])
        assert n_sel[row] == len(chosen)
        assert sel[row, : n_sel[row]].tolist() == chosen
        assert (sel[row, n_sel[row]:] == -1).all()
        assert sl_len[row] == tot


def test_select_token_budget_invariants(oracle_lib):
    cfg = syn.CONFIGS[1]
    size = syn.zipf_cluster_sizes(cfg.V, cfg.M, cfg.zipf_s)
    g = np.random.default_rng(7)
    s = g.standard_normal((40, cfg.M)).astype(np.float32)
    budget = g.integers(1, cfg.V, size=40).astype(np.int32)
    budget[:3] = [cfg.V, cfg.V + 5, 0]
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, syn.BUDGET_TOKENS, budget)
    for r in range(40):
        k = n_sel[r]
        chosen = sel[r, :k]
        # a prefix of the (score desc, id asc) order
        order = np.lexsort((np.arange(cfg.M), -s[r]))
        assert (chosen == order[:k]).all()
        tot = int(size[chosen].sum())
        assert tot == sl_len[r]
        b = max(int(budget[r]), 1)
        if k < cfg.M:
            assert tot >= b
        assert int(size[chosen[:-1]].sum()) < b  # minimal
    assert n_sel[0] == cfg.M and n_sel[1] == cfg.M and sl_len[0] == cfg.V
    assert n_sel[2] == 1  # budget 0 counts as 1 -> a single cluster


def test_select_cluster_budget_is_topk(oracle_lib):
    g = np.random.default_rng(3)
    s = g.standard_normal((4, 64)).astype(np.float32)
    size = np.full(64, 128, np.int32)
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, syn.BUDGET_CLUSTERS,
                                                    np.array([8, 6, 4, 4], np.int32))
    for r, k in enumerate([8, 6, 4, 4]):
        top = np.argsort(-s[r], kind="stable")[:k]
        assert sel[r, :k].tolist() == top.tolist()
        assert sl_len[r] == 128 * k


def test_budget_reading_reproduces_pages_shortlist_size(oracle_lib):
    """With the token-budget reading (shortest prefix reaching the budget),
    the Llama-shaped schedule 32K->16K gives a mean shortlist near the ~28K
    the pages report (DynaSpec summary, Evaluation Highlights); the rejected
    reading (largest prefix within budget) would give about 21K."""
    cfg = syn.CONFIGS[1]
    size = syn.zipf_cluster_sizes(cfg.V, cfg.M, cfg.zipf_s)
    g = np.random.default_rng(11)
    lens = []
    for t, b in enumerate(cfg.budget):
        s = g.standard_normal((200, cfg.M)).astype(np.float32)
        _, _, L = oracle_lib.select_clusters(s, size, syn.BUDGET_TOKENS, np.full(200, b, np.int32))
        lens.append(L.mean())
    assert 25000 < np.mean(lens) < 30500


# ----------------------------------------------------------------------------
# build_shortlist
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_build_is_sorted_union(oracle_lib, seed):
    g = np.random.default_rng(seed)
    V, M = int(g.integers(50, 3000)), int(g.integers(2, 40))
    cluster_of = g.integers(0, M, size=V).astype(np.int32)
    cluster_of[:M] = np.arange(M)  # every cluster non-empty
    n = 6
    sel = np.full((n, M), -1, np.int32)
    n_sel = g.integers(1, M + 1, size=n).astype(np.int32)
    for r in range(n):
        sel[r, : n_sel[r]] = g.permutation(M)[: n_sel[r]]
    st, off, ids = oracle_lib.build_shortlist(sel, n_sel, cluster_of)
    assert st == 0 and off[0] == 0
    for r in range(n):
        chosen = set(sel[r, : n_sel[r]].tolist())
        expect = sorted(y for y in range(V) if int(cluster_of[y]) in chosen)
        got = ids[off[r]: off[r + 1]].tolist()
        assert got == expect
        assert len(got) == sum(int((cluster_of == c).sum()) for c in chosen)


def test_build_full_budget_is_identity_and_chaining(oracle_lib):
    cfg = syn.CONFIGS[0]
    cluster_of, size = syn.make_clusters(cfg)
    s = np.random.default_rng(0).standard_normal((3, cfg.M)).astype(np.float32)
    sel, n_sel, sl_len = oracle_lib.select_clusters(s, size, syn.BUDGET_TOKENS,
                                                    np.full(3, cfg.V, np.int32))
    st, off, ids = oracle_lib.build_shortlist(sel, n_sel, cluster_of)
    assert st == 0
    for r in range(3):
        assert ids[off[r]: off[r + 1]].tolist() == list(range(cfg.V))
    # two chained calls (second starts where the first ended) == one call
    sel2, n2, _ = oracle_lib.select_clusters(s, size, syn.BUDGET_CLUSTERS, np.array([3, 5, 1], np.int32))
    st_a, off_a, ids_a = oracle_lib.build_shortlist(sel2, n2, cluster_of)
    st_b, off_b, ids_b = oracle_lib.build_shortlist(sel2[:1], n2[:1], cluster_of)
    st_c, off_c, ids_c = oracle_lib.build_shortlist(sel2[1:], n2[1:], cluster_of, base=int(off_b[-1]))
    assert off_c[0] == off_b[-1]
    assert np.array_equal(np.concatenate([off_b, off_c[1:]]), off_a)
    assert np.array_equal(np.concatenate([ids_b[: off_b[-1]], ids_c[off_c[0]: off_c[-1]]]),
                          ids_a[: off_a[-1]])


def test_build_capacity_and_bad_ids(oracle_lib):
    cluster_of = np.array([0, 1, 0, 1, 2, 2], np.int32)
    sel = np.array([[0, 2, -1], [1, -1, -1]], np.int32)
    n_sel = np.array([2, 1], np.int32)
    st, off, ids = oracle_lib.build_shortlist(sel, n_sel, cluster_of, capacity=5)
    assert st == 4  # capacity exceeded
    assert off.tolist() == [0, 4, 5]
    assert ids.tolist() == [0, 2, 4, 5, 1]
    st, off, ids = oracle_lib.build_shortlist(np.array([[0, 7, -1]], np.int32),
                                              np.array([2], np.int32), cluster_of)
    assert st == 1 and ids[: off[1]].tolist() == [0, 2]


# ----------------------------------------------------------------------------
# gathered LM head
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [syn.DT_F32, syn.DT_BF16])
def test_head_matches_float64_blas(oracle_lib, dtype):
    cfg = syn.shrink(syn.CONFIGS[0], dtype=dtype, V=1000, M=10)
    cluster_of = (np.arange(cfg.V) % cfg.M).astype(np.int32)
    W = syn.make_lm_head(cfg, cluster_of)
    g = np.random.default_rng(5)
    G, m = 3, 4
    h = syn._store(g.standard_normal((G, m, cfg.d)).astype(np.float32), dtype)
    lens = [17, 0, 333]
    sl_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sl_ids = np.concatenate([np.sort(g.choice(cfg.V, L, replace=False)) for L in lens]).astype(np.int32)
    got = oracle_lib.gathered_lm_head(W, h, sl_off, sl_ids)
    W64, h64 = _f64(W), _f64(h)
    for gi in range(G):
        S = sl_ids[sl_off[gi]: sl_off[gi + 1]]
        ref = h64[gi] @ W64[S].T  # [m][len]
        bound = np.abs(h64[gi]) @ np.abs(W64[S]).T
        blk = got[m * sl_off[gi]: m * sl_off[gi + 1]].reshape(m, len(S))
        if len(S) == 0:
            continue
        np.testing.assert_allclose(blk, ref, rtol=2.0 ** -23, atol=1e-13 * bound.max() + 1e-30)


def test_head_full_budget_equals_dense_and_gather_equals_dense(oracle_lib):
    cfg = syn.CONFIGS[0]
    cluster_of, _ = syn.make_clusters(cfg)
    W = syn.make_lm_head(cfg, cluster_of)
    h = syn.make_hidden(cfg)[0, :2]  # [2][d]
    dense = oracle_lib.dense_lm_head(W, h)
    full = oracle_lib.gathered_lm_head(W, h[None], np.array([0, cfg.V], np.int64),
                                       np.arange(cfg.V, dtype=np.int32))
    assert np.array_equal(full.reshape(2, cfg.V), dense)
    S = np.sort(np.random.default_rng(1).choice(cfg.V, 700, replace=False)).astype(np.int32)
    part = oracle_lib.gathered_lm_head(W, h[None], np.array([0, 700], np.int64), S)
    assert np.array_equal(part.reshape(2, 700), dense[:, S])
    ref = _f64(h) @ _f64(W).T
    np.testing.assert_allclose(dense, ref, rtol=2.0 ** -23, atol=1e-9)


def test_head_one_hot_rows(oracle_lib):
    # W[y] = e_{y mod d}: the logit is exactly h[y mod d] (catches transposes)
    V, d = 40, 8
    W = np.zeros((V, d), np.float32)
    W[np.arange(V), np.arange(V) % d] = 1.0
    h = np.arange(1, 2 * d + 1, dtype=np.float32).reshape(1, 2, d) * np.float32(0.5)
    S = np.array([3, 9, 17, 39], np.int32)
    got = oracle_lib.gathered_lm_head(W, h, np.array([0, 4], np.int64), S).reshape(2, 4)
    assert got.tolist() == [[h[0, i, y % d] for y in S] for i in range(2)]


# ----------------------------------------------------------------------------
# shortlist sampling
# ----------------------------------------------------------------------------
def test_sample_q_is_softmax(oracle_lib):
    g = np.random.default_rng(2)
    lens = [1, 5, 300]
    sl_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sl_ids = np.concatenate([np.arange(L) * 3 for L in lens]).astype(np.int32)
    logits = (g.standard_normal(int(sl_off[-1])) * 4).astype(np.float32)
    for tau in (1.0, float(np.float32(0.7))):  # the sampler receives an fp32 temperature
        tok, q, _ = oracle_lib.shortlist_sample(sl_off, sl_ids, logits, np.full(3, 0.5, np.float32),
                                                temperature=tau)
        for r in range(3):
            seg = slice(sl_off[r], sl_off[r + 1])
            ref = scipy.special.softmax(logits[seg].astype(np.float64) / tau)
            np.testing.assert_allclose(q[seg], ref, rtol=3e-7, atol=1e-37)


def test_sample_stratified_quadrature(oracle_lib):
    """With u_i = (i + 1/2)/N, token j is drawn N*q_j times up to one."""
    g = np.random.default_rng(4)
    L, N = 7, 1 << 14
    logits = g.standard_normal(L).astype(np.float32)
    ids = np.arange(100, 100 + L, dtype=np.int32)
    u = ((2 * np.arange(N) + 1) * 2.0 ** -15).astype(np.float32)
    sl_off = np.arange(N + 1, dtype=np.int64) * L
    tok, q, tie = oracle_lib.shortlist_sample(sl_off, np.tile(ids, N), np.tile(logits, N), u)
    counts = np.bincount(tok - 100, minlength=L)
    assert np.abs(counts - N * q[:L].astype(np.float64)).max() <= 1.0 + 1e-3
    assert not tie.any()


def test_sample_matches_numpy_inverse_cdf_full_vocab(oracle_lib):
    """Full-vocabulary shortlist == dense sampling: numpy cumsum (sequential,
    float64) + searchsorted gives the same token for every uniform."""
    g = np.random.default_rng(8)
    V, n = 5000, 64
    logits = (g.standard_normal((n, V)) * 3).astype(np.float32)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, n)
    sl_off = np.arange(n + 1, dtype=np.int64) * V
    tok, q, tie = oracle_lib.shortlist_sample(sl_off, np.tile(np.arange(V, dtype=np.int32), n),
                                              logits.reshape(-1), u)
    for r in range(n):
        e = np.exp(logits[r].astype(np.float64) - logits[r].max())
        c = np.cumsum(e)
        ref = int(np.searchsorted(c, u[r] * c[-1], side="right"))
        assert tie[r] or tok[r] == ref


def test_sample_chi_square_and_argmax(oracle_lib):
    g = np.random.default_rng(9)
    L, N = 12, 20000
    logits = g.standard_normal(L).astype(np.float32)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, N, instance=3)
    sl_off = np.arange(N + 1, dtype=np.int64) * L
    tok, q, _ = oracle_lib.shortlist_sample(sl_off, np.tile(np.arange(L, dtype=np.int32), N),
                                            np.tile(logits, N), u)
    obs = np.bincount(tok, minlength=L)
    p = scipy.special.softmax(logits.astype(np.float64))
    assert scipy.stats.chisquare(obs, N * p).pvalue > 1e-4
    # tau = 0: argmax, ties to the lowest token id; q one-hot
    lg = np.array([0.5, 2.0, -1.0, 2.0], np.float32)
    tok0, q0, _ = oracle_lib.shortlist_sample(np.array([0, 4], np.int64),
                                              np.array([10, 20, 30, 40], np.int32), lg,
                                              np.array([0.9], np.float32), temperature=0.0)
    assert tok0[0] == 20 and q0.tolist() == [0, 1, 0, 0]


def test_sample_temperature_is_logit_scaling(oracle_lib):
    g = np.random.default_rng(10)
    lg = (g.standard_normal(500) * 5).astype(np.float32)
    u = syn.make_uniforms(syn.CONFIGS[0], 9, 50)
    off = np.arange(51, dtype=np.int64) * 500
    ids = np.tile(np.arange(500, dtype=np.int32), 50)
    t2, q2, _ = oracle_lib.shortlist_sample(off, ids, np.tile(lg, 50), u, temperature=2.0)
    t1, q1, _ = oracle_lib.shortlist_sample(off, ids, np.tile(lg / np.float32(2), 50), u)
    assert np.array_equal(t1, t2) and np.array_equal(q1, q2)


# ----------------------------------------------------------------------------
# target softmax
# ----------------------------------------------------------------------------
def test_target_softmax_matches_scipy(oracle_lib):
    g = np.random.default_rng(12)
    lg = (g.standard_normal((3, 2, 4000)) * 3).astype(np.float32)
    p = oracle_lib.target_softmax(lg)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=-1)
    np.testing.assert_allclose(p, ref, rtol=3e-7, atol=1e-38)


# ----------------------------------------------------------------------------
# verification: the emitted tokens must be distributed as the target
# ----------------------------------------------------------------------------
TWO24 = 1 << 24


def _bisect(pred_true_low):
    """Number of k in [0, 2^24) for which a monotone predicate holds
    (it holds for every k below the count and for none above)."""
    lo, hi = 0, TWO24
    while lo < hi:
        mid = (lo + hi) // 2
        if pred_true_low(mid):
            lo = mid + 1
        else:
            hi = mid
    return lo


class _VerifyCase:
    def __init__(self, oracle_lib, V, T, seed):
        g = np.random.default_rng(seed)
        self.o, self.V, self.T = oracle_lib, V, T
        cluster_of = np.arange(V) // 2  # clusters of two tokens
        self.S, self.q = [], []
        for t in range(T):
            ncl = int(g.integers(1, V // 2 + 1))
            cl = g.choice(V // 2, ncl, replace=False)
            S = np.sort(np.flatnonzero(np.isin(cluster_of, cl))).astype(np.int32)
            q = g.dirichlet(np.full(len(S), 0.6)).astype(np.float32)
            self.S.append(S)
            self.q.append(q)
        p = g.dirichlet(np.full(V, 0.8), size=T + 1) + 1e-3
        self.p = (p / p.sum(1, keepdims=True)).astype(np.float32)[None]  # [1][T+1][V]
        self.sl_off = np.concatenate([[0], np.cumsum([len(s) for s in self.S])]).astype(np.int64)
        self.sl_ids = np.concatenate(self.S)
        self.qcat = np.concatenate(self.q)

    def run(self, draft, u_acc, u_fin):
        n, out, _ = self.o.verify_reject(np.asarray(draft, np.int32).reshape(self.T, 1),
                                         self.sl_off, self.sl_ids, self.qcat, self.p,
                                         np.asarray(u_acc, np.float32).reshape(self.T, 1),
                                         np.array([u_fin], np.float32))
        return int(n[0]), out[0]

    def accept_prob(self, t, x):
        draft = [int(self.S[k][0]) for k in range(self.T)]
        draft[t] = int(x)

        def accepted(k):
            ua = [0.0] * self.T
            ua[t] = k * 2.0 ** -24
            n, out = self.run(draft, ua, 0.5)
            return n > t
        return _bisect(accepted) / TWO24

    def token_dist(self, draft, u_acc, pos):
        """Distribution of out[pos] over u_fin (inverse CDF is monotone)."""
        prev = 0
        dist = np.zeros(self.V)
        for y in range(self.V):
            cnt = _bisect(lambda k: self.run(draft, u_acc, k * 2.0 ** -24)[1][pos] <= y)
            dist[y] = (cnt - prev) / TWO24
            prev = cnt
        return dist


@pytest.mark.parametrize("V,T,seed", [(4, 1, 0), (6, 2, 1), (8, 3, 2), (8, 2, 3), (6, 3, 4)])
def test_verify_reproduces_target_distribution(oracle_lib, V, T, seed):
    c = _VerifyCase(oracle_lib, V, T, seed)
    survive = 1.0
    for t in range(T):
        p_t = c.p[0, t].astype(np.float64)
        qd = np.zeros(V)
        qd[c.S[t]] = c.q[t]
        acc = {int(x): c.accept_prob(t, x) for x in c.S[t]}
        for x, a in acc.items():  # accept with min(1, p/q)
            assert abs(a - min(1.0, p_t[x] / qd[x])) <= 2.0 ** -23 + 1e-12
        beta = sum(qd[x] * a for x, a in acc.items())
        # closed form: acceptance probability = sum_x min(p, q) = 1 - TV(p, q)
        assert abs(beta - np.minimum(p_t, qd).sum()) < 1e-5
        # residual distribution seen after a rejection at t
        rej = [x for x in c.S[t] if acc[int(x)] < 1.0]
        if rej:
            draft = [int(c.S[k][0]) for k in range(T)]
            draft[t] = int(rej[0])
            ua = [0.0] * T
            ua[t] = 1.0 - 2.0 ** -24
            res = c.token_dist(draft, ua, t)
            emitted = qd * np.array([acc.get(y, 0.0) for y in range(V)]) + (1 - beta) * res
        else:
            emitted = qd * np.array([acc.get(y, 0.0) for y in range(V)])
        np.testing.assert_allclose(emitted, p_t / p_t.sum(), atol=2e-6)
        survive *= beta
    # bonus token after T acceptances is distributed as p_T
    draft = [int(c.S[k][0]) for k in range(T)]
    bonus = c.token_dist(draft, [0.0] * T, T)
    pT = c.p[0, T].astype(np.float64)
    np.testing.assert_allclose(bonus, pT / pT.sum(), atol=2e-6)


def test_verify_degenerate_residual_and_bonus(oracle_lib):
    V = 6
    S = np.array([1, 2, 4], np.int32)
    q = np.array([0.5, 0.3, 0.2], np.float32)
    p = np.zeros((1, 2, V), np.float32)
    p[0, 0, S] = q * np.float32(0.5)  # p <= q everywhere: residual has no mass
    p[0, 1] = np.array([0.1, 0.2, 0.3, 0.1, 0.2, 0.1], np.float32)
    off = np.array([0, 3], np.int64)
    n, out, _ = oracle_lib.verify_reject(np.array([[1]]), off, S, q, p,
                                         np.array([[0.99]], np.float32), np.array([0.7], np.float32))
    c = np.cumsum(p[0, 0].astype(np.float64))
    assert n[0] == 0 and out[0, 0] == int(np.searchsorted(c, 0.7 * c[-1], side="right"))
    assert out[0, 1] == -1
    # accepted draft -> bonus from p_T
    p[0, 0] = 0.2
    n, out, _ = oracle_lib.verify_reject(np.array([[2]]), off, S, q, p,
                                         np.array([[0.0]], np.float32), np.array([0.55], np.float32))
    c = np.cumsum(p[0, 1].astype(np.float64))
    assert n[0] == 1 and out[0, 0] == 2
    assert out[0, 1] == int(np.searchsorted(c, 0.55 * c[-1], side="right"))


# ----------------------------------------------------------------------------
# regression: the whole oracle step on the tiny workload
# ----------------------------------------------------------------------------
def test_oracle_step_matches_golden_c0(oracle_lib):
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    try:
        import make_golden
    finally:
        sys.path.remove(here)
    with open(os.path.join(here, "c0_oracle_step.json")) as f:
        want = json.load(f)
    got = json.loads(json.dumps(make_golden.c0_summary()))
    assert got == want


# ----------------------------------------------------------------------------
# static-shortlist baseline: the packed slab and the frequency-ranked list
# ----------------------------------------------------------------------------
def test_pack_rows_is_row_gather(oracle_lib):
    """The C copy against numpy fancy indexing (an independent gather), bf16
    and fp32, with NaN rows for ids outside [0, V)."""
    g = np.random.default_rng(3)
    W32 = g.standard_normal((50, 24)).astype(np.float32)
    Wb = syn.f32_to_bf16_bits(W32)
    ids = np.array([3, 49, 0, 3, -1, 50, 17], np.int32)
    ok = (ids >= 0) & (ids < 50)
    for W in (W32, Wb):
        out = oracle_lib.pack_rows(W, ids)
        assert out.dtype == W.dtype and out.shape == (7, 24)
        assert np.array_equal(out[ok], W[ids[ok]])
        if W.dtype == np.uint16:
            assert (out[~ok] == 0x7FC0).all()
        else:
            assert np.isnan(out[~ok]).all()


def test_packed_head_equals_gathered_head(oracle_lib):
    """The head over a packed slab with ids 0..L-1 is the gathered head over
    the list, bit for bit (same rows, same summation)."""
    cfg = syn.shrink(syn.CONFIGS[1], V=3000, d=64, M=20)
    cluster_of, _ = syn.make_clusters(cfg)
    W = syn.make_lm_head(cfg, cluster_of)
    ids = syn.static_shortlist(cfg, 700)
    h = syn.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((2, 1, 64)).astype(np.float32))
    off = np.array([0, 700, 1400], np.int64)
    both = np.concatenate([ids, ids])
    ref = oracle_lib.gathered_lm_head(W, h, off, both)
    slab = oracle_lib.pack_rows(W, ids)
    got = oracle_lib.gathered_lm_head(slab, h, off, np.tile(np.arange(700, dtype=np.int32), 2))
    assert np.array_equal(got, ref)


def test_static_shortlist_is_top_of_ranking():
    cfg = syn.CONFIGS[1]
    rank = syn.frequency_rank(cfg)
    assert np.array_equal(np.sort(rank), np.arange(cfg.V))
    s = syn.static_shortlist(cfg, 32768)
    assert s.shape == (32768,) and (np.diff(s) > 0).all()
    assert set(s.tolist()) == set(rank[:32768].tolist())
    assert np.array_equal(syn.static_shortlist(cfg, 10 ** 9), np.arange(cfg.V))


# ----------------------------------------------------------------------------
# spherical k-means over the LM-head rows
# ----------------------------------------------------------------------------
def _km_case(V=3000, d=64, M=20, seed=0):
    cfg = syn.shrink(syn.CONFIGS[1], V=V, d=d, M=M)
    cluster_of, size = syn.make_clusters(cfg)
    W = syn.make_lm_head(cfg, cluster_of)
    return cfg, cluster_of, size, W


def _ulp32(got, ref):
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    sp = np.spacing(np.maximum(np.abs(ref), np.float32(1e-38))).astype(np.float64)
    return (np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= sp).all()


def test_kmeans_inv_norms_vs_numpy(oracle_lib):
    cfg, _, _, W = _km_case()
    Wf = syn.bf16_bits_to_f32(W).astype(np.float64)
    ref = (1.0 / np.linalg.norm(Wf, axis=1)).astype(np.float32)
    assert _ulp32(oracle_lib.kmeans_inv_norms(W), ref)
    Wz = W.copy()
    Wz[5] = 0
    assert oracle_lib.kmeans_inv_norms(Wz)[5] == 0.0


def test_kmeans_assign_vs_brute_force(oracle_lib):
    cfg, cluster_of, _, W = _km_case(seed=1)
    g = np.random.default_rng(2)
    Cb = syn.f32_to_bf16_bits(g.standard_normal((cfg.M, cfg.d)).astype(np.float32))
    a, sc, tie = oracle_lib.kmeans_assign(W, Cb)
    S = syn.bf16_bits_to_f32(W).astype(np.float64) @ syn.bf16_bits_to_f32(Cb).astype(np.float64).T
    ref = S.argmax(1)  # first maximum: the lower cluster id on ties
    assert np.array_equal(a[~tie], ref[~tie])
    assert tie.mean() < 0.01
    assert np.allclose(sc, S.max(1), rtol=1e-6, atol=1e-6)
    # exact ties (two identical centroids) go to the lower id
    Cb2 = np.concatenate([Cb[:3], Cb[1:2]])
    a2, _, _ = oracle_lib.kmeans_assign(W, Cb2)
    assert not (a2 == 3).any()


def test_kmeans_update_vs_numpy_and_closed_forms(oracle_lib):
    cfg, cluster_of, _, W = _km_case(seed=2)
    inv = oracle_lib.kmeans_inv_norms(W)
    lab = syn.kmeans_init_assign(cfg, cluster_of, 0.3)
    lab[lab == 7] = 8  # cluster 7 empty: keeps its previous centroid
    lab[11] = 19
    lab[lab == 19] = 18
    lab[11] = 19  # cluster 19 has exactly one row
    Cp = np.random.default_rng(5).standard_normal((cfg.M, cfg.d)).astype(np.float32)
    Cn, size, nrm = oracle_lib.kmeans_update(W, inv, lab, Cp)
    Wf = syn.bf16_bits_to_f32(W).astype(np.float64) * inv.astype(np.float64)[:, None]
    for c in range(cfg.M):
        mem = lab == c
        assert size[c] == mem.sum()
        if not mem.any():
            assert np.array_equal(Cn[c], Cp[c])
            assert nrm[c] == 0.0
            continue
        s_c = Wf[mem].sum(0)
        assert abs(nrm[c] - np.linalg.norm(s_c)) <= 1e-12 * np.linalg.norm(s_c)
        assert _ulp32(Cn[c], (s_c / np.linalg.norm(s_c)).astype(np.float32))
    w11 = syn.bf16_bits_to_f32(W[11]).astype(np.float64)
    assert _ulp32(Cn[19], (w11 / np.linalg.norm(w11)).astype(np.float32))


def test_kmeans_objective_monotone_and_planted_recovery(oracle_lib):
    """Spherical k-means never decreases its objective (up to the bf16
    rounding of the centroids the assignment reads), and from a 30%-noisy
    start one update + one assignment recovers the planted partition of the
    clustered synthetic head."""
    cfg, cluster_of, _, W = _km_case(seed=3)
    inv = oracle_lib.kmeans_inv_norms(W)
    lab = syn.kmeans_init_assign(cfg, cluster_of, 0.3)
    assert (lab != cluster_of).mean() > 0.2
    Cp = np.zeros((cfg.M, cfg.d), np.float32)
    objs = []
    for it in range(4):
        Cn, size, nrm = oracle_lib.kmeans_update(W, inv, lab, Cp)
        objs.append(float(nrm.sum()))
        lab, _, _ = oracle_lib.kmeans_assign(W, syn.f32_to_bf16_bits(Cn))
        if it == 0:
            assert np.array_equal(lab, cluster_of)
        Cp = Cn
    assert all(b >= a * (1 - 1e-6) for a, b in zip(objs, objs[1:]))
    assert objs[-1] > objs[0]


# ----------------------------------------------------------------------------
# tree verification (multi-step speculative sampling): exact enumeration
# ----------------------------------------------------------------------------
class _TreeCase:
    """Root (node 0) with k leaf children (nodes 1..k) sharing shortlist S;
    child i's token is drawn from its own proposal q_i (all equal when
    same_q: one drafter sampling with replacement)."""

    def __init__(self, oracle_lib, V, nS, k, seed, same_q=False):
        g = np.random.default_rng(seed)
        self.o, self.V, self.k, self.m = oracle_lib, V, k, k
        self.S = np.sort(g.choice(V, nS, replace=False)).astype(np.int32)
        q = g.dirichlet(np.full(nS, 0.7), size=k).astype(np.float32)  # proposal of nodes 1..k
        if same_q:
            q[:] = q[0]
        p = g.dirichlet(np.full(V, 0.8), size=k + 1) + 1e-3
        self.p = (p / p.sum(1, keepdims=True)).astype(np.float32)[None]  # [1][k+1][V]
        self.qs = q
        self.qcat = q.reshape(-1)  # layout m * sl_off[b] + (i-1) * len + j
        self.sl_off = np.array([0, nS], np.int64)
        self.parent = np.zeros((1, k), np.int32)

    def run(self, toks, u_acc, u_fin):
        token = np.array([list(toks)], np.int32)
        ua = np.array([list(u_acc)], np.float32)
        n, out, path, _ = self.o.verify_tree(self.parent, token, self.sl_off, self.S, self.qcat,
                                             self.p, ua, np.array([u_fin], np.float32))
        return int(n[0]), out[0], path[0]


@pytest.mark.parametrize("V,nS,k,seed,same_q", [(5, 3, 2, 0, False), (6, 4, 3, 1, False),
                                                (4, 4, 2, 2, True), (6, 2, 3, 3, False),
                                                (5, 3, 3, 4, True)])
def test_verify_tree_reproduces_target_distribution(oracle_lib, V, nS, k, seed, same_q):
    """Exact enumeration: over every combination of child tokens (child i
    drawn from q_i) and the whole 2^-24 grid of uniforms (by bisection),
    the first emitted token is distributed as p_root, and the first child is
    accepted with probability min(1, p/q_1)."""
    import itertools
    c = _TreeCase(oracle_lib, V, nS, k, seed, same_q)
    p0 = c.p[0, 0].astype(np.float64)
    q1 = np.zeros(V)
    q1[c.S] = c.qs[0]
    hi = 1.0 - 2.0 ** -24
    emitted = np.zeros(V)
    for combo in itertools.product(range(nS), repeat=k):
        toks = [int(c.S[j]) for j in combo]
        w = float(np.prod([c.qs[i][j] for i, j in enumerate(combo)], dtype=np.float64))
        reach = 1.0
        for i in range(k):  # child i tried after children 0..i-1 were rejected
            def acc(kk, i=i):
                ua = [hi] * i + [kk * 2.0 ** -24] + [0.0] * (k - i - 1)
                n, out, path = c.run(toks, ua, 0.5)
                return n >= 1 and path[0] == i + 1
            a = _bisect(acc) / TWO24
            if i == 0:  # against the target itself: min(1, p/q)
                assert abs(a - min(1.0, p0[toks[0]] / q1[toks[0]])) <= 2.0 ** -23 + 1e-12
            emitted[toks[i]] += w * reach * a
            reach *= 1.0 - a
            if reach <= 0.0:
                break
        if reach > 0.0:  # every child rejected: the final draw from the residual
            prev = 0
            for y in range(V):
                cnt = _bisect(lambda kk: c.run(toks, [hi] * k, kk * 2.0 ** -24)[1][0] <= y)
                emitted[y] += w * reach * (cnt - prev) / TWO24
                prev = cnt
    np.testing.assert_allclose(emitted, p0 / p0.sum(), atol=4e-6 * k)


def test_verify_tree_bonus_and_childless_root(oracle_lib):
    c = _TreeCase(oracle_lib, 6, 3, 2, 7)
    # child 1 accepted (u = 0): the next token is the bonus from p of node 1
    toks = [int(c.S[0]), int(c.S[1])]
    prev, dist = 0, np.zeros(6)
    for y in range(6):
        cnt = _bisect(lambda kk: c.run(toks, [0.0, 0.0], kk * 2.0 ** -24)[1][1] <= y)
        dist[y] = (cnt - prev) / TWO24
        prev = cnt
    n, out, path = c.run(toks, [0.0, 0.0], 0.3)
    assert n == 1 and path[0] == 1 and out[0] == toks[0] and path[1] == -1 and out[2] == -1
    p1 = c.p[0, 1].astype(np.float64)
    np.testing.assert_allclose(dist, p1 / p1.sum(), atol=2e-6)
    # a root without children draws straight from p_root
    parent = np.array([[5, 5]], np.int32)  # no node has a parent in [0, i): all detached
    n, out, path, tie = oracle_lib.verify_tree(parent, np.array([[0, 1]], np.int32), c.sl_off,
                                               c.S, c.qcat, c.p, np.zeros((1, 2), np.float32),
                                               np.array([0.0], np.float32))
    assert n[0] == 0 and (path[0] == -1).all() and (out[0, 1:] == -1).all()
    assert out[0, 0] == int(np.flatnonzero(c.p[0, 0] > 0)[0])


def test_verify_tree_path_is_the_chain_verifier(oracle_lib):
    """A tree whose nodes form one path (parent of node i is i-1) is a
    drafted chain: outputs equal the chain verifier's (pinned above by its
    own enumeration) on the same proposals, targets and uniforms, wherever
    neither flags a near-threshold decision."""
    g = np.random.default_rng(11)
    B, T, V, nS = 6, 4, 40, 12
    S = [np.sort(g.choice(V, nS, replace=False)).astype(np.int32) for _ in range(B)]
    q = g.dirichlet(np.full(nS, 0.5), size=(B, T)).astype(np.float32)
    p = g.dirichlet(np.full(V, 0.5), size=(B, T + 1)).astype(np.float32)
    for b in range(B):  # make the drafts likely to be accepted part of the time
        p[b, :T, S[b]] += 0.5 * q[b].T
    p /= p.sum(-1, keepdims=True)
    draft = np.array([[S[b][g.integers(nS)] for b in range(B)] for _ in range(T)], np.int32)
    u_acc = g.random((T, B), dtype=np.float32)
    u_fin = g.random(B, dtype=np.float32)
    # chain layout: row t*B + b owns S[b] and q[b][t]
    c_off = np.arange(T * B + 1, dtype=np.int64) * nS
    c_ids = np.concatenate([S[r % B] for r in range(T * B)])
    c_q = np.concatenate([q[r % B, r // B] for r in range(T * B)])
    n_c, out_c, tie_c = oracle_lib.verify_reject(draft, c_off, c_ids, c_q, p, u_acc, u_fin)
    # tree layout: sequence b owns S[b]; node i's proposal is row i-1
    parent = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    t_off = np.arange(B + 1, dtype=np.int64) * nS
    n_t, out_t, path_t, tie_t = oracle_lib.verify_tree(
        parent, draft.T.copy(), t_off, np.concatenate(S), q.reshape(-1), p, u_acc.T.copy(),
        u_fin)
    ok = ~(tie_c | tie_t)
    assert ok.sum() >= B - 1 and 0 < n_c.sum() < B * T
    np.testing.assert_array_equal(n_t[ok], n_c[ok])
    np.testing.assert_array_equal(out_t[ok], out_c[ok])
    for b in np.flatnonzero(ok):
        np.testing.assert_array_equal(path_t[b, :n_t[b]], np.arange(1, n_t[b] + 1))


# ----------------------------------------------------------- router training
def test_topl_labels_brute_force(oracle_lib):
    """Top-L by (logit desc, id asc), brute force in Python, on tie-heavy
    rows; ids without a cluster are skipped; L >= V and L = 0 edge cases."""
    g = np.random.default_rng(5)
    n, V, M, L = 6, 300, 17, 12
    lg = g.integers(-5, 6, size=(n, V)).astype(np.float32)  # heavy ties
    lg[0] = g.standard_normal(V).astype(np.float32)
    cluster_of = g.integers(0, M, size=V).astype(np.int32)
    cluster_of[np.argsort(-lg[1], kind="stable")[0]] = -1  # row 1's best token has no cluster
    for LL in (L, 0, V + 5):
        got = oracle_lib.topl_labels(lg, cluster_of, M, LL)
        for i in range(n):
            top = sorted(range(V), key=lambda y: (-float(lg[i, y]), y))[:LL]
            ref = np.zeros(M, np.uint8)
            for y in top:
                if 0 <= cluster_of[y] < M:
                    ref[cluster_of[y]] = 1
            assert np.array_equal(got[i], ref), (LL, i)


def _router_case(seed, n=3, d=5, r=4, M=6, act=syn.ACT_SILU):
    g = np.random.default_rng(seed)
    h = g.standard_normal((n, d)).astype(np.float32)
    W1 = (g.standard_normal((r, d)) * 0.7).astype(np.float32)
    b1 = (g.standard_normal(r) * 0.3).astype(np.float32)
    if act == syn.ACT_RELU:  # keep every pre-activation away from the kink
        a = h.astype(np.float64) @ W1.T.astype(np.float64) + b1
        b1 = (b1 + np.where(np.abs(a) < 0.05, 0.1, 0.0).max(0)).astype(np.float32)
    W2 = (g.standard_normal((M, r)) * 0.7).astype(np.float32)
    b2 = (g.standard_normal(M) * 0.3).astype(np.float32)
    y = (g.random((n, M)) < 0.4).astype(np.uint8)
    return h, y, W1, b1, W2, b2


@pytest.mark.parametrize("act", [syn.ACT_RELU, syn.ACT_SILU])
def test_router_train_loss_is_log_loss(oracle_lib, act):
    """The step's loss is the mean binary cross entropy of sigmoid(router
    scores) against the labels, as sklearn computes it."""
    from scipy.special import expit
    from sklearn.metrics import log_loss
    h, y, W1, b1, W2, b2 = _router_case(1, n=7, d=9, r=8, M=11, act=act)
    loss, _, _ = oracle_lib.router_train_step(h, y, W1, b1, W2, b2, act, 0.0)
    s = oracle_lib.router_score(h, W1, b1, W2, b2, act).astype(np.float64)
    ref = log_loss(y.ravel(), expit(s.ravel()), labels=[0, 1])
    assert abs(loss - ref) <= 1e-6 * ref


@pytest.mark.parametrize("act", [syn.ACT_RELU, syn.ACT_SILU])
def test_router_train_gradients_match_finite_differences(oracle_lib, act):
    """Every gradient entry against a central difference of the loss."""
    h, y, W1, b1, W2, b2 = _router_case(2, act=act)
    _, grad, _ = oracle_lib.router_train_step(h, y, W1, b1, W2, b2, act, 0.0)
    params = {"W1": W1, "b1": b1, "W2": W2, "b2": b2}
    for name, P in params.items():
        flat = P.reshape(-1)
        for e in range(flat.size):
            hi, lo = flat.copy(), flat.copy()
            hi[e] = np.float32(flat[e] + np.float32(2e-3))
            lo[e] = np.float32(flat[e] - np.float32(2e-3))
            Lh = oracle_lib.router_train_step(h, y, **{**params, name: hi.reshape(P.shape)},
                                              act=act, lr=0.0)[0]
            Ll = oracle_lib.router_train_step(h, y, **{**params, name: lo.reshape(P.shape)},
                                              act=act, lr=0.0)[0]
            fd = (Lh - Ll) / (float(hi[e]) - float(lo[e]))
            an = grad[name].reshape(-1)[e]
            assert abs(fd - an) <= 2e-5 + 1e-3 * abs(an), (name, e, fd, an)


def test_router_train_step_update_and_zero_head(oracle_lib):
    """SGD moves every parameter by -lr * grad (rounded to fp32); with the
    second layer at zero the loss is log 2, db2 = mean(0.5 - y) per column
    and no gradient reaches the first layer."""
    h, y, W1, b1, W2, b2 = _router_case(3, n=5, d=6, r=4, M=3)
    lr = 0.37
    loss, grad, new = oracle_lib.router_train_step(h, y, W1, b1, W2, b2, syn.ACT_SILU, lr)
    for name, P in (("W1", W1), ("b1", b1), ("W2", W2), ("b2", b2)):
        ref = (P.astype(np.float64) - float(np.float32(lr)) * grad[name]).astype(np.float32)
        assert np.array_equal(new[name], ref), name
    W2z, b2z = np.zeros_like(W2), np.zeros_like(b2)
    loss, grad, _ = oracle_lib.router_train_step(h, y, W1, b1, W2z, b2z, syn.ACT_SILU, 0.0)
    assert abs(loss - np.log(2.0)) < 1e-15
    np.testing.assert_allclose(grad["b2"], (0.5 - y).sum(0) / y.size, rtol=0, atol=1e-16)
    assert not grad["W1"].any() and not grad["b1"].any()
