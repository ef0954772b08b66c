"""Distribution of the emitted tokens (DynaSpec abstract: verification over
the whole vocabulary keeps the output exact; summary page, "Pipeline Flow:
Rejection Sampling Verification").

Speculative sampling emits, at the first position, a token distributed
exactly as the target's p_0 whatever the draft distribution q_0 is, and
after an acceptance the bonus token is distributed as p_1.  These tests draw
many independent trials through the GPU verifier (every trial: a fresh
draft token x ~ q_0 and fresh uniforms; the same shortlist and target rows)
and compare the emitted tokens with p by a chi-square test over equal-mass
bins, and the acceptance rate with its closed form sum_y min(p_0, q_0).
Shapes: the Llama-shaped (V = 128256) and Gemma-shaped (V = 262144)
vocabularies with shortlists of their budgets' size; targets correlated
with the draft (high acceptance, few residual draws) or independent of it
(mostly residual draws).

Each test also checks that the chi-square test has the power to see
plausible mistakes: the accept test with p and q swapped, and (with
correlated targets, where acceptance is common) drawing from p_0 instead of
the residual after a rejection.  Their binned distributions are computed in
closed form, and the expected statistic under each must lie far beyond the
rejection threshold at the test's sample size.
"""
import numpy as np
import pytest
import torch
from scipy import stats

from dynamic_vocabulary_draft_amd.pipeline import to_dev

pytestmark = pytest.mark.gpu

NBINS = 200
PVALUE_FLOOR = 1e-5


@pytest.fixture(scope="module")
def N():
    from dynamic_vocabulary_draft_amd import native
    return native


def _softmax64(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _bins(p):
    """Equal-mass bins over the tokens ordered by decreasing p."""
    order = np.argsort(-p, kind="stable")
    cum = np.cumsum(p[order]) - p[order]  # mass before each token
    b = np.minimum((cum * NBINS).astype(np.int64), NBINS - 1)
    binof = np.empty(p.shape[0], np.int64)
    binof[order] = b
    return binof


def _chi2(tokens, p):
    binof = _bins(p)
    mass = np.bincount(binof, weights=p, minlength=NBINS)
    keep = mass > 0
    n = tokens.shape[0]
    obs = np.bincount(binof[tokens], minlength=NBINS)[keep]
    exp = n * mass[keep] / mass.sum()
    stat = float(((obs - exp) ** 2 / exp).sum())
    df = int(keep.sum()) - 1
    return stat, df, float(stats.chi2.sf(stat, df)), binof, mass


def _noncentrality(n, p, wrong, binof, mass):
    """Expected excess of the chi-square statistic when tokens follow `wrong`."""
    wm = np.bincount(binof, weights=wrong, minlength=NBINS)
    keep = mass > 0
    return float(n * (((wm[keep] - mass[keep]) ** 2) / mass[keep]).sum())


def _case(V, L, mode, seed):
    g = np.random.default_rng(seed)
    ids = np.sort(g.choice(V, L, replace=False)).astype(np.int32)
    dl = (g.standard_normal(L) * 2).astype(np.float32)
    q32 = _softmax64(dl).astype(np.float32)
    tl = np.empty((2, V), np.float32)
    for t in range(2):
        if mode == "correlated":
            row = np.full(V, -6.0)
            row[ids] = dl
            tl[t] = (row + g.standard_normal(V) * 0.5).astype(np.float32)
        else:
            tl[t] = (g.standard_normal(V) * 3).astype(np.float32)
    return ids, q32, tl


@pytest.mark.parametrize("V,L,mode", [(128256, 28000, "correlated"),
                                      (128256, 28000, "independent"),
                                      (262144, 40000, "correlated"),
                                      (262144, 40000, "independent")])
def test_verify_emits_target_distribution(N, V, L, mode):
    B, calls, T = 512, 400, 1
    ids, q32, tl = _case(V, L, mode, seed=V + L + len(mode))
    p0, p1 = _softmax64(tl[0]), _softmax64(tl[1])
    qd = np.zeros(V)
    qd[ids] = q32.astype(np.float64) / q32.astype(np.float64).sum()
    alpha = float(np.minimum(p0, qd).sum())  # acceptance probability

    dev = "cuda"
    logits = torch.from_numpy(tl).to(dev).unsqueeze(0).expand(B, 2, V).contiguous()
    sl_off = to_dev((np.arange(B + 1) * L).astype(np.int64))
    sl_ids = to_dev(np.tile(ids, B))
    q = to_dev(np.tile(q32, B))
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty(B, T + 1, dtype=torch.int32, device=dev)
    ws = N.workspace(N.verify_logits_workspace_bytes(B, T, V))
    g = np.random.default_rng(V + 3 * L)
    cq = np.cumsum(q32.astype(np.float64))
    first, bonus, accepted = [], [], 0
    for _ in range(calls):
        x = ids[np.minimum(np.searchsorted(cq, g.random(B) * cq[-1], side="right"), L - 1)]
        # uniforms on the 2^-24 grid: exact in fp32 and below 1
        u_acc = (g.integers(0, 1 << 24, size=(T, B)) * 2.0 ** -24).astype(np.float32)
        u_fin = (g.integers(0, 1 << 24, size=B) * 2.0 ** -24).astype(np.float32)
        N.verify_reject_logits(to_dev(x.reshape(T, B).astype(np.int32)), sl_off, sl_ids, q, logits,
                               to_dev(u_acc), to_dev(u_fin), n_acc, out, ws)
        o = out.cpu().numpy()
        na = n_acc.cpu().numpy()
        assert ((na == 0) | (na == 1)).all()
        assert (o[:, 0] >= 0).all() and (o[:, 0] < V).all()
        acc = na == 1
        assert (o[acc, 0] == x[acc]).all()  # an accepted draft is emitted as is
        assert (o[~acc, 1] == -1).all()
        first.append(o[:, 0])
        bonus.append(o[acc, 1])
        accepted += int(acc.sum())
    first = np.concatenate(first)
    bonus = np.concatenate(bonus)
    n = first.shape[0]

    # acceptance rate against sum_y min(p_0, q_0): within 5 standard deviations
    sd = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(accepted / n - alpha) <= 5 * sd + 1e-12, (accepted / n, alpha)
    if mode == "correlated":
        assert alpha > 0.5
    else:
        assert alpha < 0.2

    stat, df, pv, binof, mass = _chi2(first, p0)
    assert pv > PVALUE_FLOOR, "first token: chi2 %.1f on %d df (p = %.2e)" % (stat, df, pv)
    assert (bonus >= 0).all() and (bonus < V).all()
    stat1, df1, pv1, _, _ = _chi2(bonus, p1)
    assert pv1 > PVALUE_FLOOR, "bonus token: chi2 %.1f on %d df (p = %.2e)" % (stat1, df1, pv1)

    # power: the statistic expected under each mistake is far past the
    # threshold (threshold = the chi-square quantile at the p-value floor)
    thr = float(stats.chi2.isf(PVALUE_FLOOR, df))
    wrong_p = np.minimum(p0, qd) + (1 - alpha) * p0  # rejection draws from p_0
    acc_sw = qd * np.minimum(1.0, np.divide(qd, p0, out=np.ones_like(qd), where=p0 > 0))
    res = np.maximum(p0 - qd, 0.0)
    wrong_sw = acc_sw + (1 - acc_sw.sum()) * res / res.sum()  # accept test with p, q swapped
    # (drawing from p_0 on rejection differs from the truth only through the
    # accepted share alpha: with independent targets alpha is a few percent
    # and that mistake is left to the correlated cases)
    for wrong in ((wrong_p, wrong_sw) if mode == "correlated" else (wrong_sw,)):
        lam = _noncentrality(n, p0, wrong, binof, mass)
        assert df + lam > thr + 6 * np.sqrt(2 * (df + 2 * lam)), (lam, thr)
