"""Validity of draws that fall in a tie zone.

Where the threshold u * total lies within rounding of a boundary of the
cumulative weights (the oracle flags these), the GPU's fixed-association
sums may take the entry on either side of that boundary.  Such a draw is not
compared with the oracle's.  It must still be a real draw: an entry with
positive weight that is the oracle's pick or one of its neighbours among
the positive-weight entries.
"""
import numpy as np


def adjacent_ok(w, ref_pos, got_pos):
    """got_pos is ref_pos or the positive-weight entry just before or after
    it (positions index the weight vector w)."""
    if got_pos < 0 or got_pos >= w.shape[0] or not w[got_pos] > 0:
        return False
    nz = np.flatnonzero(w > 0)
    k = int(np.searchsorted(nz, ref_pos))
    allowed = set(int(nz[i]) for i in (k - 1, k, k + 1) if 0 <= i < nz.shape[0])
    return int(got_pos) in allowed


def check_sample_ties(got, ref, tie, sl_off, sl_ids, q_ref, m=1):
    """Sampler draws (row r = group r // m, head row r % m; q in the ragged
    layout m * off + i * len): tie rows must be adjacent draws."""
    for r in np.flatnonzero(tie):
        if got[r] == ref[r]:
            continue
        g, i = divmod(int(r), m)
        off, length = int(sl_off[g]), int(sl_off[g + 1] - sl_off[g])
        ids = np.asarray(sl_ids[off:off + length])
        w = np.asarray(q_ref[m * off + i * length: m * off + (i + 1) * length], np.float64)
        ref_pos = int(np.searchsorted(ids, ref[r]))
        hit = np.flatnonzero(ids == got[r])
        assert hit.shape[0] == 1, "row %d: token %d is not on the shortlist" % (r, got[r])
        assert adjacent_ok(w, ref_pos, int(hit[0])), "row %d: %d not next to %d" % (r, got[r],
                                                                                   ref[r])


def check_verify_ties(out, ref_out, n_acc, tie, draft, sl_off, sl_ids, q, p):
    """Chain verification: in tie sequences every emitted token but the drawn
    one equals the oracle's; the drawn one (position n_acc) is an adjacent
    draw from the residual max(0, p - q) (from p itself if that has no mass,
    and from p_T after T acceptances)."""
    T, B = np.asarray(draft).shape
    V = p.shape[-1]
    for b in np.flatnonzero(tie):
        t = int(n_acc[b])
        keep = np.arange(T + 1) != t
        assert np.array_equal(out[b][keep], ref_out[b][keep]), b
        pt = np.asarray(p[b, t], np.float64)
        w = pt
        if t < T:
            row = t * B + b
            qd = np.zeros(V)
            ids = np.asarray(sl_ids[sl_off[row]:sl_off[row + 1]])
            ok = (ids >= 0) & (ids < V)
            qd[ids[ok]] = np.asarray(q[sl_off[row]:sl_off[row + 1]], np.float64)[ok]
            res = np.maximum(pt - qd, 0.0)
            if res.sum() > 0:
                w = res
        if out[b][t] != ref_out[b][t]:
            assert adjacent_ok(w, int(ref_out[b][t]), int(out[b][t])), (b, out[b][t],
                                                                        ref_out[b][t])
