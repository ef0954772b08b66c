"""One speculative draft step composed from the oracle's functions
(TEST INFRASTRUCTURE ONLY).

Chains (batch B, depth T): for each position t the router reads h[:, t]
(H_{t-1} in the pages' notation), clusters are selected under budget[t], the
shortlist is built (rows are position-major, offsets chained across
positions), the head projects h[:, t+1] (H_t) onto it and a token is sampled
with u_draft[t].  Then the target distribution is the softmax of the target
logits and the drafts are verified.  Trees (tree_nodes > 1): one router row
per sequence (h[:, 0]), one shortlist per sequence shared by its nodes
h[:, 1:], one sample per node (node i's token from its own row), then the
tree is verified by multi-step speculative sampling against the target at
every node.

Sources: DynaSpec summary page, "Pipeline Flow" (router, drafter,
synchronisation and gathered projection, rejection-sampling verification) and
"Problem Definition" (router input H_{t-1}).
"""
from __future__ import annotations

import numpy as np

import oracle


def run_step(wl, temperature: float = 1.0, p: np.ndarray | None = None) -> dict:
    cfg = wl.cfg
    B, T, M, V = cfg.B, cfg.T, cfg.M, cfg.V
    R = wl.router
    res = {"scores": [], "sel": [], "n_sel": [], "sl_len": [], "status": []}
    if cfg.is_tree:
        m = cfg.tree_nodes
        sc = oracle.router_score(wl.h[:, 0], R["W1"], R["b1"], R["W2"], R["b2"], cfg.act)
        sel, n_sel, sl_len = oracle.select_clusters(sc, wl.cluster_size, cfg.budget_kind, wl.budget[0])
        st, sl_off, sl_ids = oracle.build_shortlist(sel, n_sel, wl.cluster_of)
        logits = oracle.gathered_lm_head(wl.W, np.ascontiguousarray(wl.h[:, 1:]), sl_off, sl_ids)
        tok, q, tie = oracle.shortlist_sample(sl_off, sl_ids, logits, wl.u_draft.reshape(-1), m,
                                              temperature)
        res.update(scores=[sc], sel=[sel], n_sel=[n_sel], sl_len=[sl_len], status=[st],
                   sl_off=sl_off, sl_ids=sl_ids[:sl_off[-1]], logits=logits, token=tok, q=q,
                   tie=tie)
        if wl.target_logits is not None:
            if p is None:
                p = oracle.target_softmax(wl.target_logits)
            n_acc, out, path, vtie = oracle.verify_tree(wl.parent, tok.reshape(B, m), sl_off,
                                                        sl_ids[:sl_off[-1]], q, p, wl.u_acc,
                                                        wl.u_fin)
            res.update(p=p, n_acc=n_acc, out=out, path=path, verify_tie=vtie)
        return res
    offs = [np.zeros(1, np.int64)]
    ids, logit_parts, q_parts, toks, ties = [], [], [], [], []
    base = 0
    for t in range(T):
        sc = oracle.router_score(wl.h[:, t], R["W1"], R["b1"], R["W2"], R["b2"], cfg.act)
        sel, n_sel, sl_len = oracle.select_clusters(sc, wl.cluster_size, cfg.budget_kind, wl.budget[t])
        st, off_t, ids_t = oracle.build_shortlist(sel, n_sel, wl.cluster_of, base=base)
        lo, hi = int(off_t[0]), int(off_t[-1])
        ids_t = ids_t[lo:hi]
        local_off = off_t - lo
        lg = oracle.gathered_lm_head(wl.W, np.ascontiguousarray(wl.h[:, t + 1][:, None, :]),
                                     local_off, ids_t)
        tok, q, tie = oracle.shortlist_sample(local_off, ids_t, lg, wl.u_draft[t], 1, temperature)
        for k, v in (("scores", sc), ("sel", sel), ("n_sel", n_sel), ("sl_len", sl_len),
                     ("status", st)):
            res[k].append(v)
        offs.append(off_t[1:])
        ids.append(ids_t)
        logit_parts.append(lg)
        q_parts.append(q)
        toks.append(tok)
        ties.append(tie)
        base = hi
    sl_off = np.concatenate(offs)
    sl_ids = np.concatenate(ids)
    q = np.concatenate(q_parts)
    draft = np.stack(toks)  # [T][B]
    res.update(sl_off=sl_off, sl_ids=sl_ids, logits=np.concatenate(logit_parts), q=q,
               token=draft, tie=np.stack(ties))
    if wl.target_logits is not None:
        if p is None:
            p = oracle.target_softmax(wl.target_logits)
        n_acc, out, vtie = oracle.verify_reject(draft, sl_off, sl_ids, q, p, wl.u_acc, wl.u_fin)
        res.update(p=p, n_acc=n_acc, out=out, verify_tie=vtie)
    return res


def run_static_step(wl, static_ids: np.ndarray, temperature: float = 1.0,
                    p: np.ndarray | None = None) -> dict:
    """The static baseline's step: every position drafts from the same fixed
    shortlist (no router, selection or build), then the same verification.
    Source: DynaSpec abstract, on fixed frequency-ranked shortlists
    (FR-Spec, VocabTrim)."""
    cfg = wl.cfg
    B, T = cfg.B, cfg.T
    L = int(static_ids.shape[0])
    local_off = (np.arange(B + 1) * L).astype(np.int64)
    ids_t = np.tile(static_ids, B)
    lg_parts, q_parts, toks, ties = [], [], [], []
    for t in range(T):
        lg = oracle.gathered_lm_head(wl.W, np.ascontiguousarray(wl.h[:, t + 1][:, None, :]),
                                     local_off, ids_t)
        tok, q, tie = oracle.shortlist_sample(local_off, ids_t, lg, wl.u_draft[t], 1, temperature)
        lg_parts.append(lg)
        q_parts.append(q)
        toks.append(tok)
        ties.append(tie)
    sl_off = (np.arange(T * B + 1) * L).astype(np.int64)
    sl_ids = np.tile(static_ids, T * B)
    q = np.concatenate(q_parts)
    draft = np.stack(toks)
    res = dict(sl_off=sl_off, sl_ids=sl_ids, logits=np.concatenate(lg_parts), q=q, token=draft,
               tie=np.stack(ties))
    if wl.target_logits is not None:
        if p is None:
            p = oracle.target_softmax(wl.target_logits)
        n_acc, out, vtie = oracle.verify_reject(draft, sl_off, sl_ids, q, p, wl.u_acc, wl.u_fin)
        res.update(p=p, n_acc=n_acc, out=out, verify_tie=vtie)
    return res
