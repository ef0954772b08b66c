"""One speculative draft step on the GPU, through the C-ABI only.

``DraftStep`` owns the device buffers for one workload and enqueues:
  chains (batch B, depth T): ds_draft_chain (router/select/build of position
      t+1 on a second stream, overlapped with head + sample of position t),
      then ds_verify_reject_logits (verification straight from the target's
      logits) on the head stream;
  trees (B sequences x m nodes sharing one shortlist): router, select and
      build for the B roots, then one gathered head with m rows per group and
      one sample per node, then ds_verify_tree_logits (from the target
      logits of the m+1 nodes).
PyTorch only allocates memory and provides the streams.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import native as N
from . import synthetic as syn


def to_dev(a: np.ndarray | None, device="cuda") -> torch.Tensor | None:
    if a is None:
        return None
    src = np.ascontiguousarray(a)
    if src.dtype == np.uint16:  # bf16 bit patterns
        src = src.view(np.int16)
    host = torch.from_numpy(src)
    # a fresh tensor has canonical strides (numpy may give size-1 dims any stride)
    out = torch.empty(host.shape, dtype=host.dtype, device=device).copy_(host)
    return out.view(torch.bfloat16) if a.dtype == np.uint16 else out


def row_bounds(cfg: syn.Config, cluster_size: np.ndarray) -> np.ndarray:
    """Host-side upper bound of one shortlist's length at each position: the
    budget plus the largest cluster (token budgets; the prefix stops at the
    first cluster reaching the budget), or the k largest clusters (cluster
    budgets)."""
    srt = np.sort(cluster_size)[::-1].astype(np.int64)
    out = []
    for b in cfg.budget:
        if cfg.budget_kind == syn.BUDGET_TOKENS:
            per_row = min(int(cfg.V), max(int(b), 1) + int(srt[0]))
        else:
            k = min(max(int(b), 1), cfg.M)
            per_row = int(srt[:k].sum())
        out.append(per_row)
    return np.asarray(out, dtype=np.int64)


def shortlist_bounds(cfg: syn.Config, cluster_size: np.ndarray) -> np.ndarray:
    """Host-side upper bound of the shortlist rows of each position-call."""
    return row_bounds(cfg, cluster_size) * cfg.B


class DraftStep:
    """One draft step (chain or tree) and its verification from target
    logits.  ``q_mode``: "dense" writes the draft distribution q (the
    sampler's output, read back by verification and by host()); "stats"
    (temperature > 0) writes each draft row's statistics instead and
    verification recomputes q from the draft logits, bit for bit the same
    values, so tokens and verification outputs are those of "dense"."""

    def __init__(self, wl: syn.Workload, device="cuda", W: torch.Tensor | None = None,
                 temperature: float = 1.0, q_mode: str = "dense"):
        cfg = self.cfg = wl.cfg
        self.device = device
        self.temperature = float(temperature)
        if q_mode not in ("dense", "stats"):
            raise ValueError("q_mode is 'dense' or 'stats'")
        if q_mode == "stats" and not self.temperature > 0.0:
            raise ValueError("q_mode 'stats' needs a temperature > 0")
        self.q_mode = q_mode
        dev = lambda a: to_dev(a, device)  # noqa: E731
        self.W = W if W is not None else dev(wl.W)
        R = wl.router
        self.W1, self.b1, self.W2, self.b2 = (dev(R[k]) for k in ("W1", "b1", "W2", "b2"))
        self.cluster_of = dev(wl.cluster_of)
        self.cluster_size = dev(wl.cluster_size)
        self.err_flag = torch.zeros(1, dtype=torch.int32, device=device)
        # per-clustering preprocessing: chunk-prefix counts of every cluster
        self.cluster_index = N.cluster_index(self.cluster_of, cfg.M, err_flag=self.err_flag)
        self.h = dev(wl.h)
        self.budget = dev(wl.budget)
        self.u_draft = dev(wl.u_draft)
        self.u_acc = dev(wl.u_acc)
        self.u_fin = dev(wl.u_fin)
        self.target_logits = dev(wl.target_logits)
        B, T, M, V = cfg.B, cfg.T, cfg.M, cfg.V
        self.max_len = row_bounds(cfg, wl.cluster_size)
        self.max_rows = self.max_len * cfg.B
        self.capacity = int(self.max_rows.sum())
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.scores = torch.empty(T, B, M, **f32)
        self.sel = torch.empty(T, B, M, **i32)
        self.n_sel = torch.empty(T, B, **i32)
        self.sl_len = torch.empty(T, B, **i32)
        self.sl_off = torch.zeros(T * B + 1, dtype=torch.int64, device=device)
        self.sl_ids = torch.empty(max(self.capacity, 1), **i32)
        m = cfg.tree_nodes
        self.logits = torch.empty(max(self.capacity * m, 1), **f32)
        if q_mode == "dense":
            self.q, self.qstats = torch.empty(max(self.capacity * m, 1), **f32), None
        else:  # one ds_qstats record per draft row
            self.q, self.qstats = None, N.qstats_buffer(B * m if cfg.is_tree else T * B, device)
        self.token = torch.empty((B, m) if cfg.is_tree else (T, B), **i32)
        nbytes = N.draft_chain_workspace_bytes(B, T, V, cfg.r, int(self.max_len.max()))
        if cfg.is_tree:
            nbytes = max(nbytes, N.sample_workspace_bytes(B, m, int(self.max_len.max())))
        self.ws = N.workspace(nbytes, device)
        self.head_ws = N.workspace(N.head_workspace_bytes(B, m, V), device)
        self.router_stream = torch.cuda.Stream(device=device)
        if self.target_logits is not None:
            rows = syn.target_rows(cfg)
            self.p = torch.empty(B, rows, V, **f32)
            self.n_acc = torch.empty(B, **i32)
            self.out = torch.empty(B, rows, **i32)
            self.softmax_ws = N.workspace(N.softmax_workspace_bytes(B * rows, V), device)
            if cfg.is_tree:
                self.parent = dev(wl.parent)
                self.path = torch.empty(B, m, **i32)
                self.verify_ws = N.workspace(
                    N.verify_tree_logits_workspace_bytes(B, m, V, int(self.max_len[0])), device)
            else:
                self.verify_ws = N.workspace(N.verify_logits_workspace_bytes(B, T, V), device)
        self._events = None
        self._args = None
        if not cfg.is_tree:
            # stream-ordering events of ds_draft_chain (destroyed in close())
            self._events = N.HipEvents()
            self._sync = self._events.array(2 * T + 1, timing=False)
            self._args = self._chain_args()
            self._args.sync_events = ctypes.cast(self._sync, ctypes.c_void_p)

    def close(self) -> None:
        """Destroy the chain's HIP events (after the work that uses them)."""
        if self._events is not None:
            torch.cuda.synchronize(self.device)
            self._events.close()
            self._events = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ chains
    def _chain_args(self) -> N.ChainArgs:
        cfg = self.cfg
        p = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        return N.ChainArgs(
            B=cfg.B, T=cfg.T, V=cfg.V, d=cfg.d, r=cfg.r, M=cfg.M,
            dtype=N.BF16 if cfg.dtype == syn.DT_BF16 else N.F32, act=cfg.act,
            budget_kind=cfg.budget_kind, temperature=self.temperature,
            W=p(self.W), W1=p(self.W1), b1=p(self.b1), W2=p(self.W2), b2=p(self.b2),
            cluster_of=p(self.cluster_of), cluster_index=p(self.cluster_index),
            cluster_size=p(self.cluster_size), h=p(self.h),
            budget=p(self.budget), u_draft=p(self.u_draft), capacity=self.capacity,
            max_rows=self.max_rows.ctypes.data, max_len=self.max_len.ctypes.data,
            scores=p(self.scores), sel=p(self.sel),
            n_sel=p(self.n_sel), sl_len=p(self.sl_len), sl_off=p(self.sl_off),
            sl_ids=p(self.sl_ids), logits=p(self.logits), q=p(self.q), token=p(self.token),
            err_flag=p(self.err_flag), ws=p(self.ws), ws_bytes=self.ws.numel(),
            qstats=p(self.qstats))

    def set_W(self, W: torch.Tensor) -> None:
        """Point the head at another (identical) copy of W."""
        self.W = W
        if self._args is not None:
            self._args.W = W.data_ptr()

    def set_W_positions(self, Ws: list[torch.Tensor] | None) -> None:
        """One head matrix per draft position (None: W everywhere)."""
        if self._args is None:
            if Ws is not None:
                raise ValueError("per-position head matrices apply to chain drafting only")
            return
        if Ws is None:
            self._W_pos, self._args.W_pos = None, None
            return
        assert len(Ws) == self.cfg.T
        self._W_pos_keep = Ws
        self._W_pos = (ctypes.c_void_p * self.cfg.T)(*[w.data_ptr() for w in Ws])
        self._args.W_pos = ctypes.cast(self._W_pos, ctypes.c_void_p)

    def set_head_events(self, events) -> None:
        """events: ctypes array of hipEvent_t handles recorded around every
        head launch, two per position (2T for chains, 2 for trees), or None."""
        self._head_events = events
        if self._args is not None:
            self._args.head_events = (None if events is None
                                      else ctypes.cast(events, ctypes.c_void_p))

    def draft(self, stream=None) -> None:
        stream = stream or torch.cuda.current_stream()
        if self.cfg.is_tree:
            return self._draft_tree(stream)
        N.draft_chain(self._args, stream, self.router_stream)

    def verify(self, stream=None) -> None:
        stats = self.q_mode == "stats"
        if self.cfg.is_tree:
            if stats:
                N.verify_tree_logits_qstats(self.parent, self.token, self.sl_off, self.sl_ids,
                                            self.logits, self.qstats, self.temperature,
                                            self.target_logits, self.u_acc, self.u_fin,
                                            int(self.max_len[0]), self.n_acc, self.out,
                                            self.path, self.verify_ws, stream=stream)
                return
            N.verify_tree_logits(self.parent, self.token, self.sl_off, self.sl_ids, self.q,
                                 self.target_logits, self.u_acc, self.u_fin,
                                 int(self.max_len[0]), self.n_acc, self.out, self.path,
                                 self.verify_ws, stream=stream)
            return
        if stats:
            N.verify_reject_logits_qstats(self.token, self.sl_off, self.sl_ids, self.logits,
                                          self.qstats, self.temperature, self.target_logits,
                                          self.u_acc, self.u_fin, self.n_acc, self.out,
                                          self.verify_ws, stream=stream)
            return
        N.verify_reject_logits(self.token, self.sl_off, self.sl_ids, self.q, self.target_logits,
                               self.u_acc, self.u_fin, self.n_acc, self.out, self.verify_ws,
                               stream=stream)

    def target_probs(self) -> torch.Tensor:
        """The target probabilities the verification used (it works from the
        logits and writes none: computed here, for inspection)."""
        N.target_softmax(self.target_logits, self.p, self.softmax_ws)
        return self.p

    def step(self, stream=None) -> None:
        self.draft(stream)
        if self.target_logits is not None:
            self.verify(stream)

    def capture(self, stream) -> "N.Graph":
        """One whole step (draft + verification) as a HIP graph on `stream`
        (a non-default stream); replay it with graph.launch(stream)."""
        return N.capture(lambda: self.step(stream), stream)

    # ------------------------------------------------------------------- trees
    def _draft_tree(self, stream) -> None:
        cfg = self.cfg
        B, m, d = cfg.B, cfg.tree_nodes, cfg.d
        zbytes = (N.router_workspace_bytes(B, cfg.r) + 255) // 256 * 256
        bbytes = (N.build_workspace_bytes(B, cfg.V) + 255) // 256 * 256
        N.router_score(self.h, self.W1, self.b1, self.W2, self.b2, cfg.act, self.scores[0],
                       self.ws[:zbytes], n=B, ldh=(1 + m) * d, stream=stream)
        N.select_clusters(self.scores[0], self.cluster_size, cfg.budget_kind, self.budget[0],
                          self.sel[0], self.n_sel[0], self.sl_len[0], stream=stream)
        N.build_shortlist(self.sel[0], self.n_sel[0], self.cluster_of, self.cluster_index,
                          self.capacity, self.sl_off, self.sl_ids, self.err_flag,
                          self.ws[zbytes:zbytes + bbytes], stream=stream)
        ev = getattr(self, "_head_events", None)
        N.gathered_lm_head(self.W, self.h[:, 1:], self.sl_off, self.sl_ids, self.max_rows[0],
                           self.logits, self.head_ws, G=B, m=m, ldh_g=(1 + m) * d,
                           stream=stream, events=None if ev is None else (ev[0], ev[1]))
        if self.q_mode == "stats":
            N.shortlist_sample_stats(self.sl_off, self.sl_ids, self.logits, self.temperature,
                                     self.u_draft, self.token, self.qstats, self.ws,
                                     max_len=int(self.max_len[0]), m=m, stream=stream)
            return
        N.shortlist_sample(self.sl_off, self.sl_ids, self.logits, self.temperature,
                           self.u_draft, self.token, self.q, self.ws,
                           max_len=int(self.max_len[0]), m=m, stream=stream)

    # ----------------------------------------------------------------- results
    def host(self) -> dict:
        torch.cuda.synchronize(self.device)
        n = int(self.sl_off[-1].item())
        r = {k: getattr(self, k).cpu().numpy() for k in
             ("scores", "sel", "n_sel", "sl_len", "sl_off", "token", "err_flag")}
        r["sl_ids"] = self.sl_ids[:n].cpu().numpy()
        mm = self.cfg.tree_nodes
        r["logits"] = self.logits[: n * mm].cpu().numpy()
        if self.q is not None:
            r["q"] = self.q[: n * mm].cpu().numpy()
        else:  # fp32 M at byte 0, fp64 1/Z at byte 8 of each 16-byte record
            raw = self.qstats.cpu().numpy()
            r["qstats_M"] = raw.view(np.float32)[0::4].copy()
            r["qstats_rZ"] = raw.view(np.float64)[1::2].copy()
        if self.target_logits is not None:
            r.update(n_acc=self.n_acc.cpu().numpy(), out=self.out.cpu().numpy(),
                     p=self.target_probs().cpu().numpy())
            if self.cfg.is_tree:
                r["path"] = self.path.cpu().numpy()
        return r


class StaticStep:
    """The static baseline the pages compare against (DynaSpec abstract, on
    FR-Spec / VocabTrim: drafting from a fixed, frequency-ranked shortlist):
    every position drafts from the same list, with no router, selection or
    build, then the same verification.  ``packed``: the list's rows are
    copied once into a contiguous slab (ds_pack_rows) and the head runs over
    the slab (ids 0..L-1) instead of gathering from W; the sampler still
    reports real token ids."""

    def __init__(self, wl: syn.Workload, static_ids: np.ndarray, device="cuda",
                 W: torch.Tensor | None = None, packed: bool = False,
                 temperature: float = 1.0, q_mode: str = "dense"):
        cfg = self.cfg = wl.cfg
        assert not cfg.is_tree, "the static step drafts chains"
        self.device = device
        self.temperature = float(temperature)
        if q_mode not in ("dense", "stats") or (q_mode == "stats" and not self.temperature > 0):
            raise ValueError("q_mode is 'dense', or 'stats' with a temperature > 0")
        self.q_mode = q_mode
        self.packed = packed
        dev = lambda a: to_dev(a, device)  # noqa: E731
        B, T, V, d = cfg.B, cfg.T, cfg.V, cfg.d
        L = self.L = int(static_ids.shape[0])
        self.W = W if W is not None else dev(wl.W)
        self.h = dev(wl.h)
        self.u_draft = dev(wl.u_draft)
        self.u_acc = dev(wl.u_acc)
        self.u_fin = dev(wl.u_fin)
        self.target_logits = dev(wl.target_logits)
        self.static_ids = dev(static_ids)
        self.sl_off = dev((np.arange(T * B + 1) * L).astype(np.int64))
        self.sl_ids = dev(np.tile(static_ids, T * B).astype(np.int32))
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        if packed:
            self.slab = torch.empty(L, d, dtype=self.W.dtype, device=device)
            N.pack_rows(self.W, self.static_ids, self.slab)
            self.head_ids = dev(np.tile(np.arange(L, dtype=np.int32), T * B))
        self.logits = torch.empty(max(T * B * L, 1), **f32)
        if q_mode == "dense":
            self.q, self.qstats = torch.empty(max(T * B * L, 1), **f32), None
        else:
            self.q, self.qstats = None, N.qstats_buffer(T * B, device)
        self.token = torch.empty(T, B, **i32)
        self.err_flag = torch.zeros(1, **i32)
        self.head_ws = N.workspace(N.head_workspace_bytes(B, 1, L if packed else V), device)
        self.sample_ws = N.workspace(N.sample_workspace_bytes(B, 1, max(L, 1)), device)
        if self.target_logits is not None:
            self.p = torch.empty(B, T + 1, V, **f32)
            self.n_acc = torch.empty(B, **i32)
            self.out = torch.empty(B, T + 1, **i32)
            self.softmax_ws = N.workspace(N.softmax_workspace_bytes(B * (T + 1), V), device)
            self.verify_ws = N.workspace(N.verify_logits_workspace_bytes(B, T, V), device)
        self._W_pos = None
        self._head_events = None

    def head_matrix(self) -> torch.Tensor:
        """What the head reads: the packed slab, or W."""
        return self.slab if self.packed else self.W

    def set_W_positions(self, Ws: list[torch.Tensor] | None) -> None:
        """One head matrix per draft position (identical copies of the slab,
        or of W), or None."""
        assert Ws is None or len(Ws) == self.cfg.T
        self._W_pos = Ws

    def set_head_events(self, events) -> None:
        self._head_events = events

    def draft(self, stream=None) -> None:
        cfg = self.cfg
        B, T, d = cfg.B, cfg.T, cfg.d
        ids = self.head_ids if self.packed else self.sl_ids
        for t in range(T):
            rb = t * B
            Wt = self._W_pos[t] if self._W_pos is not None else self.head_matrix()
            ev = self._head_events
            N.gathered_lm_head(Wt, self.h[:, t + 1], self.sl_off[rb:rb + B + 1], ids, B * self.L,
                               self.logits, self.head_ws, G=B, m=1, ldh_g=(T + 1) * d,
                               stream=stream,
                               events=None if ev is None else (ev[2 * t], ev[2 * t + 1]))
            if self.q_mode == "stats":
                N.shortlist_sample_stats(self.sl_off[rb:rb + B + 1], self.sl_ids, self.logits,
                                         self.temperature, self.u_draft[t], self.token[t],
                                         self.qstats[rb * N.QSTATS_BYTES:], self.sample_ws,
                                         max_len=self.L, stream=stream)
                continue
            N.shortlist_sample(self.sl_off[rb:rb + B + 1], self.sl_ids, self.logits,
                               self.temperature, self.u_draft[t], self.token[t], self.q,
                               self.sample_ws, max_len=self.L, stream=stream)

    def verify(self, stream=None) -> None:
        if self.q_mode == "stats":
            N.verify_reject_logits_qstats(self.token, self.sl_off, self.sl_ids, self.logits,
                                          self.qstats, self.temperature, self.target_logits,
                                          self.u_acc, self.u_fin, self.n_acc, self.out,
                                          self.verify_ws, stream=stream)
            return
        N.verify_reject_logits(self.token, self.sl_off, self.sl_ids, self.q, self.target_logits,
                               self.u_acc, self.u_fin, self.n_acc, self.out, self.verify_ws,
                               stream=stream)

    def target_probs(self) -> torch.Tensor:
        """The target probabilities (computed here, for inspection)."""
        N.target_softmax(self.target_logits, self.p, self.softmax_ws)
        return self.p

    def step(self, stream=None) -> None:
        self.draft(stream)
        if self.target_logits is not None:
            self.verify(stream)

    def capture(self, stream) -> "N.Graph":
        return N.capture(lambda: self.step(stream), stream)

    def host(self) -> dict:
        torch.cuda.synchronize(self.device)
        r = {k: getattr(self, k).cpu().numpy() for k in ("sl_off", "token", "err_flag")}
        r["sl_ids"] = self.sl_ids.cpu().numpy()
        r["logits"] = self.logits.cpu().numpy()
        if self.q is not None:
            r["q"] = self.q.cpu().numpy()
        if self.target_logits is not None:
            r.update(n_acc=self.n_acc.cpu().numpy(), out=self.out.cpu().numpy(),
                     p=self.target_probs().cpu().numpy())
        return r
