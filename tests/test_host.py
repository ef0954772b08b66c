"""Host-side tests (no GPU): the C-ABI library loads and exports everything
include/dynaspec.h declares, rejects bad arguments before enqueueing, and the
host logic (seeded generator, capacity bounds) holds.

Every validation case below is rejected on the host before any HIP call, so
none of them can launch a kernel.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

from dynamic_vocabulary_draft_amd import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dynaspec.h")


@pytest.fixture(scope="module")
def N():
    from dynamic_vocabulary_draft_amd import build, native  # noqa: F401
    return native


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(ds_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(N):
    decl = declared_functions()
    assert len(decl) >= 13
    lib = C.CDLL(N.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(N.SYMBOLS) == decl


def test_status_strings_and_version(N):
    assert "gfx950" in N.version()
    for code in range(6):
        assert N.lib.ds_status_string(code)
    assert N.lib.ds_status_string(99) == b"unknown status"


def test_workspace_queries(N):
    assert N.router_workspace_bytes(4, 1024) == 4 * 1024 * 4
    # 8 or more inputs: plus the first layer's partial sums, 32 windows x 64 inputs
    assert N.router_workspace_bytes(64, 1024) == 64 * 1024 * 4 + 32 * 64 * 1024 * 4
    assert N.router_workspace_bytes(0, 4) == 0
    nch = (262144 + 4095) // 4096
    assert N.build_workspace_bytes(64, 262144) == 256 + 64 * 8
    assert N.cluster_index_bytes(2048, 262144) == (nch + 1) * 2048 * 4
    assert N.sample_workspace_bytes(1, 1, 1024) == 24 + 256
    assert N.sample_workspace_bytes(3, 4, 1025) == 12 * 2 * 24 + 256
    assert N.softmax_workspace_bytes(7, 128256) == 7 * 32 * 12 + 256  # 4096-entry segments
    assert N.verify_workspace_bytes(2, 6, 128256) >= 2 * 126 * 8 + 2 * 16  # chunk sums, t*, row norms
    assert N.draft_chain_workspace_bytes(1, 6, 128256, 1024, 55734) >= 4096 + 256
    # batched chains: two 32-token tile-index slots (8 bytes per tile and row)
    tiles = (128256 + 31) // 32 + 1
    assert (N.draft_chain_workspace_bytes(32, 6, 128256, 1024, 55734)
            >= N.router_workspace_bytes(32, 1024) + 2 * 32 * tiles * 8)
    assert N.head_workspace_bytes(8, 64, 151936) == 0  # tree head: no workspace
    assert N.sample_workspace_bytes(0, 1, 10) == 0


FAKE = C.c_void_p(4096)  # aligned, never dereferenced: every call below fails validation


def test_router_rejects_bad_arguments(N):
    L = N.lib
    args = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("dt", N.BF16), ("n", 4), ("d", 64), ("r", 64), ("M", 8), ("act", N.SILU),
        ("h", FAKE), ("ldh", 64), ("W1", FAKE), ("b1", None), ("W2", FAKE), ("b2", None),
        ("scores", FAKE), ("ws", None), ("ws_bytes", 0)]]
    assert L.ds_router_score(*args(h=None)) == 1
    assert L.ds_router_score(*args(n=0)) == 1
    assert L.ds_router_score(*args(dt=7)) == 2
    assert L.ds_router_score(*args(act=9)) == 2
    assert L.ds_router_score(*args(d=60, ldh=60)) == 3
    assert L.ds_router_score(*args(ldh=32)) == 3
    assert L.ds_router_score(*args(h=C.c_void_p(4100))) == 1  # misaligned
    assert L.ds_router_score(*args()) == 1  # no workspace
    # 8 or more inputs also need the first layer's partial sums: a workspace
    # that holds only z is rejected before anything is enqueued
    assert L.ds_router_score(*args(n=8, ws=FAKE, ws_bytes=8 * 64 * 4)) == 1
    assert L.ds_router_score(*args(n=8, d=8200, ldh=8200, ws=FAKE, ws_bytes=1 << 30)) == 3


def test_select_build_head_sample_verify_reject_bad_arguments(N):
    L = N.lib
    assert L.ds_select_clusters(None, 2, 5000, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE) == 3
    assert L.ds_select_clusters(None, 2, 64, FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE) == 2
    assert L.ds_select_clusters(None, 0, 64, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE) == 1
    assert L.ds_select_clusters(None, 2, 64, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE) == 1
    bld = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("n", 2), ("M", 64), ("V", 1000), ("sel", FAKE), ("n_sel", FAKE),
        ("cluster_of", FAKE), ("index", FAKE), ("cap", 10), ("sl_off", FAKE), ("sl_ids", FAKE),
        ("flag", None), ("ws", FAKE), ("ws_bytes", 1 << 20)]]
    assert L.ds_build_shortlist(*bld(ws_bytes=0)) == 1  # workspace too small
    assert L.ds_build_shortlist(*bld(M=99999)) == 3
    assert L.ds_build_shortlist(*bld(cap=-1)) == 1
    assert L.ds_build_shortlist(*bld(index=None)) == 1
    assert L.ds_cluster_index(None, 64, 1000, None, FAKE, None) == 1
    assert L.ds_cluster_index(None, 5000, 1000, FAKE, FAKE, None) == 3
    assert L.ds_cluster_index(None, 0, 1000, FAKE, FAKE, None) == 1
    head = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("dt", N.BF16), ("V", 100), ("d", 64), ("W", FAKE), ("G", 2), ("m", 1),
        ("h", FAKE), ("ldh_g", 64), ("sl_off", FAKE), ("sl_ids", FAKE), ("max_rows", 10),
        ("logits", FAKE), ("ws", None), ("ws_bytes", 0)]]
    assert L.ds_gathered_lm_head(*head(W=None)) == 1
    assert L.ds_gathered_lm_head(*head(dt=5)) == 2
    assert L.ds_gathered_lm_head(*head(d=62, ldh_g=62)) == 3
    assert L.ds_gathered_lm_head(*head(m=2)) == 3  # ldh_g < m*d
    assert L.ds_gathered_lm_head(*head(m=300, ldh_g=300 * 64)) == 3
    assert L.ds_gathered_lm_head(*head(d=8200, ldh_g=8200)) == 3
    assert L.ds_gathered_lm_head(*head(dt=N.F32, d=4104, ldh_g=4104)) == 3
    assert L.ds_gathered_lm_head(*head(max_rows=-1)) == 1
    assert L.ds_gathered_lm_head(*head(G=16)) == 1  # union path needs its workspace
    assert N.head_workspace_bytes(16, 1, 100) > 0 and N.head_workspace_bytes(4, 1, 100) == 0
    smp = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("G", 2), ("m", 1), ("sl_off", FAKE), ("sl_ids", FAKE), ("logits", FAKE),
        ("tau", C.c_float(1.0)), ("u", FAKE), ("max_len", 100), ("token", FAKE), ("q", FAKE),
        ("ws", FAKE), ("ws_bytes", 0)]]
    assert L.ds_shortlist_sample(*smp(tau=C.c_float(-1.0))) == 1
    assert L.ds_shortlist_sample(*smp(tau=C.c_float(float("nan")))) == 1
    assert L.ds_shortlist_sample(*smp(G=0)) == 1
    assert L.ds_shortlist_sample(*smp(max_len=0)) == 1
    assert L.ds_shortlist_sample(*smp(max_len=(1 << 20) + 1)) == 3
    assert L.ds_shortlist_sample(*smp()) == 1  # workspace too small
    assert L.ds_target_softmax(None, 0, 10, FAKE, FAKE, FAKE, 1 << 20) == 1
    assert L.ds_target_softmax(None, 2, (1 << 20) + 4, FAKE, FAKE, FAKE, 1 << 30) == 3
    assert L.ds_target_softmax(None, 2, 1000, FAKE, FAKE, FAKE, 8) == 1
    ver = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("B", 2), ("T", 3), ("V", 100), ("draft", FAKE), ("sl_off", FAKE),
        ("sl_ids", FAKE), ("q", FAKE), ("p", FAKE), ("u_acc", FAKE), ("u_fin", FAKE),
        ("n_acc", FAKE), ("out", FAKE), ("ws", FAKE), ("ws_bytes", 0)]]
    assert L.ds_verify_reject(*ver(T=65)) == 3
    assert L.ds_verify_reject(*ver(V=(1 << 20) + 1)) == 3
    assert L.ds_verify_reject(*ver(draft=None)) == 1
    assert L.ds_verify_reject(*ver()) == 1  # workspace too small
    # the allocation-free variant: same checks, plus its scratch limit
    nver = lambda **kw: ver(**kw)[:-2]  # noqa: E731  (no workspace arguments)
    assert L.ds_verify_reject_noalloc(*nver(T=65)) == 3
    assert L.ds_verify_reject_noalloc(*nver(draft=None)) == 1
    assert L.ds_verify_reject_noalloc(*nver(B=0)) == 1
    assert L.ds_verify_reject_noalloc(*nver(B=1024, V=1 << 20)) == 3  # over the scratch
    assert N.verify_workspace_bytes(1024, 3, 1 << 20) > (8 << 20)
    assert N.verify_workspace_bytes(64, 5, 262144) <= (8 << 20)
    # verification from logits: the same checks, plus one statistics row per
    # target position
    assert L.ds_verify_reject_logits(*ver(T=65)) == 3
    assert L.ds_verify_reject_logits(*ver(p=None)) == 1
    assert L.ds_verify_reject_logits(*ver(B=2048, T=32, ws_bytes=1 << 40)) == 3
    assert L.ds_verify_reject_logits(*ver()) == 1  # workspace too small
    assert N.verify_logits_workspace_bytes(2, 3, 100) >= N.verify_workspace_bytes(2, 3, 100) + 8 * 12
    # tree verification from logits: argument and shape checks
    tv = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("B", 2), ("m", 3), ("V", 100), ("parent", FAKE), ("token", FAKE),
        ("sl_off", FAKE), ("sl_ids", FAKE), ("q", FAKE), ("logits", FAKE), ("u_acc", FAKE),
        ("u_fin", FAKE), ("max_len", 50), ("n_acc", FAKE), ("out", FAKE), ("path", FAKE),
        ("ws", FAKE), ("ws_bytes", 0)]]
    assert L.ds_verify_tree_logits(*tv(logits=None)) == 1
    assert L.ds_verify_tree_logits(*tv(m=0)) == 1
    assert L.ds_verify_tree_logits(*tv(B=2048, m=64, ws_bytes=1 << 40)) == 3  # B*(m+1) rows
    assert L.ds_verify_tree_logits(*tv()) == 1  # workspace too small
    assert (N.verify_tree_logits_workspace_bytes(2, 3, 100, 50)
            > N.verify_tree_workspace_bytes(2, 3, 100, 50))
    assert L.ds_draft_chain(None, None, None) == 1
    a = N.ChainArgs(B=0, T=6)
    assert L.ds_draft_chain(None, None, C.byref(a)) == 1


def test_row_statistics_entry_points_reject_bad_arguments(N):
    """The sampler and verifiers that take per-row draft statistics in place
    of q: a positive temperature and the statistics are required; the other
    checks are those of the q forms."""
    L = N.lib
    smp = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("G", 2), ("m", 1), ("sl_off", FAKE), ("sl_ids", FAKE), ("logits", FAKE),
        ("tau", C.c_float(1.0)), ("u", FAKE), ("max_len", 100), ("token", FAKE),
        ("qstats", FAKE), ("ws", FAKE), ("ws_bytes", 0)]]
    assert L.ds_shortlist_sample_stats(*smp(tau=C.c_float(0.0))) == 1  # argmax keeps q
    assert L.ds_shortlist_sample_stats(*smp(qstats=None)) == 1
    assert L.ds_shortlist_sample_stats(*smp(max_len=(1 << 20) + 1)) == 3
    assert L.ds_shortlist_sample_stats(*smp()) == 1  # workspace too small
    ver = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("B", 2), ("T", 3), ("V", 100), ("draft", FAKE), ("sl_off", FAKE),
        ("sl_ids", FAKE), ("dl", FAKE), ("qstats", FAKE), ("tau", C.c_float(1.0)),
        ("logits", FAKE), ("u_acc", FAKE), ("u_fin", FAKE), ("n_acc", FAKE), ("out", FAKE),
        ("ws", FAKE), ("ws_bytes", 0)]]
    assert L.ds_verify_reject_logits_qstats(*ver(qstats=None)) == 1
    assert L.ds_verify_reject_logits_qstats(*ver(tau=C.c_float(0.0))) == 1
    assert L.ds_verify_reject_logits_qstats(*ver(dl=None)) == 1
    assert L.ds_verify_reject_logits_qstats(*ver(T=65)) == 3
    assert L.ds_verify_reject_logits_qstats(*ver(B=2048, T=32, ws_bytes=1 << 40)) == 3
    assert L.ds_verify_reject_logits_qstats(*ver()) == 1  # workspace too small
    tv = lambda **kw: [kw.get(k, v) for k, v in [  # noqa: E731
        ("s", None), ("B", 2), ("m", 3), ("V", 100), ("parent", FAKE), ("token", FAKE),
        ("sl_off", FAKE), ("sl_ids", FAKE), ("dl", FAKE), ("qstats", FAKE),
        ("tau", C.c_float(1.0)), ("logits", FAKE), ("u_acc", FAKE), ("u_fin", FAKE),
        ("max_len", 50), ("n_acc", FAKE), ("out", FAKE), ("path", FAKE), ("ws", FAKE),
        ("ws_bytes", 0)]]
    assert L.ds_verify_tree_logits_qstats(*tv(qstats=None)) == 1
    assert L.ds_verify_tree_logits_qstats(*tv(tau=C.c_float(float("nan")))) == 1
    assert L.ds_verify_tree_logits_qstats(*tv(m=0)) == 1
    assert L.ds_verify_tree_logits_qstats(*tv(B=2048, m=64, ws_bytes=1 << 40)) == 3
    assert L.ds_verify_tree_logits_qstats(*tv()) == 1  # workspace too small
    assert C.sizeof(N.ChainArgs) == N.ChainArgs.qstats.offset + 8  # the last field


def test_draft_chain_requires_sync_events(N):
    """Arguments that pass every other check, with no stream-ordering
    events: rejected on the host before anything is enqueued."""
    L = N.lib
    T, B = 2, 1
    max_rows = (C.c_int64 * T)(1000, 1000)
    max_len = (C.c_int64 * T)(1000, 1000)
    f = FAKE.value
    a = N.ChainArgs(B=B, T=T, V=5000, d=64, r=64, M=16, dtype=N.BF16, act=N.SILU,
                    budget_kind=N.BUDGET_TOKENS, temperature=1.0, W=f, W1=f, b1=f, W2=f, b2=f,
                    cluster_of=f, cluster_index=f, cluster_size=f, h=f, budget=f, u_draft=f,
                    capacity=4000, max_rows=C.cast(max_rows, C.c_void_p),
                    max_len=C.cast(max_len, C.c_void_p), scores=f, sel=f, n_sel=f, sl_len=f,
                    sl_off=f, sl_ids=f, logits=f, q=f, token=f, err_flag=None, ws=f,
                    ws_bytes=1 << 30)
    assert L.ds_draft_chain(None, None, C.byref(a)) == 1
    a.q = None  # no q: the row statistics are then required, with temperature > 0
    ev_ok = (C.c_void_p * (2 * T + 1))(*([f] * (2 * T + 1)))
    a.sync_events = C.cast(ev_ok, C.c_void_p)
    assert L.ds_draft_chain(None, None, C.byref(a)) == 1
    a.qstats, a.temperature = f, 0.0
    assert L.ds_draft_chain(None, None, C.byref(a)) == 1
    a.q, a.qstats, a.temperature, a.sync_events = f, None, 1.0, None
    ev = (C.c_void_p * (2 * T + 1))(*([f] * (2 * T)), None)  # one handle missing
    a.sync_events = C.cast(ev, C.c_void_p)
    assert L.ds_draft_chain(None, None, C.byref(a)) == 1
    assert L.ds_capture_begin(None) == 1
    assert L.ds_capture_end(None, None) == 1
    assert L.ds_graph_launch(None, None) == 1
    assert L.ds_graph_destroy(None) == 1


# ----------------------------------------------------------------------------
# host logic
# ----------------------------------------------------------------------------
def test_generator_is_deterministic_and_shaped():
    a = syn.make_workload(0)
    b = syn.make_workload(0)
    for k in ("W", "h", "u_draft", "u_acc", "u_fin", "cluster_of", "target_logits"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    c = syn.make_workload(0, instance=1)
    assert not np.array_equal(a.h, c.h)
    assert np.array_equal(a.W, c.W)
    assert a.h.shape == (1, 5, 256) and a.W.shape == (8192, 256)
    assert (a.u_draft * 2 ** 24 == np.round(a.u_draft * 2 ** 24)).all()
    assert ((a.u_draft >= 0) & (a.u_draft < 1)).all()


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [0.0, -0.0, 1e-40, 3.4e38]
    ours = syn.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(syn.bf16_bits_to_f32(ours),
                          torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("index", [1, 3, 4])
def test_zipf_clusters_partition_vocabulary(index):
    cfg = syn.CONFIGS[index]
    cluster_of, size = syn.make_clusters(cfg)
    assert size.sum() == cfg.V and size.min() >= 1
    assert np.array_equal(np.bincount(cluster_of, minlength=cfg.M), size)
    assert (np.diff(size) <= 0).all()  # ranks ordered by size


def test_budget_schedules():
    assert syn.CONFIGS[1].budget == (32768, 29491, 26214, 22938, 19661, 16384)
    assert syn.CONFIGS[4].budget == (49152, 43008, 36864, 30720, 24576)
    assert syn.linear_budget(5, 5, 1) == (5,)


@pytest.mark.parametrize("index", [0, 1, 4])
def test_capacity_bounds_cover_every_selection(oracle_lib, index):
    from dynamic_vocabulary_draft_amd.pipeline import shortlist_bounds
    cfg = syn.CONFIGS[index]
    cluster_of, size = syn.make_clusters(cfg)
    bounds = shortlist_bounds(cfg, size)
    g = np.random.default_rng(index)
    for t, b in enumerate(cfg.budget):
        s = g.standard_normal((50, cfg.M)).astype(np.float32)
        _, _, L = oracle_lib.select_clusters(s, size, cfg.budget_kind, np.full(50, b, np.int32))
        assert L.max() * cfg.B <= bounds[t]


def test_traffic_from_scales_counters(tmp_path):
    """bench.py --traffic-from: per-dispatch FETCH_SIZE / WRITE_SIZE of the
    head kernel, scaled by what the same counter reads for the probe's plain
    copy of known size, averaged per launch and set against the algorithmic
    bytes the probe recorded."""
    import json
    import subprocess
    import sys
    copy = 1 << 30

    def csv(d, counter, head_kib, copy_kib):
        d.mkdir()
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        for i, v in enumerate(head_kib):
            rows.append('%d,"void ds::head_gemv_kernel<true, 8, 2>(int)",%s,%r' % (i + 1, counter, v))
        rows.append('%d,"__amd_rocclr_copyBuffer",%s,%r' % (len(head_kib) + 1, counter, copy_kib))
        (d / "p_counter_collection.csv").write_text("\n".join(rows) + "\n")

    csv(tmp_path / "fetch", "FETCH_SIZE", [1000.0, 1200.0], copy / 2 / 1024)  # reads half
    csv(tmp_path / "write", "WRITE_SIZE", [10.0, 20.0], copy / 1024)
    probe = tmp_path / "probe.json"
    probe.write_text(json.dumps({"workload": "w", "head_kernel": "head_gemv_kernel",
                                 "launch_bytes": [2.0e6, 2.4e6], "copy_bytes": copy,
                                 "kernel_source_sha256": "x"}))
    out = tmp_path / "traffic.json"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-from",
                        str(tmp_path / "fetch"), str(tmp_path / "write"), "--probe-file",
                        str(probe), "--traffic-out", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    t = json.loads(out.read_text())
    assert t["fetch_bytes_per_launch"] == 1100 * 1024 * 2
    assert t["write_bytes_per_launch"] == 15 * 1024
    assert t["bytes_per_launch"] == 1100 * 1024 * 2 + 15 * 1024
    assert t["algorithmic_bytes_per_launch"] == 2200000
    assert t["traffic_over_algorithmic"] == round((1100 * 1024 * 2 + 15 * 1024) / 2.2e6, 4)
    assert t["launches"] == 2 and t["workload"] == "w"


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_committed_traffic_matches_head_sources(config):
    """Each full-size workload's committed head traffic counters were taken
    from the current sources of its head kernel, so the bench line reports
    `roofline.traffic` for it (bench.py drops it when the hash, the kernel or
    the workload differs).  An edit to those sources needs new counters."""
    import json
    import sys
    sys.path.insert(0, ROOT)
    import bench
    cfg = syn.CONFIGS[config]
    kernel = bench.head_kernel_name(cfg)
    with open(bench.traffic_file(cfg.name)) as f:
        t = json.load(f)
    assert t["kernel_source_sha256"] == bench.head_source_sha(kernel), \
        "head sources changed since the traffic counters were taken"
    assert t["workload"] == cfg.name and t["head_kernel"] == kernel
    # the GEMV and union heads read each needed row once; the tree head
    # re-reads some rows shared by several trees (1.24x when measured)
    assert 1.0 <= t["traffic_over_algorithmic"] < (1.3 if cfg.is_tree else 1.05)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it says so and exits
    non-zero before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
