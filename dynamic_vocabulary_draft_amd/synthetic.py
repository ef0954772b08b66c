"""Seeded synthetic workloads for the shortlisted draft head.

This module only draws random inputs; it holds none of the method's
arithmetic, so that both the HIP path and the CPU oracle can consume the very
same bytes.  Every array comes from ``numpy.random.default_rng([SEED, cfg,
stream, ...])`` with the stream numbers below; bf16 values are fp32 draws
rounded to nearest-even and stored as their raw 16-bit patterns (uint16).

Streams: 0 centroids, 1 noise (one sub-stream per block of ``ROW_BLOCK`` rows),
2 token permutation, 3-6 router W1/b1/W2/b2, 7 hidden states (sub-stream =
instance), 8 target logits, 9 draft uniforms, 10 accept uniforms, 11 final
uniforms (9-11 also take the instance), 12 token frequency ranking (the
order a fixed, frequency-ranked shortlist takes tokens in), 13 initial
k-means labels, 14 router-training hidden states (sub-stream = instance).

The workload shapes stand in for the pages' Llama-3-8B, Qwen3-8B and
Gemma-3-12B drafting set-ups (DynaSpec summary page, "Evaluation Setup" and
"Key Results"): only V, d, the shortlist budgets (about 28K dynamic versus
32K static tokens) and the batch/tree shapes are taken; no benchmark item is
used or needed.  Trained weights are not available, so the LM head is a
clustered Gaussian: W[y] = c[cluster(y)] + eps_y, which gives the head the
cluster structure that the spherical k-means of the method would find.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 20251011  # the arXiv first-post date of DynaSpec (11 Oct 2025)
ROW_BLOCK = 4096  # W rows per noise sub-stream (lets generation run in threads)
U_BITS = 24  # uniforms are k * 2**-24, exact in fp32 and fp64

ACT_RELU, ACT_SILU = 0, 1
BUDGET_CLUSTERS, BUDGET_TOKENS = 0, 1
DT_F32, DT_BF16 = 0, 1


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload (shapes, distributions, budgets)."""

    index: int
    name: str
    V: int
    d: int
    M: int
    r: int
    act: int
    dtype: int
    B: int  # sequences
    T: int  # draft positions per sequence (tree configs: 1 router row)
    budget_kind: int
    budget: tuple  # per position
    contiguous_clusters: bool  # True: M runs of V/M tokens; False: Zipf sizes
    zipf_s: float = 1.1
    tree_nodes: int = 1  # head rows per group sharing one shortlist
    centroid_std: float = 0.05
    noise_std: float = 0.02
    target_std: float = 3.0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == DT_BF16 else 4

    @property
    def is_tree(self) -> bool:
        return self.tree_nodes > 1

    @property
    def n_head_rows(self) -> int:
        """Head rows per position-call: B groups of tree_nodes rows each."""
        return self.B * self.tree_nodes


def linear_budget(b0: int, b1: int, T: int) -> tuple:
    """Budget decaying linearly from b0 (first position) to b1 (last one),
    rounded half away from zero."""
    if T == 1:
        return (int(b0),)
    out = []
    for t in range(T):
        x = b0 + (b1 - b0) * t / (T - 1)
        out.append(int(math.floor(abs(x) + 0.5)) * (1 if x >= 0 else -1))
    return tuple(out)


CONFIGS = {
    0: Config(0, "tiny-fp32 V=8192 d=256 M=64", 8192, 256, 64, 256, ACT_RELU,
              DT_F32, 1, 4, BUDGET_CLUSTERS, (8, 6, 4, 4), True),
    1: Config(1, "llama3-8b-shaped V=128256 d=4096 bf16 b1 depth6", 128256,
              4096, 1024, 1024, ACT_SILU, DT_BF16, 1, 6, BUDGET_TOKENS,
              linear_budget(32768, 16384, 6), False),
    2: Config(2, "llama3-8b-shaped V=128256 d=4096 bf16 b32 depth6", 128256,
              4096, 1024, 1024, ACT_SILU, DT_BF16, 32, 6, BUDGET_TOKENS,
              linear_budget(32768, 16384, 6), False),
    3: Config(3, "qwen3-8b-shaped tree V=151936 d=4096 bf16 8x64 nodes",
              151936, 4096, 1024, 1024, ACT_SILU, DT_BF16, 8, 1,
              BUDGET_TOKENS, (24576,), False, tree_nodes=64),
    4: Config(4, "gemma3-12b-shaped V=262144 d=3840 bf16 b64 depth5", 262144,
              3840, 2048, 1024, ACT_SILU, DT_BF16, 64, 5, BUDGET_TOKENS,
              linear_budget(49152, 24576, 5), False),
}


def rng(cfg: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng([SEED, cfg, *stream])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == DT_BF16 else np.ascontiguousarray(x, np.float32)


def zipf_cluster_sizes(V: int, M: int, s: float) -> np.ndarray:
    """Cluster sizes proportional to (k+1)^-s, rounded by largest remainder so
    they sum to V exactly (ties in the fractional part go to the lower k)."""
    w = np.arange(1, M + 1, dtype=np.float64) ** (-s)
    raw = V * w / w.sum()
    base = np.floor(raw).astype(np.int64)
    rem = V - int(base.sum())
    frac = raw - base
    order = sorted(range(M), key=lambda k: (-frac[k], k))
    for k in order[:rem]:
        base[k] += 1
    if (base < 1).any():
        raise ValueError("a Zipf cluster came out empty; lower M or s")
    return base.astype(np.int32)


def make_clusters(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Returns (cluster_of[V] int32, cluster_size[M] int32)."""
    if cfg.contiguous_clusters:
        size = np.full(cfg.M, cfg.V // cfg.M, dtype=np.int32)
        assert int(size.sum()) == cfg.V
        cluster_of = (np.arange(cfg.V) // (cfg.V // cfg.M)).astype(np.int32)
        return cluster_of, size
    size = zipf_cluster_sizes(cfg.V, cfg.M, cfg.zipf_s)
    perm = rng(cfg.index, 2).permutation(cfg.V)
    cluster_of = np.empty(cfg.V, dtype=np.int32)
    cluster_of[perm] = np.repeat(np.arange(cfg.M, dtype=np.int32), size)
    return cluster_of, size


def make_lm_head(cfg: Config, cluster_of: np.ndarray, threads: int = 8) -> np.ndarray:
    """W[V][d] = centroid[cluster_of[y]] + noise, in the config's dtype."""
    cent = rng(cfg.index, 0).standard_normal((cfg.M, cfg.d), dtype=np.float32)
    cent *= np.float32(cfg.centroid_std)
    out = np.empty((cfg.V, cfg.d), dtype=np.uint16 if cfg.dtype == DT_BF16 else np.float32)

    def block(bi: int) -> None:
        lo, hi = bi * ROW_BLOCK, min(cfg.V, (bi + 1) * ROW_BLOCK)
        x = rng(cfg.index, 1, bi).standard_normal((hi - lo, cfg.d), dtype=np.float32)
        x *= np.float32(cfg.noise_std)
        x += cent[cluster_of[lo:hi]]
        out[lo:hi] = _store(x, cfg.dtype)

    nblk = (cfg.V + ROW_BLOCK - 1) // ROW_BLOCK
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(block, range(nblk)))
    return out


def make_router(cfg: Config) -> dict:
    """Two-layer router weights: W1 ~ N(0, d^-1/2), W2 ~ N(0, r^-1/2),
    biases ~ N(0, 0.02) (second argument = standard deviation)."""
    W1 = rng(cfg.index, 3).standard_normal((cfg.r, cfg.d), dtype=np.float32) * np.float32(cfg.d ** -0.5)
    b1 = rng(cfg.index, 4).standard_normal(cfg.r, dtype=np.float32) * np.float32(0.02)
    W2 = rng(cfg.index, 5).standard_normal((cfg.M, cfg.r), dtype=np.float32) * np.float32(cfg.r ** -0.5)
    b2 = rng(cfg.index, 6).standard_normal(cfg.M, dtype=np.float32) * np.float32(0.02)
    return {k: _store(v, cfg.dtype) for k, v in dict(W1=W1, b1=b1, W2=W2, b2=b2).items()}


def make_hidden(cfg: Config, instance: int = 0) -> np.ndarray:
    """Hidden states h[B][T+1][d] (chains: router reads index t, head t+1) or
    h[B][1+nodes][d] (trees: router reads index 0, head rows 1..nodes)."""
    rows = (1 + cfg.tree_nodes) if cfg.is_tree else (cfg.T + 1)
    h = rng(cfg.index, 7, instance).standard_normal((cfg.B, rows, cfg.d), dtype=np.float32)
    return _store(h, cfg.dtype)


def make_train_hidden(cfg: Config, n: int, instance: int = 0) -> np.ndarray:
    """n router-training inputs h ~ N(0, 1), [n][d] in the config's dtype
    (drafter hidden states; the pages train on the drafter's states of
    ShareGPT/UltraChat prompts, which are not available)."""
    g = rng(cfg.index, 14, instance)
    return _store(g.standard_normal((n, cfg.d), dtype=np.float32), cfg.dtype)


def frequency_rank(cfg: Config) -> np.ndarray:
    """Token ids from most to least frequent.  There is no corpus here, so a
    seeded permutation of [0, V) stands in for the ranking a static
    baseline would count (its head and sampling costs depend only on the
    list's size and scatter, not on which tokens it holds)."""
    return rng(cfg.index, 12).permutation(cfg.V).astype(np.int32)


def static_shortlist(cfg: Config, size: int) -> np.ndarray:
    """The ``size`` most frequent tokens in ascending id: the fixed list of
    a frequency-ranked static baseline."""
    return np.sort(frequency_rank(cfg)[: min(int(size), cfg.V)]).astype(np.int32)


def kmeans_init_assign(cfg: Config, cluster_of: np.ndarray, noise: float) -> np.ndarray:
    """Initial labels for the clustering: the planted cluster of each row,
    with a fraction ``noise`` of rows given a seeded uniformly random label
    instead (noise = 1 is a random partition)."""
    g = rng(cfg.index, 13)
    lab = np.asarray(cluster_of, np.int32).copy()
    flip = g.random(cfg.V) < noise
    lab[flip] = g.integers(0, cfg.M, size=int(flip.sum()), dtype=np.int32)
    return lab


def make_uniforms(cfg: Config, stream: int, shape, instance: int = 0) -> np.ndarray:
    k = rng(cfg.index, stream, instance).integers(0, 1 << U_BITS, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -U_BITS).astype(np.float32)


def target_rows(cfg: Config) -> int:
    """Target distributions per sequence: one per drafted position plus the
    bonus position (chains), one per tree node including the root (trees)."""
    return cfg.tree_nodes + 1 if cfg.is_tree else cfg.T + 1


def make_target_logits(cfg: Config, instance: int = 0) -> np.ndarray:
    """Full-vocabulary target logits N(0, 3) of shape [B][rows][V] (fp32)."""
    g = rng(cfg.index, 8, instance)
    rows = target_rows(cfg)
    out = np.empty((cfg.B, rows, cfg.V), dtype=np.float32)
    for b in range(cfg.B):
        out[b] = g.standard_normal((rows, cfg.V), dtype=np.float32) * np.float32(cfg.target_std)
    return out


def tree_parent(cfg: Config) -> np.ndarray:
    """Tree shape [B][m]: entry i-1 is the parent of drafted node i.  The
    tree workload fixes 64 nodes per tree but no shape; a complete binary
    tree in heap order (parent of node i is (i-1) // 2, depth 6 for 64
    nodes) is taken, the same for every sequence.  No random draw."""
    i = np.arange(1, cfg.tree_nodes + 1, dtype=np.int64)
    return np.tile(((i - 1) // 2).astype(np.int32), (cfg.B, 1))


def budget_rows(cfg: Config) -> np.ndarray:
    """budget[T][B]: every sequence at position t gets the schedule's value."""
    return np.repeat(np.asarray(cfg.budget, dtype=np.int32)[:, None], cfg.B, axis=1)


@dataclasses.dataclass
class Workload:
    cfg: Config
    W: np.ndarray
    cluster_of: np.ndarray
    cluster_size: np.ndarray
    router: dict
    h: np.ndarray
    budget: np.ndarray  # [T][B]
    u_draft: np.ndarray  # chains [T][B]; trees [B][nodes]
    u_acc: np.ndarray  # chains [T][B]; trees [B][nodes]
    u_fin: np.ndarray  # [B]
    target_logits: np.ndarray | None  # [B][target_rows][V]
    parent: np.ndarray | None = None  # trees: [B][nodes]


def make_workload(index: int, instance: int = 0, with_W: bool = True,
                  with_target: bool = True, threads: int = 8,
                  cfg: Config | None = None) -> Workload:
    cfg = cfg or CONFIGS[index]
    cluster_of, cluster_size = make_clusters(cfg)
    W = make_lm_head(cfg, cluster_of, threads) if with_W else None
    udraft_shape = (cfg.B, cfg.tree_nodes) if cfg.is_tree else (cfg.T, cfg.B)
    return Workload(
        cfg=cfg, W=W, cluster_of=cluster_of, cluster_size=cluster_size,
        router=make_router(cfg), h=make_hidden(cfg, instance),
        budget=budget_rows(cfg),
        u_draft=make_uniforms(cfg, 9, udraft_shape, instance),
        u_acc=make_uniforms(cfg, 10, udraft_shape, instance),
        u_fin=make_uniforms(cfg, 11, (cfg.B,), instance),
        target_logits=make_target_logits(cfg, instance) if with_target else None,
        parent=tree_parent(cfg) if cfg.is_tree else None,
    )


def shrink(cfg: Config, **kw) -> Config:
    """A copy of a config with some fields replaced (used for small test cases)."""
    return dataclasses.replace(cfg, **kw)
