"""Seeded synthetic inputs for sparse prefill attention (shared by tests and bench).

This module generates inputs only.  It holds none of the attention method's
arithmetic: no softmax, no estimate, no selection, no index building.  Both
the HIP path (through the Python binding) and the CPU oracle consume the
arrays it returns, so neither side ever produces the other's inputs.

The workloads stand in for one layer of post-RoPE activations of an 8B
long-context model (LLaMA-3-8B-1M head shapes: 32 query heads, 8 key/value
heads, head dim 128), which the MInference pages evaluate on long prompts
(arXiv 2407.02490 abstract).  Weights and prompts are not available, so the
activations are standard-normal draws with rotary embeddings applied and a
planted structure (hot key positions, hot key blocks) of the kind each
attention pattern looks for.

Recipe (every array is a pure function of its config and seed):
  * stream for (config seed s, tensor t, head h):
        numpy PCG64(SeedSequence([s, t, h])), t = 0 Q, 1 K, 2 V, 3 plants,
        4 per-head pattern assignment;
  * Q, K, V rows: standard_normal((N, d), float32), upcast to float64;
  * rotary embedding (rotate-half form, base 10000, positions 0..N-1) on Q
    and K in float64;
  * plant: m_g = mean of post-rotary Q over the g query heads of a kv group
    and all N positions; K[j] += alpha * m_g for each planted key j;
  * local bias (the clustered-slash variant only): after the rotary
    embedding, alpha_local * v_i is added to Q row i and to K row i, with
    v_i = (cos(w_r i + p_r), sin(w_r i + p_r))_{r < d/2} / sqrt(d/2),
    w_r = (pi / local_span) (r + 1/2) / (d/2) and phases p_r drawn per kv
    group (stream t = 3, head 2000 + g); then v_i . v_j = mean_r
    cos(w_r (i - j)), a term that depends on the offset i - j only, peaks on
    the diagonal and falls to zero at offset local_span (a sinc-shaped main
    lobe), so the selected slash lines cluster at small offsets as in local
    attention;
  * a single rounding to the storage dtype (fp32, or bf16 by
    round-to-nearest-even), after which the arrays are exact in both the
    GPU's storage format and the oracle's float64.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

T_Q, T_K, T_V, T_PLANT, T_PATTERN = 0, 1, 2, 3, 4

# Pattern codes; the same numbering is used by the C ABI.
ASHAPE, VSLASH, BSPARSE, DENSE, VSLASH_EXACT = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    patterns: str  # "vs", "bs", "mixed", "ashape", "dense"
    alpha_vertical: float = 0.0
    n_vertical_plants: int = 0
    alpha_block: float = 0.0
    alpha_local: float = 0.0
    local_span: int = 8192
    n_hot_blocks: int = 0
    last_q: int = 64
    n_vertical: int = 1000
    n_slash: int = 6096
    top_blocks: int = 100
    sink: int = 128
    local: int = 4096
    force_vertical: int = 1
    force_slash: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def n_blocks(self) -> int:
        return self.seq_len // 64

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Sizes are those of the evaluation shapes; smaller
# variants for tests are made with Workload.with_(seq_len=..., ...).
C1 = Workload("vs_1h_2k_f32", 1001, 1, 1, 1, 2048, 64, "f32", "vs",
              alpha_vertical=3.0, n_vertical_plants=8,
              last_q=64, n_vertical=64, n_slash=128)
C2 = Workload("bs_gqa_32k_bf16", 1002, 1, 32, 8, 32768, 128, "bf16", "bs",
              alpha_block=2.0, n_hot_blocks=16, top_blocks=100)
C3 = Workload("vs_llama8b_128k_bf16", 1003, 1, 32, 8, 131072, 128, "bf16", "vs",
              alpha_vertical=3.0, n_vertical_plants=64,
              last_q=64, n_vertical=1000, n_slash=6096)
C4 = Workload("mixed_256k_bf16", 1004, 1, 32, 8, 262144, 128, "bf16", "mixed",
              alpha_vertical=3.0, n_vertical_plants=64,
              alpha_block=2.0, n_hot_blocks=16,
              last_q=64, n_vertical=1000, n_slash=6096, top_blocks=100,
              sink=128, local=4096)
C5 = Workload("vs_llama8b_1m_bf16", 1005, 1, 32, 8, 1048576, 128, "bf16", "vs",
              alpha_vertical=3.0, n_vertical_plants=64,
              last_q=64, n_vertical=1000, n_slash=6096)

# Clustered-slash variant of the 128K Vertical-Slash layer (not one of the five
# evaluation shapes): the same shapes and budgets with the local bias, so that
# the selected slash offsets cluster near the diagonal.
C3_LOCAL = C3.with_(name="vs_local_128k_bf16", seed=1013, alpha_local=16.0, local_span=8192)

WORKLOADS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5, "c3local": C3_LOCAL}


def rng(seed: int, tensor: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, head])))


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    out = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rotary_tables(n: int, d: int):
    half = d // 2
    inv = 10000.0 ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    half = x.shape[-1] // 2
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=1)


def head_patterns(w: Workload) -> np.ndarray:
    """Per-query-head pattern codes [Hq] (int32)."""
    if w.patterns == "vs":
        return np.full(w.heads_q, VSLASH, np.int32)
    if w.patterns == "bs":
        return np.full(w.heads_q, BSPARSE, np.int32)
    if w.patterns == "ashape":
        return np.full(w.heads_q, ASHAPE, np.int32)
    if w.patterns == "dense":
        return np.full(w.heads_q, DENSE, np.int32)
    if w.patterns == "mixed":
        # 1/4 A-shape, 1/2 Vertical-Slash, 1/4 Block-Sparse, by a seeded permutation.
        perm = rng(w.seed, T_PATTERN, 0).permutation(w.heads_q)
        out = np.empty(w.heads_q, np.int32)
        na = w.heads_q // 4
        nv = w.heads_q // 2
        out[perm[:na]] = ASHAPE
        out[perm[na:na + nv]] = VSLASH
        out[perm[na + nv:]] = BSPARSE
        return out
    raise ValueError(w.patterns)


def vertical_plants(w: Workload, kvh: int) -> np.ndarray:
    """Planted vertical key positions of one kv head: {0} plus distinct draws on [1, N)."""
    if w.n_vertical_plants <= 0:
        return np.zeros(0, np.int64)
    g = rng(w.seed, T_PLANT, kvh)
    others = g.choice(np.arange(1, w.seq_len), size=w.n_vertical_plants - 1, replace=False)
    return np.sort(np.concatenate([[0], others]).astype(np.int64))


def hot_blocks(w: Workload, kvh: int) -> np.ndarray:
    """Planted hot 64-token key blocks of one kv head: distinct draws on [1, nb)."""
    if w.n_hot_blocks <= 0:
        return np.zeros(0, np.int64)
    g = rng(w.seed, T_PLANT, 1000 + kvh)
    nb = w.n_blocks
    n = min(w.n_hot_blocks, nb - 1)
    return np.sort(g.choice(np.arange(1, nb), size=n, replace=False).astype(np.int64))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return round_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload, with_v: bool = True):
    """Returns dict(q, k, v, patterns, plants, hot) for batch index 0..B-1.

    q: [B, Hq, N, d], k, v: [B, Hkv, N, d] in the storage format: float32, or
    uint16 bf16 bit patterns.  Batch b uses seed + 7919*b.
    """
    B, Hq, Hkv, N, d = w.batch, w.heads_q, w.heads_kv, w.seq_len, w.head_dim
    sdt = np.float32 if w.dtype == "f32" else np.uint16
    q = np.empty((B, Hq, N, d), sdt)
    k = np.empty((B, Hkv, N, d), sdt)
    v = np.empty((B, Hkv, N, d), sdt) if with_v else None
    cos, sin = _rotary_tables(N, d)
    g = w.group
    plants = {kvh: vertical_plants(w, kvh) for kvh in range(Hkv)}
    hot = {kvh: hot_blocks(w, kvh) for kvh in range(Hkv)}

    def one_kv_group(b: int, kvh: int):
        seed = w.seed + 7919 * b
        qsum = np.zeros(d, np.float64)
        loc = None
        if w.alpha_local:
            half = d // 2
            ph = rng(w.seed, T_PLANT, 2000 + kvh).uniform(0.0, 2.0 * np.pi, half)
            om = (np.pi / w.local_span) * (np.arange(half) + 0.5) / half
            ang = np.arange(N, dtype=np.float64)[:, None] * om[None, :] + ph[None, :]
            loc = w.alpha_local * np.concatenate([np.cos(ang), np.sin(ang)], axis=1) / np.sqrt(half)
            del ang
        for hq in range(kvh * g, (kvh + 1) * g):
            qh = rng(seed, T_Q, hq).standard_normal((N, d), dtype=np.float32).astype(np.float64)
            qh = _rotate(qh, cos, sin)
            if loc is not None:
                qh += loc
            qsum += qh.sum(axis=0)
            q[b, hq] = _store(qh, w.dtype)
            del qh
        m_g = qsum / (g * N)
        kh = rng(seed, T_K, kvh).standard_normal((N, d), dtype=np.float32).astype(np.float64)
        kh = _rotate(kh, cos, sin)
        if loc is not None:
            kh += loc
        if w.alpha_vertical and len(plants[kvh]):
            kh[plants[kvh]] += w.alpha_vertical * m_g
        if w.alpha_block and len(hot[kvh]):
            rows = (hot[kvh][:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
            kh[rows] += w.alpha_block * m_g
        k[b, kvh] = _store(kh, w.dtype)
        del kh
        if with_v:
            vh = rng(seed, T_V, kvh).standard_normal((N, d), dtype=np.float32)
            v[b, kvh] = _store(vh, w.dtype)

    jobs = [(b, kvh) for b in range(B) for kvh in range(Hkv)]
    if len(jobs) == 1 or N * d < (1 << 16):
        for j in jobs:
            one_kv_group(*j)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(lambda j: one_kv_group(*j), jobs))
    return dict(q=q, k=k, v=v, patterns=head_patterns(w), plants=plants, hot=hot)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored array to float64."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    return bf16_bits_to_f32(x).astype(np.float64)


def random_qkv(seed: int, heads_q: int, heads_kv: int, n: int, d: int, dtype: str = "f32",
               batch: int = 1, scale_std: float = 1.0):
    """Plain seeded N(0, scale_std^2) Q, K, V (no rotary, no plants) for small tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    q = g.standard_normal((batch, heads_q, n, d)) * scale_std
    k = g.standard_normal((batch, heads_kv, n, d)) * scale_std
    v = g.standard_normal((batch, heads_kv, n, d))
    return _store(q, dtype), _store(k, dtype), _store(v, dtype)
