"""Seeded synthetic inputs for the CSA2 FP4 sparse-decode path.

This module only draws random numbers and lays them out. It holds none of
the method's arithmetic (no compression, quantisation, scoring, selection or
attention); both the CPU oracle and the HIP library consume what it returns.

Every array is drawn from its own stream, keyed by (seed, stream id, ...),
so one sequence's inputs can be regenerated without drawing the others.
That lets parity tests at full size re-create a sample of sequences on the
host while the device holds the whole batch.

Shapes follow the workloads the pages describe: a 576-number MLA entry
(512 latent + 64 RoPE) per cache row [P2 "突破二：MLA，低秩压缩"], a sliding
window of the last 128 tokens and Top-512 sparse selection
[P2 "突破四：滑动窗口和稀疏注意力"], 2 tokens compressed into 1 entry
[same section], group sizes 32/64/128 [P1 §4.3], and long-context decode
at 64K-1M tokens [P2 "KV Cache 到底有多大"].

Sources cited as [P1]/[P2]/[P3]:
  P1  "DeepSeek V4.1 Flash KV Cache压缩实战：FP4+CSA2+CED将显存降至1/4"
  P2  "DeepSeek V1 到 V4.1-Flash，单 token 的 global KV 如何从 389,000 B 压缩到 890 B的？"
  P3  "KV Cache 瘦身 437 倍：DeepSeek V4.1-Flash 的推理效率革命"
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DIM = 576          # 512 latent + 64 RoPE dims per entry
ROPE = 64
VDIM = DIM - ROPE  # value dims
TOPK = 512
SWA_W = 128

# stream ids
S_ENTRIES = 1
S_IDXKEY = 2
S_WCOMP = 3
S_TOKENS = 4
S_STEP = 5
S_Q = 6
S_QIDX = 7
S_SWA = 8
S_LENGTHS = 9
S_HEADW = 10


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(s) for s in stream]]))


# ---------------------------------------------------------------- value laws

def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def student_t3(g: np.random.Generator, shape) -> np.ndarray:
    """Unscaled Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3)."""
    z = g.standard_normal(size=shape, dtype=np.float32)
    chi2 = np.float32(2.0) * g.standard_gamma(1.5, size=shape, dtype=np.float32)
    np.maximum(chi2, np.float32(1e-30), out=chi2)
    return (z / np.sqrt(chi2 / np.float32(3.0))).astype(np.float32)


def normal_outliers(g: np.random.Generator, shape, p: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """N(0,1) where each element is independently scaled by `factor` with probability p."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    hit = g.random(size=shape, dtype=np.float32) < np.float32(p)
    x[hit] *= np.float32(factor)
    return x


def int_bf16(g: np.random.Generator, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers uniform on {lo..hi} inclusive, returned as bf16 bit patterns (uint16).

    Small integers are exact in bf16, so the bit pattern is the top half of the
    float32 pattern."""
    v = g.integers(lo, hi + 1, size=shape, dtype=np.int32).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def normal_bf16_trunc(g: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) samples truncated toward zero to bf16 (uint16 bit patterns).

    Used for window rows that are already resident in the cache; the rows a
    step appends go through the library's own fp32->bf16 conversion instead."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- configs

@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  Sizes are per sequence unless stated."""
    name: str
    seed: int
    batch: int
    k_group: int
    v_group: int            # 0: values are read from the key plane
    idx_heads: int
    idx_dim: int
    q_heads: int
    entries: Optional[int]  # fixed compressed entries per sequence (None: ragged / prefill)
    entry_law: str          # "normal" | "t3" | "outliers"
    prefill_tokens: Optional[int] = None   # built through the compressor instead of entries
    ragged_tokens: Optional[tuple] = None  # (lo, hi) tokens per sequence, uniform
    chunk_tokens: int = 0                  # mixed step: prefill chunk appended to sequence 0
    layers: tuple = ("full",)              # CSA2 layer modes of one group step
    topk: int = TOPK
    window: int = SWA_W
    dim: int = DIM
    rope_dim: int = ROPE

    @property
    def vdim(self) -> int:
        return self.dim - self.rope_dim


WORKLOADS = {
    # T=4096 tokens -> 2048 entries via the stand-in compressor, one sequence.
    "tiny_t4096": Workload("tiny_t4096", seed=0, batch=1, k_group=32, v_group=0, idx_heads=4,
                           idx_dim=64, q_heads=16, entries=None, entry_law="normal",
                           prefill_tokens=4095),
    # 32 sequences x 64K tokens (32,768 entries), group 64, Student-t(3) cache values.
    "decode_64k_b32": Workload("decode_64k_b32", seed=1, batch=32, k_group=64, v_group=0,
                               idx_heads=64, idx_dim=128, q_heads=64, entries=32768,
                               entry_law="t3"),
    # one sequence of 1M tokens (500,000 entries), group 32.
    "decode_1m_b1": Workload("decode_1m_b1", seed=2, batch=1, k_group=32, v_group=0,
                             idx_heads=64, idx_dim=128, q_heads=64, entries=500000,
                             entry_law="normal"),
    # one CSA2 layer group: Full + Reindex + 3 Reuse on a shared 128K cache, batch 64.
    "group_128k_b64": Workload("group_128k_b64", seed=3, batch=64, k_group=64, v_group=0,
                               idx_heads=64, idx_dim=128, q_heads=64, entries=65536,
                               entry_law="normal",
                               layers=("full", "reindex", "reuse", "reuse", "reuse")),
    # 256 ragged sequences (2K-32K tokens), K plane g32 + V plane g128, 16K-token chunk.
    "mixed_ragged_b256": Workload("mixed_ragged_b256", seed=4, batch=256, k_group=32, v_group=128,
                                  idx_heads=64, idx_dim=128, q_heads=64, entries=None,
                                  entry_law="outliers", ragged_tokens=(2048, 32768),
                                  chunk_tokens=16384),
}


# The layer plan of the pages' model as workload layout: one (name, tokens per
# entry, layer modes) per stored cache, in layer order [P2 四、"CSA2：三种模式，
# 40 层只存 4 份"]: three encoder caches (2->1), each read by one Full and five
# Reuse layers; one decoder cache (one entry per token) read by Full + 3 Reuse
# and then four times Reindex + 3 Reuse.  The two encoder layers the page gives
# no mode are not in it.  Mode strings and ratios only; the GPU workloads and
# tests build their caches and layers from this table.
CSA2_PLAN = (
    ("encoder0", 2, ("full",) + ("reuse",) * 5),
    ("encoder1", 2, ("full",) + ("reuse",) * 5),
    ("encoder2", 2, ("full",) + ("reuse",) * 5),
    ("decoder", 1, ("full",) + ("reuse",) * 3 + (("reindex",) + ("reuse",) * 3) * 4),
)


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some sizes replaced (small parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(over)
    return Workload(**d)


# ---------------------------------------------------------------- generators

def _law(w: Workload, g: np.random.Generator, shape) -> np.ndarray:
    if w.entry_law == "normal":
        return normal(g, shape)
    if w.entry_law == "t3":
        return student_t3(g, shape)
    if w.entry_law == "outliers":
        return normal_outliers(g, shape)
    raise ValueError(w.entry_law)


def entry_counts(w: Workload) -> np.ndarray:
    """Compressed entries resident per sequence before the step (int64 [B])."""
    if w.entries is not None:
        return np.full(w.batch, w.entries, dtype=np.int64)
    if w.ragged_tokens is not None:
        lo, hi = w.ragged_tokens
        t = rng(w.seed, S_LENGTHS).integers(lo, hi + 1, size=w.batch, dtype=np.int64)
        return t // 2
    return np.zeros(w.batch, dtype=np.int64)


def cache_entries(w: Workload, b: int, n: Optional[int] = None) -> np.ndarray:
    """fp32 [n, dim] pre-quantisation entries of sequence b (entries-mode cache build)."""
    if n is None:
        n = int(entry_counts(w)[b])
    return _law(w, rng(w.seed, S_ENTRIES, b), (n, w.dim))


def cache_idx_keys(w: Workload, b: int, n: Optional[int] = None) -> np.ndarray:
    """bf16 bits [n, idx_dim] indexer keys of sequence b, integers in [-8, 8]."""
    if n is None:
        n = int(entry_counts(w)[b])
    return int_bf16(rng(w.seed, S_IDXKEY, b), (n, w.idx_dim))


def w_comp(w: Workload) -> np.ndarray:
    """fp32 [dim, 2*dim] stand-in compressor weights, N(0, 0.02)."""
    return normal(rng(w.seed, S_WCOMP), (w.dim, 2 * w.dim), std=0.02)


def prefill_tokens(w: Workload, b: int, n: int) -> np.ndarray:
    """fp32 [n, dim] tokens appended through the compressor."""
    g = rng(w.seed, S_TOKENS, b)
    return _law(w, g, (n, w.dim)) if w.entry_law == "outliers" else normal(g, (n, w.dim))


def prefill_idx_rows(w: Workload, b: int, n: int) -> np.ndarray:
    """bf16 bits [n, idx_dim]: one indexer-key row per appended token."""
    return int_bf16(rng(w.seed, S_TOKENS, b, 1), (n, w.idx_dim))


@dataclass
class StepInputs:
    """Per-step inputs of one decode step (one token per sequence)."""
    token: np.ndarray       # fp32 [B, dim]  new token row fed to the compressor
    idx_row: np.ndarray     # bf16 [B, idx_dim] indexer key row of the new token
    q: list = field(default_factory=list)        # per layer fp32 [B, Hq, dim]
    q_idx: list = field(default_factory=list)    # per layer bf16 [B, Hi, idx_dim] (None for reuse)
    swa_ring: list = field(default_factory=list)  # per layer bf16 [B, W, dim] resident window
    swa_row: list = field(default_factory=list)   # per layer fp32 [B, dim] row appended this step


def step_inputs(w: Workload, step: int = 0, seqs=None) -> StepInputs:
    seqs = range(w.batch) if seqs is None else list(seqs)
    tok, irow = [], []
    for b in seqs:
        g = rng(w.seed, S_STEP, step, b)
        tok.append(normal(g, (w.dim,)))
        irow.append(int_bf16(g, (w.idx_dim,)))
    out = StepInputs(token=np.stack(tok), idx_row=np.stack(irow))
    for li, mode in enumerate(w.layers):
        qs, qis, rings, rows = [], [], [], []
        for b in seqs:
            qs.append(normal(rng(w.seed, S_Q, step, li, b), (w.q_heads, w.dim)))
            if mode in ("full", "reindex"):
                qis.append(int_bf16(rng(w.seed, S_QIDX, step, li, b), (w.idx_heads, w.idx_dim)))
            g = rng(w.seed, S_SWA, li, b)
            rings.append(normal_bf16_trunc(g, (w.window, w.dim)))
            rows.append(normal(rng(w.seed, S_SWA, li, b, step + 1), (w.dim,)))
        out.q.append(np.stack(qs))
        out.q_idx.append(np.stack(qis) if qis else None)
        out.swa_ring.append(np.stack(rings))
        out.swa_row.append(np.stack(rows))
    return out


def head_weights_int(seed: int, batch: int, heads: int, lo: int = 0, hi: int = 3) -> np.ndarray:
    """Optional per-sequence indexer head weights, small integers as fp32 [B, Hi]."""
    return rng(seed, S_HEADW).integers(lo, hi + 1, size=(batch, heads)).astype(np.float32)
