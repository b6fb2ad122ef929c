"""Seeded synthetic decode-attention workloads.

This module only draws inputs: it holds none of the attention or stopping
arithmetic.  Both the HIP path (through the Python binding) and the CPU
oracle consume exactly the arrays it returns.

Source of the shapes: the five decode configurations the method is measured
on (tiny single-head fp32, a Llama-3-8B-shaped contiguous layer, large-batch
paged, very-large-batch paged, long context with a kept-block list).  The
pages evaluate on LongBench with real models; those are absent here, and these
generators stand in for them.

Two readings of "same key/value generator as config 1" exist for the paged
configurations (see ``READINGS``):

* ``"A"`` -- the literal tiny-config generator: q, K, V ~ N(0, 1) i.i.d.; the
  64 most recent keys get ``+2.0 * u`` where ``u`` is the unit's mean query
  direction.
* ``"B"`` -- the Llama-shaped generator: V ~ N(0, 1); each key gets noise plus
  a logit shift along ``u`` of ``3 * exp(-dist / 2048)`` (recency), ``+6`` at
  positions 0..3 (attention sinks), and ``-4`` at 1 % random positions whose
  values are scaled by 8 (low score, large value).  A logit shift ``delta`` is
  applied as ``k += delta * sqrt(d) / |qbar| * u`` so the mean query's scaled
  score moves by exactly ``delta``.

Storage: bf16 configurations hold bf16 bit patterns (``uint16``) produced by
round-to-nearest-even from float32; fp32 configurations hold ``float32``.
Slots that hold no valid token (the tail of a sequence's last page, the tail
of a contiguous row, and one extra "poison" page that every unused
block-table entry points at) are filled with NaN, so a kernel that reads or
weights an invalid token produces NaN instead of a plausible number.

Determinism: every (batch, kv head) unit draws from its own generator seeded
with ``[seed, reading, b, h]``, so any unit can be regenerated alone and the
generation can run on several threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

READINGS = ("A", "B")
_READING_CODE = {"A": 1, "B": 2}

ORDER_NATURAL = 0
ORDER_RECENT_FIRST = 1
ORDER_GIVEN = 2

BF16_NAN = np.uint16(0x7FC0)


# ---------------------------------------------------------------------------
# storage conversions (no method arithmetic)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values (bf16 bits or float32) to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# workload description
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic decode workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                     # "bf16" | "f32"
    ctx: tuple                     # (lo, hi) inclusive; lo == hi for fixed
    page_size: int = 0             # 0 = contiguous [B, Hkv, max_ctx, d]
    block_size: int = 64
    reading: str = "A"
    eps_scale: float = 1e-3
    eps_dir: float = 1e-4
    patience: int = 2
    order: int = ORDER_RECENT_FIRST
    kept_frac: float = 0.0         # 0 = no kept list
    kept_recent: int = 256         # most recent blocks always kept
    kept_sink: int = 1             # leading blocks always kept
    seed: int = 1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class Workload:
    spec: Spec
    context_lens: np.ndarray                 # int32 [B]
    q: np.ndarray                            # [B, Hq, d] bf16 bits or f32
    k: np.ndarray                            # contiguous [B,Hkv,Nmax,d] or paged [P+1,Hkv,page,d]
    v: np.ndarray
    block_table: Optional[np.ndarray] = None  # int32 [B, max_pages]
    kept_blocks: Optional[np.ndarray] = None  # int32 [B, Hkv, max_kept]
    kept_count: Optional[np.ndarray] = None   # int32 [B, Hkv]
    max_ctx: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> np.ndarray:
        bs = self.spec.block_size
        return (self.context_lens.astype(np.int64) + bs - 1) // bs

    def traversal_lengths(self) -> np.ndarray:
        """T' per unit [B, Hkv]: kept count, or all blocks of the sequence."""
        if self.kept_count is not None:
            return self.kept_count.astype(np.int64)
        return np.repeat(self.num_blocks[:, None], self.spec.num_kv_heads, axis=1)

    def kv_bytes_resident(self) -> int:
        es = 2 if self.spec.dtype == "bf16" else 4
        return int(self.context_lens.astype(np.int64).sum()) * self.spec.num_kv_heads * self.spec.head_dim * 2 * es


# The five measured configurations at full size.
CONFIGS = {
    1: Spec("cfg1-tiny-f32", 1, 1, 1, 64, "f32", (1024, 1024), 0, 64, "A",
            1e-3, 1e-4, 2, ORDER_RECENT_FIRST, seed=1),
    2: Spec("cfg2-llama3-8b-contig", 16, 32, 8, 128, "bf16", (32768, 32768), 0, 64, "B",
            1e-3, 1e-4, 2, ORDER_RECENT_FIRST, seed=2),
    3: Spec("cfg3-paged-b64", 64, 32, 8, 128, "bf16", (8192, 32768), 16, 64, "A",
            2e-3, 2e-4, 3, ORDER_RECENT_FIRST, seed=3),
    4: Spec("cfg4-paged-b128", 128, 32, 8, 128, "bf16", (16384, 16384), 16, 64, "A",
            2e-3, 2e-4, 2, ORDER_RECENT_FIRST, seed=4),
    5: Spec("cfg5-long-kept", 4, 32, 8, 128, "bf16", (131072, 131072), 16, 64, "A",
            1e-3, 1e-4, 2, ORDER_RECENT_FIRST, kept_frac=0.5, kept_recent=256,
            kept_sink=1, seed=5),
}
# Patience values swept on config 4.
CFG4_PATIENCE_SWEEP = (1, 2, 4)


def config(n: int, reading: Optional[str] = None, **overrides) -> Spec:
    s = CONFIGS[n]
    if reading is not None:
        overrides["reading"] = reading
    return replace(s, **overrides) if overrides else s


# ---------------------------------------------------------------------------
# per-unit draws
# ---------------------------------------------------------------------------
def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def draw_unit(spec: Spec, b: int, h: int, n_ctx: int):
    """Draw (q[G,d], K[N,d], V[N,d]) for unit (b, h) in storage format."""
    G, d = spec.group, spec.head_dim
    rng = np.random.default_rng([spec.seed, _READING_CODE[spec.reading], b, h])
    q = _store(rng.standard_normal((G, d), dtype=np.float32), spec.dtype)
    K = rng.standard_normal((n_ctx, d), dtype=np.float32)
    V = rng.standard_normal((n_ctx, d), dtype=np.float32)
    qv = storage_to_f64(q, spec.dtype)
    qbar = qv.mean(axis=0)
    qn = float(np.linalg.norm(qbar))
    u = qbar / qn if qn > 0 else np.zeros(d)
    if spec.reading == "A":
        lo = max(0, n_ctx - 64)
        K[lo:] += (2.0 * u).astype(np.float32)
    else:
        n = np.arange(n_ctx, dtype=np.float64)
        delta = 3.0 * np.exp(-(n_ctx - 1 - n) / 2048.0)
        delta[: min(4, n_ctx)] += 6.0
        n_low = n_ctx // 100
        if n_low > 0 and n_ctx > 4:
            pos = 4 + rng.choice(n_ctx - 4, size=n_low, replace=False)
            delta[pos] += -4.0
            V[pos] *= np.float32(8.0)
        scale = math.sqrt(d) / qn if qn > 0 else 0.0
        K += ((delta * scale)[:, None] * u[None, :]).astype(np.float32)
    return q, _store(K, spec.dtype), _store(V, spec.dtype)


def draw_context_lens(spec: Spec) -> np.ndarray:
    lo, hi = spec.ctx
    if lo == hi:
        return np.full(spec.batch, lo, dtype=np.int32)
    rng = np.random.default_rng([spec.seed, 7919])
    return rng.integers(lo, hi, size=spec.batch, endpoint=True).astype(np.int32)


def select_kept_blocks(spec: Spec, q_unit: np.ndarray, K_unit: np.ndarray, n_ctx: int) -> np.ndarray:
    """Key-based block selection standing in for a KV-pruning method.

    Keeps the first ``kept_sink`` blocks, the ``kept_recent`` most recent
    blocks, and fills up to ``ceil(kept_frac * T)`` blocks with the highest
    mean-query score against the block-mean key (ties to the lower index).
    Returns the kept block indices sorted ascending.
    """
    bs, d = spec.block_size, spec.head_dim
    T = (n_ctx + bs - 1) // bs
    n_keep = min(T, int(math.ceil(spec.kept_frac * T)))
    sink = set(range(min(spec.kept_sink, T, n_keep)))
    n_recent = min(spec.kept_recent, n_keep - len(sink))
    forced = sink | set(range(max(0, T - n_recent), T))
    if len(forced) >= n_keep:
        return np.array(sorted(forced), dtype=np.int32)
    qv = storage_to_f64(q_unit, spec.dtype).mean(axis=0)
    Kv = storage_to_f64(K_unit, spec.dtype)
    pad = T * bs - n_ctx
    sums = np.concatenate([Kv, np.zeros((pad, d))]).reshape(T, bs, d).sum(axis=1)
    counts = np.full(T, bs, dtype=np.float64)
    counts[-1] = n_ctx - (T - 1) * bs
    score = (sums / counts[:, None]) @ qv
    rest = np.array([j for j in range(T) if j not in forced], dtype=np.int64)
    order = rest[np.lexsort((rest, -score[rest]))]
    chosen = sorted(forced | set(order[: n_keep - len(forced)].tolist()))
    return np.array(chosen, dtype=np.int32)


# ---------------------------------------------------------------------------
# whole workloads
# ---------------------------------------------------------------------------
def _threads(threads: Optional[int]) -> int:
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def make_workload(spec: Spec, threads: Optional[int] = None, context_lens=None) -> Workload:
    """Build the whole workload in host memory (storage formats)."""
    B, Hq, Hkv, d = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    G = spec.group
    assert Hq % Hkv == 0
    lens = draw_context_lens(spec) if context_lens is None else np.asarray(context_lens, dtype=np.int32)
    assert lens.shape == (B,)
    sdt = np.uint16 if spec.dtype == "bf16" else np.float32
    nan = BF16_NAN if spec.dtype == "bf16" else np.float32(np.nan)
    max_ctx = int(max(1, lens.max())) if B else 1
    q = np.empty((B, Hq, d), dtype=sdt)
    block_table = None
    kept_lists = {}

    if spec.page_size == 0:
        k = np.full((B, Hkv, max_ctx, d), nan, dtype=sdt)
        v = np.full((B, Hkv, max_ctx, d), nan, dtype=sdt)
    else:
        P = spec.page_size
        n_pages = (lens.astype(np.int64) + P - 1) // P
        total = int(n_pages.sum())
        max_pages = int(max(1, n_pages.max())) if B else 1
        rng = np.random.default_rng([spec.seed, 104729])
        perm = rng.permutation(total).astype(np.int32)
        poison = total  # extra page full of NaN
        block_table = np.full((B, max_pages), poison, dtype=np.int32)
        off = 0
        for b in range(B):
            block_table[b, : n_pages[b]] = perm[off: off + n_pages[b]]
            off += int(n_pages[b])
        k = np.full((total + 1, Hkv, P, d), nan, dtype=sdt)
        v = np.full((total + 1, Hkv, P, d), nan, dtype=sdt)

    def fill(bh):
        b, h = bh
        n = int(lens[b])
        qu, Ku, Vu = draw_unit(spec, b, h, n)
        q[b, h * G:(h + 1) * G] = qu
        if spec.page_size == 0:
            k[b, h, :n] = Ku
            v[b, h, :n] = Vu
        else:
            P = spec.page_size
            np_b = (n + P - 1) // P
            pages = block_table[b, :np_b]
            full = n // P
            if full:
                k[pages[:full], h] = Ku[: full * P].reshape(full, P, d)
                v[pages[:full], h] = Vu[: full * P].reshape(full, P, d)
            if n % P:
                k[pages[full], h, : n % P] = Ku[full * P:]
                v[pages[full], h, : n % P] = Vu[full * P:]
        if spec.kept_frac > 0:
            kept_lists[(b, h)] = select_kept_blocks(spec, qu, Ku, n)

    units = [(b, h) for b in range(B) for h in range(Hkv)]
    nt = _threads(threads)
    if nt > 1 and len(units) > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, units))
    else:
        for u in units:
            fill(u)

    kept_blocks = kept_count = None
    if spec.kept_frac > 0:
        max_kept = max(1, max(len(x) for x in kept_lists.values())) if kept_lists else 1
        kept_blocks = np.full((B, Hkv, max_kept), -1, dtype=np.int32)
        kept_count = np.zeros((B, Hkv), dtype=np.int32)
        for (b, h), lst in kept_lists.items():
            kept_blocks[b, h, : len(lst)] = lst
            kept_count[b, h] = len(lst)

    return Workload(spec=spec, context_lens=lens, q=q, k=k, v=v, block_table=block_table,
                    kept_blocks=kept_blocks, kept_count=kept_count, max_ctx=max_ctx,
                    meta={"reading": spec.reading, "seed": spec.seed})


def multi_row_queries(w: Workload, rows: int, spread: float = 0.5) -> np.ndarray:
    """Query rows [B, rows, Hq, d] in storage format for multi-row decode:
    row 0 is the workload's own query, row i >= 1 adds spread * N(0, 1)
    noise (seeded per workload and row), like the nearby draft tokens of a
    speculative step."""
    s = w.spec
    base = storage_to_f64(w.q, s.dtype)
    out = [w.q]
    for i in range(1, rows):
        rng = np.random.default_rng([s.seed, 104729, i])
        out.append(_store(base + spread * rng.standard_normal(base.shape), s.dtype))
    return np.stack(out, axis=1)


def scaled(n: int, reading: Optional[str] = None, **overrides) -> Spec:
    """Small versions of the five configurations, for CPU-checkable parity.

    They keep each configuration's dtype, head geometry, layout, block size,
    generator and parameters, and shrink batch and context so that the oracle
    finishes in seconds while still spanning several blocks, a ragged tail
    and (paged) several pages per block.
    """
    small = {
        1: dict(),
        2: dict(batch=2, num_q_heads=8, num_kv_heads=2, ctx=(4096 + 37, 4096 + 37)),
        3: dict(batch=4, num_q_heads=8, num_kv_heads=2, ctx=(700, 5000)),
        4: dict(batch=6, num_q_heads=8, num_kv_heads=2, ctx=(2048 + 5, 2048 + 5)),
        5: dict(batch=2, num_q_heads=8, num_kv_heads=2, ctx=(8192 + 100, 8192 + 100), kept_recent=24),
    }[n]
    small.update(overrides)
    return config(n, reading, **small)
