"""Plain fp64 CPU oracle for key-based block selection (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library.

What it computes
----------------
The gist.science explainer of the ART paper, section 2.4, integrates ART with
KV-cache managers by changing the traversal sequence of the KV blocks,
naming "importance-first" as one such order, and states that reordering adds
no error.  The pages define neither the importance of a block nor a
selection rule.  Readings (listed with their reasons in the design notes):

* R21 / R26  a block's importance is the mean query of the unit (the mean of
  its G query rows) dotted with the block's mean key (the mean of its valid
  key rows).  The selection keeps the first ``sink`` blocks, the ``recent``
  most recent blocks, and fills up to ceil(keep_frac * T) blocks with the
  highest importance, ties to the lower block index.
* R27  the importance order lists the kept blocks by decreasing importance,
  ties to the lower block index; the traversal rule (explainer section 2.4)
  still moves block 0 to the front when ART walks the list.

Everything is fp64 and written out directly: means by summation and
division, scores by a dot product, the selection by one stable sort.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

SELECT_ASCENDING = 0   # kept blocks in ascending block order
SELECT_IMPORTANCE = 1  # kept blocks by decreasing importance


def block_means(K: np.ndarray, n_ctx: int, block_size: int = 64) -> np.ndarray:
    """Mean of the valid key rows of every block: [T, d] (fp64)."""
    K = np.asarray(K, dtype=np.float64)
    T = (n_ctx + block_size - 1) // block_size
    out = np.zeros((T, K.shape[1]))
    for j in range(T):
        rows = K[j * block_size: min(n_ctx, (j + 1) * block_size)]
        out[j] = rows.sum(axis=0) / rows.shape[0]
    return out


def mean_query(q_unit: np.ndarray) -> np.ndarray:
    """Mean of the unit's G query rows: [d]."""
    return np.asarray(q_unit, dtype=np.float64).mean(axis=0)


def block_scores(q_unit: np.ndarray, means: np.ndarray) -> np.ndarray:
    """Importance of every block: mean query . block-mean key (R26)."""
    return means @ mean_query(q_unit)


def keep_count(T: int, keep_frac: float) -> int:
    """ceil(keep_frac * T) blocks, at most T (keep_frac as float32, as it
    crosses the library's interface)."""
    return min(T, int(math.ceil(float(np.float32(keep_frac)) * T)))


def select_blocks(scores: np.ndarray, keep_frac: float, sink: int, recent: int,
                  order: int = SELECT_ASCENDING) -> np.ndarray:
    """The kept list of one unit (R26, R27)."""
    T = int(scores.shape[0])
    n_keep = keep_count(T, keep_frac)
    forced = set(range(min(sink, T, n_keep)))
    n_recent = max(0, min(recent, n_keep - len(forced)))
    forced |= set(range(T - n_recent, T))
    # rank: forced blocks first, then decreasing score, then increasing index
    rank = sorted(range(T), key=lambda j: (0 if j in forced else 1, -scores[j], j))
    kept = rank[:n_keep]
    if order == SELECT_ASCENDING:
        return np.array(sorted(kept), dtype=np.int32)
    return np.array(sorted(kept, key=lambda j: (-scores[j], j)), dtype=np.int32)


def select_unit(q_unit: np.ndarray, K: np.ndarray, n_ctx: int, keep_frac: float, sink: int,
                recent: int, order: int = SELECT_ASCENDING, block_size: int = 64):
    """Means, scores and the kept list of one unit."""
    means = block_means(K, n_ctx, block_size)
    scores = block_scores(q_unit, means)
    return means, scores, select_blocks(scores, keep_frac, sink, recent, order)


def select_workload(w, keep_frac: float, sink: int, recent: int, order: int = SELECT_ASCENDING,
                    units: Optional[list] = None):
    """Kept lists for a ``workloads.Workload``-shaped object (its own kept
    list, if any, is ignored: selection runs over every block).

    Returns (kept_blocks [B, Hkv, max_kept] int32 padded with -1, kept_count
    [B, Hkv] int32, {(b, h): (means, scores)})."""
    from .art_oracle import gather_unit, widen
    s = w.spec
    G = s.num_q_heads // s.num_kv_heads
    lists, detail = {}, {}
    allu = [(b, h) for b in range(s.batch) for h in range(s.num_kv_heads)]
    for (b, h) in (units or allu):
        n = int(w.context_lens[b])
        q_unit = widen(w.q[b, h * G:(h + 1) * G], s.dtype)
        Ks, _ = gather_unit(w.k, w.v, b, h, n, s.page_size, w.block_table)
        means, scores, kept = select_unit(q_unit, widen(Ks, s.dtype), n, keep_frac, sink, recent, order,
                                          s.block_size)
        lists[(b, h)] = kept
        detail[(b, h)] = (means, scores)
    max_kept = max([1] + [len(x) for x in lists.values()])
    kb = np.full((s.batch, s.num_kv_heads, max_kept), -1, dtype=np.int32)
    kc = np.zeros((s.batch, s.num_kv_heads), dtype=np.int32)
    for (b, h), lst in lists.items():
        kb[b, h, :len(lst)] = lst
        kc[b, h] = len(lst)
    return kb, kc, detail
