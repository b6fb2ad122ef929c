"""Plain fp64 CPU oracle for ART decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP library; both sides only read the same seeded inputs.

What it computes, in the pages' order and notation
--------------------------------------------------
Sources (cited by page and section):

* [ART-3.1]  ART paper (arXiv 2606.00024, Chinese rendering), section 3.1,
  Eq. (1): O = softmax(Q K^T / sqrt(d)) V; the kernel splits K, V into blocks
  {(K_t, V_t)}, t = 1..T, and O^(t) is the attention output after the first
  t blocks, converging to O^(T).
* [ART-3.2]  same paper, section 3.2: a probe vector x^(t) taken from a
  deterministic, scattered subsample of the head dimensions of O^(t).
* [GIST-2.2] gist.science explainer of the same paper, section 2.2: two
  stability metrics -- magnitude variation d_scale (L2-norm difference between
  current and previous probe) and direction change d_direction (deviation of
  their cosine similarity) -- and termination only when both are below their
  thresholds (tau for scale, phi for direction) at the same time.
* [GIST-2.3] same explainer, section 2.3: the criteria must hold for
  ``patience`` consecutive KV blocks before termination.
* [GIST-2.4] same explainer, section 2.4: blocks may be traversed in another
  order (recency-first, importance-first); reordering adds no error because
  attention is permutation invariant; block 0 (often an attention sink) is
  always evaluated before any termination.
* [FLEX-A3]  FlexPrefill summary, background section: attention restricted to
  an index set S is softmax((Q K^T + M_S)/sqrt(d)) V with M_S in {0, -inf}.

Readings taken where the pages are silent or ambiguous (each one is used
below and listed with its reason in the design notes):

* R1  d_scale = | |x^(t)| - |x^(t-1)| | / |x^(t-1)|  (relative norm change,
      previous norm in the denominator).
* R2  d_dir = 1 - cos(x^(t), x^(t-1)).
* R3  both comparisons are strict (<).
* R4  the probe is taken from the normalized output O^(t), not from an
      unnormalized accumulator.
* R5  probe dims are {0, 4, 8, ..., d-4} of every query head of the group,
      concatenated head by head (m = G*d/4).
* R6  one decision per (batch, kv head) unit; the G query heads that share
      the kv head share the probe.
* R7  a check exists for t >= 2 (there is no O^(0)); the counter counts
      consecutive stable checks; stop after block t once counter >= patience.
      So the stop index lies in [min(T', p+1), T'].
* R8  block 0 goes first in every traversal when it is a candidate.
* R9  recency-first = highest block index first (after block 0); a partial
      last block is one block; tokens beyond the context length do not exist.
* R10 stop_idx = number of traversal blocks processed (1..T'); T' = number of
      candidate blocks (all blocks, or the kept list).
* R11 a zero-norm probe (previous or current) is never stable.
* R12 query head g of kv head h is q head h*G + g.
* R13 scale 1/sqrt(d); no mask inside the cache beyond the context length.
* Thresholds are single-precision values (as passed through the C ABI)
      compared in double precision.
* R28 multi-row queries (Q with M rows per sequence, Eq. (1)): the M*G query
      vectors of a unit share its traversal and its one stop; the probe
      concatenates all of them (row by row, head by head), as R6 does for
      the G heads.

Numerics: all arithmetic in float64 on exactly widened inputs.  O^(t) is
computed from per-block weighted sums and their prefix sums with one shift
by the maximum score over all candidate tokens; the shift cancels in the
ratio, and the code refuses inputs where it would underflow a block away.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

ORDER_NATURAL = 0
ORDER_RECENT_FIRST = 1
ORDER_GIVEN = 2

MODE_FULL = 0
MODE_ART = 1

# Ablation and measurement switches (the library's art_params.flags bits).
# The pages attribute the method's robustness to requiring both metrics at
# once (gist.science explainer, section 2.2) and measure the detector's own
# cost with termination disabled (same explainer, experiments); these
# switches take one metric out, or keep the detector but never stop.
FLAG_NO_SCALE = 1     # the magnitude test always passes
FLAG_NO_DIR = 2       # the direction test always passes
FLAG_DETECT_ONLY = 4  # evaluate the rule, report its stop, attend over every block

PROBE_STRIDE = 4  # R5


# ---------------------------------------------------------------------------
# input widening (exact)
# ---------------------------------------------------------------------------
def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 bit patterns or float32 -> float64, exactly."""
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# traversal [GIST-2.4], R8, R9
# ---------------------------------------------------------------------------
def traversal(num_blocks: int, kept: Optional[Sequence[int]] = None,
              order: int = ORDER_RECENT_FIRST) -> list:
    """Block indices in the order they are processed.

    Candidates are ``kept`` (a kept-block list from a key-based KV manager;
    distinct blocks of the sequence, else ValueError) or every block
    0..num_blocks-1.  Block 0, when a candidate, is first.
    NATURAL: ascending.  RECENT_FIRST: descending.  GIVEN: the list order.
    """
    cand = list(range(num_blocks)) if kept is None else [int(c) for c in kept]
    if kept is not None:
        # the candidates are a set of the sequence's blocks (the blocks a KV
        # manager retains, [GIST-2.4]); a list naming a block twice or one
        # outside the sequence is not such a set and is refused
        if len(set(cand)) != len(cand):
            raise ValueError("kept list names a block more than once")
        if any(c < 0 or c >= num_blocks for c in cand):
            raise ValueError("kept list names a block outside the sequence")
    head = [0] if 0 in cand else []
    rest = [c for c in cand if c != 0]
    if order == ORDER_NATURAL:
        rest = sorted(rest)
    elif order == ORDER_RECENT_FIRST:
        rest = sorted(rest, reverse=True)
    elif order == ORDER_GIVEN:
        pass
    else:
        raise ValueError(f"unknown order {order}")
    return head + rest


def block_tokens(j: int, n_ctx: int, block_size: int) -> np.ndarray:
    """Token positions of block j: [j*bs, min(n_ctx, (j+1)*bs))."""
    return np.arange(j * block_size, min(n_ctx, (j + 1) * block_size))


# ---------------------------------------------------------------------------
# partial outputs O^(t) [ART-3.1], Eq. (1) restricted to processed blocks
# ---------------------------------------------------------------------------
def prefix_outputs(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_ctx: int,
                   order_blocks: Sequence[int], block_size: int):
    """O^(t) for t = 1..T' (float64 [T', G, d]) and the per-block softmax mass.

    q: [G, d]; K, V: [n_ctx, d] (float64).  O^(t) is softmax attention of the
    G query rows over the tokens of the first t traversal blocks.
    """
    G, d = q.shape
    Tp = len(order_blocks)
    if Tp == 0:
        return np.zeros((0, G, d)), np.zeros((0, G))
    toks = [block_tokens(j, n_ctx, block_size) for j in order_blocks]
    allt = np.concatenate(toks)
    s = (q @ K[allt].T) / math.sqrt(d)            # [G, n_cand] scores, Eq. (1)
    M = s.max(axis=1, keepdims=True)
    w = np.exp(s - M)                              # unnormalized softmax weights
    # Per-block sums W_t = sum w, A_t = sum w v over the block's tokens.
    Wb = np.empty((Tp, G))
    Ab = np.empty((Tp, G, d))
    off = 0
    blk_min_gap = np.inf
    for t, tk in enumerate(toks):
        n = len(tk)
        wt = w[:, off:off + n]
        Wb[t] = wt.sum(axis=1)
        Ab[t] = wt @ V[tk]
        if n:
            blk_min_gap = min(blk_min_gap, float((s[:, off:off + n].max(axis=1) - M[:, 0]).min()))
        off += n
    if blk_min_gap < -600.0:
        raise NotImplementedError("scores span more than e^600; the single-shift prefix sums would underflow")
    cumW = np.cumsum(Wb, axis=0)
    cumA = np.cumsum(Ab, axis=0)
    O = cumA / cumW[:, :, None]
    mass = Wb / cumW[-1][None, :]                   # softmax mass of each block over all candidates
    return O, mass


# ---------------------------------------------------------------------------
# probe [ART-3.2], R4, R5
# ---------------------------------------------------------------------------
def probe(O: np.ndarray) -> np.ndarray:
    """x^(t): dims 0, 4, 8, ... of each query head of O^(t), concatenated."""
    T, G, d = O.shape
    return O[:, :, 0::PROBE_STRIDE].reshape(T, G * ((d + PROBE_STRIDE - 1) // PROBE_STRIDE))


# ---------------------------------------------------------------------------
# stability metrics [GIST-2.2], R1, R2, R11
# ---------------------------------------------------------------------------
def stability_trace(x: np.ndarray):
    """d_scale[t], d_dir[t] for every traversal step (NaN for t = 1).

    Also returns the cancellation-free form of d_dir,
    0.5 * | x_t/|x_t| - x_{t-1}/|x_{t-1}| |^2, which equals 1 - cos exactly
    in real arithmetic; and a validity mask (False where a norm is zero).
    """
    T = x.shape[0]
    d_scale = np.full(T, np.nan)
    d_dir = np.full(T, np.nan)
    d_dir_stable = np.full(T, np.nan)
    valid = np.zeros(T, dtype=bool)
    for t in range(1, T):
        prev, cur = x[t - 1], x[t]
        a = float(np.sqrt(prev @ prev))
        b = float(np.sqrt(cur @ cur))
        if a == 0.0 or b == 0.0:
            continue
        valid[t] = True
        d_scale[t] = abs(b - a) / a
        d_dir[t] = 1.0 - float(cur @ prev) / (a * b)
        diff = cur / b - prev / a
        d_dir_stable[t] = 0.5 * float(diff @ diff)
    return d_scale, d_dir, d_dir_stable, valid


def threshold(eps: float) -> float:
    """A threshold as the single-precision value the C ABI carries."""
    return float(np.float32(eps))


# ---------------------------------------------------------------------------
# dual threshold + patience [GIST-2.2], [GIST-2.3], R3, R7
# ---------------------------------------------------------------------------
def stop_index(d_scale: np.ndarray, d_dir: np.ndarray, valid: np.ndarray,
               eps_scale: float, eps_dir: float, patience: int, mode: int = MODE_ART,
               flags: int = 0) -> int:
    """Number of traversal blocks processed before the criterion fires.

    ``flags`` may switch one metric's test off (FLAG_NO_SCALE, FLAG_NO_DIR);
    a zero-norm probe still never counts as stable."""
    T = len(d_scale)
    if mode == MODE_FULL or T == 0:
        return T
    if patience < 1:
        raise ValueError("patience must be >= 1")
    tau, phi = threshold(eps_scale), threshold(eps_dir)
    use_scale, use_dir = not (flags & FLAG_NO_SCALE), not (flags & FLAG_NO_DIR)
    count = 0
    for t in range(1, T):                   # check for traversal step t+1 (1-based)
        stable = bool(valid[t]) and (not use_scale or d_scale[t] < tau) and (not use_dir or d_dir[t] < phi)
        count = count + 1 if stable else 0
        if count >= patience:
            return t + 1
    return T


@dataclass
class UnitResult:
    out: np.ndarray          # [G, d] O^(stop)
    stop: int                # stop_idx
    num_traversal: int       # T'
    order_blocks: list       # pi
    O: np.ndarray            # [T', G, d] every O^(t)
    d_scale: np.ndarray
    d_dir: np.ndarray
    d_dir_stable: np.ndarray
    valid: np.ndarray
    mass: np.ndarray         # [T', G] softmax mass of each traversal block


def art_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_ctx: int, block_size: int,
             eps_scale: float, eps_dir: float, patience: int, order: int = ORDER_RECENT_FIRST,
             kept: Optional[Sequence[int]] = None, mode: int = MODE_ART, flags: int = 0) -> UnitResult:
    """ART for one (batch, kv head) unit; q [G, d], K/V [n_ctx, d] in float64.

    With FLAG_DETECT_ONLY the stop is reported but the output covers every
    traversal block (O^(T'))."""
    T = (n_ctx + block_size - 1) // block_size
    pi = traversal(T, kept, order)
    O, mass = prefix_outputs(q, K, V, n_ctx, pi, block_size)
    x = probe(O)
    ds, dd, dds, valid = stability_trace(x)
    stop = stop_index(ds, dd, valid, eps_scale, eps_dir, patience, mode, flags)
    last = len(pi) if (flags & FLAG_DETECT_ONLY) else stop
    out = O[last - 1] if last > 0 else np.zeros(q.shape)
    return UnitResult(out, stop, len(pi), pi, O, ds, dd, dds, valid, mass)


# ---------------------------------------------------------------------------
# batch front end: contiguous or paged KV, as the C ABI sees it
# ---------------------------------------------------------------------------
def gather_unit(k: np.ndarray, v: np.ndarray, b: int, h: int, n_ctx: int,
                page_size: int, block_table: Optional[np.ndarray]):
    """Keys and values of unit (b, h) in token order (storage format).

    Contiguous: k[b, h, :n_ctx].  Paged: token n lives in page
    block_table[b][n // page_size], slot n % page_size, of k[page, h].
    """
    if page_size == 0:
        return k[b, h, :n_ctx], v[b, h, :n_ctx]
    n = np.arange(n_ctx)
    pages = block_table[b][n // page_size]
    slots = n % page_size
    return k[pages, h, slots], v[pages, h, slots]


def art_decode(q, k, v, context_lens, dtype: str, num_kv_heads: int, block_size: int,
               eps_scale: float, eps_dir: float, patience: int, order: int, mode: int,
               page_size: int = 0, block_table=None, kept_blocks=None, kept_count=None,
               units=None, keep_results: bool = False, flags: int = 0):
    """Oracle for the whole call (or a subset of units).

    Returns out [B, Hq, d] float64 (rows of skipped units are NaN), stop
    [B, Hkv] int64 (-1 for skipped units) and, when ``keep_results``, the
    per-unit ``UnitResult`` objects keyed by (b, h).
    """
    B, Hq, d = q.shape
    G = Hq // num_kv_heads
    out = np.full((B, Hq, d), np.nan)
    stop = np.full((B, num_kv_heads), -1, dtype=np.int64)
    results = {}
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(num_kv_heads)]
    for (b, h) in todo:
        n = int(context_lens[b])
        Ks, Vs = gather_unit(k, v, b, h, n, page_size, block_table)
        kept = None
        if kept_blocks is not None:
            kept = kept_blocks[b, h, : int(kept_count[b, h])]
        r = art_unit(widen(q[b, h * G:(h + 1) * G], dtype), widen(Ks, dtype), widen(Vs, dtype), n,
                     block_size, eps_scale, eps_dir, patience, order, kept, mode, flags)
        out[b, h * G:(h + 1) * G] = r.out
        stop[b, h] = r.stop
        if keep_results:
            results[(b, h)] = r
    return out, stop, results


def art_decode_rows(q_rows, k, v, context_lens, dtype: str, num_kv_heads: int, block_size: int,
                    eps_scale: float, eps_dir: float, patience: int, order: int, mode: int,
                    page_size: int = 0, block_table=None, kept_blocks=None, kept_count=None,
                    units=None, keep_results: bool = False, flags: int = 0):
    """Multi-row queries (R28): q_rows [B, M, Hq, d], M query rows per
    sequence against the same cached context.  The M*G query vectors of unit
    (b, h), taken row by row (row i, head g at position i*G + g), share the
    unit's traversal and its one stop decision, exactly as the G heads of a
    GQA group do [ART-3.1 Eq. (1) with Q of M*G rows; GIST-2.2 on their
    concatenated probe].  Returns out [B, M, Hq, d], stop [B, Hkv] and the
    per-unit results (their rows in that order)."""
    B, M, Hq, d = q_rows.shape
    G = Hq // num_kv_heads
    q_units = (np.asarray(q_rows).reshape(B, M, num_kv_heads, G, d).transpose(0, 2, 1, 3, 4)
               .reshape(B, num_kv_heads * M * G, d))
    out, stop, res = art_decode(q_units, k, v, context_lens, dtype, num_kv_heads, block_size, eps_scale, eps_dir,
                                patience, order, mode, page_size, block_table, kept_blocks, kept_count, units,
                                keep_results, flags)
    out = out.reshape(B, num_kv_heads, M, G, d).transpose(0, 2, 1, 3, 4).reshape(B, M, Hq, d)
    return out, stop, res


def art_decode_workload(w, mode: int = MODE_ART, patience: Optional[int] = None, units=None,
                        keep_results: bool = False, eps_scale=None, eps_dir=None, order=None, flags: int = 0):
    """Convenience wrapper over a ``workloads.Workload``-shaped object."""
    s = w.spec
    return art_decode(w.q, w.k, w.v, w.context_lens, s.dtype, s.num_kv_heads, s.block_size,
                      s.eps_scale if eps_scale is None else eps_scale,
                      s.eps_dir if eps_dir is None else eps_dir,
                      s.patience if patience is None else patience,
                      s.order if order is None else order, mode, s.page_size, w.block_table,
                      w.kept_blocks, w.kept_count, units, keep_results, flags)


def relative_margin(d: np.ndarray, eps: float) -> np.ndarray:
    """|d / eps - 1| per check: how close a metric sits to its threshold."""
    e = threshold(eps)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.abs(np.asarray(d) / e - 1.0)
