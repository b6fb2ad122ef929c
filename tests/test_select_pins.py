"""Pins for the selection oracle (key-based kept lists, importance order).

Each pin checks the oracle against something other than itself: the
workload generator's separate implementation of the same rule, a brute-force
search over subsets, closed forms, and hand-built scores with ties.
"""
import itertools

import numpy as np
import pytest

import oracle as orc
from workloads import make_workload, scaled
from workloads.gen import select_kept_blocks


def test_block_means_closed_form_and_partial_block():
    """Blockwise-constant keys: every block's mean is its constant row, also
    the partial last block (its invalid rows must not count)."""
    d, bs, n = 8, 4, 10  # blocks of 4, 4, 2 rows
    rows = np.array([[1.0] * d] * 4 + [[-2.0] * d] * 4 + [[5.0] * d] * 2)
    m = orc.block_means(rows, n, bs)
    np.testing.assert_array_equal(m, [[1.0] * d, [-2.0] * d, [5.0] * d])
    # count-weighted means recombine to the overall mean
    rng = np.random.default_rng(1)
    K = rng.standard_normal((37, 5))
    m = orc.block_means(K, 37, 8)
    counts = np.array([8, 8, 8, 8, 5])
    np.testing.assert_allclose((m * counts[:, None]).sum(0) / 37, K.mean(0), rtol=1e-13)


def test_scores_use_the_mean_query():
    """Score = mean of the G query rows . block mean; with rows q and -q the
    mean query is zero and every score vanishes."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal(6)
    means = rng.standard_normal((4, 6))
    np.testing.assert_allclose(orc.block_scores(np.stack([q, -q]), means), 0.0, atol=1e-15)
    q2 = np.stack([q, 3 * q])  # mean 2q
    np.testing.assert_allclose(orc.block_scores(q2, means), means @ (2 * q), rtol=1e-14)


def test_keep_count():
    assert orc.keep_count(10, 0.5) == 5
    assert orc.keep_count(11, 0.5) == 6
    assert orc.keep_count(7, 1.0) == 7
    assert orc.keep_count(3, 0.01) == 1
    assert orc.keep_count(0, 0.5) == 0


def test_forced_recent_blocks_are_kept_even_with_low_scores():
    scores = np.array([-9.0, 5.0, 4.0, 3.0, 2.0, 1.0, -8.0, -7.0])  # the two most recent score lowest
    kept = orc.select_blocks(scores, 0.5, sink=1, recent=2)  # keep 4 of 8
    np.testing.assert_array_equal(kept, [0, 1, 6, 7])
    # keep_frac crosses the interface as float32: 2/3 of 6 rounds up to 5 blocks
    assert orc.keep_count(6, 2 / 3) == 5


def test_ties_go_to_the_lower_block_index():
    scores = np.array([0.0, 2.0, 7.0, 2.0, 2.0, 0.0])
    # keep 3 of 6 with one sink and no recent: block 0, block 2 (7.0), then
    # the tie at 2.0 among blocks 1, 3, 4 goes to block 1
    np.testing.assert_array_equal(orc.select_blocks(scores, 0.5, sink=1, recent=0), [0, 1, 2])
    # importance order: decreasing score, ties to the lower index
    imp = orc.select_blocks(scores, 1.0, sink=0, recent=0, order=orc.SELECT_IMPORTANCE)
    np.testing.assert_array_equal(imp, [2, 1, 3, 4, 0, 5])


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force(seed):
    """Tiny T: the kept set is the forced blocks plus the best subset of the
    rest, found by trying every subset of the right size."""
    rng = np.random.default_rng(seed)
    T = int(rng.integers(3, 9))
    scores = np.round(rng.standard_normal(T), 1)  # ties happen
    frac = float(rng.choice([0.3, 0.5, 0.75, 1.0]))
    sink, recent = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    kept = set(orc.select_blocks(scores, frac, sink, recent).tolist())
    n_keep = orc.keep_count(T, frac)
    forced = set(range(min(sink, T, n_keep)))
    forced |= set(range(T - max(0, min(recent, n_keep - len(forced))), T))
    rest = [j for j in range(T) if j not in forced]
    m = n_keep - len(forced)
    best = None
    for sub in itertools.combinations(rest, m):
        key = sorted(((scores[j], -j) for j in sub), reverse=True)
        if best is None or key > best[0]:
            best = (key, set(sub))
    assert len(kept) == n_keep
    assert kept == forced | best[1]


def test_importance_order_is_sorted_and_complete():
    rng = np.random.default_rng(3)
    scores = rng.standard_normal(50)
    imp = orc.select_blocks(scores, 1.0, sink=1, recent=4, order=orc.SELECT_IMPORTANCE)
    assert sorted(imp.tolist()) == list(range(50))
    assert np.all(np.diff(scores[imp]) <= 0)


@pytest.mark.parametrize("frac,sink,recent", [(0.5, 1, 24), (0.25, 2, 8), (0.9, 1, 0), (1.0, 1, 24)])
def test_agrees_with_the_generators_selection(frac, sink, recent):
    """The workload generator implements the same rule separately (as the
    stand-in KV manager of the long-context configuration)."""
    from dataclasses import replace
    spec = replace(scaled(5, "B"), kept_frac=frac, kept_sink=sink, kept_recent=recent)
    w = make_workload(spec)
    kb, kc, _ = orc.select_workload(w, frac, sink, recent)
    for b in range(spec.batch):
        for h in range(spec.num_kv_heads):
            n = int(w.context_lens[b])
            G = spec.group
            from oracle import gather_unit
            Ks, _ = gather_unit(w.k, w.v, b, h, n, spec.page_size, w.block_table)
            ref = select_kept_blocks(spec, w.q[b, h * G:(h + 1) * G], Ks, n)
            np.testing.assert_array_equal(kb[b, h, :kc[b, h]], ref)
