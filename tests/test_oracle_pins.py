"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each test names what it pins and which plausible mistake it would catch.
Sources: ART paper section 3.1 Eq. (1) and section 3.2 (probe); the
gist.science explainer sections 2.2 (two metrics, dual threshold), 2.3
(patience) and 2.4 (traversal order, block 0, permutation invariance); the
FlexPrefill summary (restricted attention with a 0/-inf mask; Appendix A
error identity and bound).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
from workloads import make_workload, scaled, Spec

torch.set_num_threads(4)


def sdpa64(q, K, V, mask=None):
    """Library attention in float64 on the CPU (q [G,d], K/V [N,d])."""
    qt = torch.from_numpy(q)[None, :, None, :]            # [1, G, 1, d]
    Kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    m = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m)
    return o[0, :, 0].numpy()


def rand_unit(rng, G=4, d=128, n=1000, spread=1.0):
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d)) * spread
    V = rng.standard_normal((n, d))
    return q, K, V


# ---------------------------------------------------------------------------
# Eq. (1): full attention and restricted prefixes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("order", [orc.ORDER_NATURAL, orc.ORDER_RECENT_FIRST])
@pytest.mark.parametrize("G,d,n,bs", [(4, 128, 1000, 64), (1, 64, 1024, 64), (2, 64, 77, 16)])
def test_full_output_is_library_attention(order, G, d, n, bs):
    """O^(T') equals softmax(q K^T/sqrt(d)) V from torch's SDPA (fp64).

    Catches: wrong scale, dropped ragged-tail tokens, transposed operands,
    a wrong normalization."""
    rng = np.random.default_rng(11)
    q, K, V = rand_unit(rng, G, d, n)
    r = orc.art_unit(q, K, V, n, bs, 1e-3, 1e-4, 2, order, mode=orc.MODE_FULL)
    assert r.stop == r.num_traversal == (n + bs - 1) // bs
    ref = sdpa64(q, K, V)
    np.testing.assert_allclose(r.out, ref, rtol=1e-12, atol=1e-14)


def test_prefix_outputs_are_restricted_attention():
    """O^(t) equals attention over exactly the tokens of the first t blocks
    of the recency-first traversal [0, T-1, T-2, ...], written as a 0/-inf
    mask as in the FlexPrefill background definition.

    Catches: off-by-one prefixes, wrong traversal order, mixing blocks."""
    rng = np.random.default_rng(12)
    G, d, n, bs = 4, 128, 700, 64
    q, K, V = rand_unit(rng, G, d, n)
    r = orc.art_unit(q, K, V, n, bs, 1e-3, 1e-4, 2, orc.ORDER_RECENT_FIRST, mode=orc.MODE_FULL)
    T = (n + bs - 1) // bs
    pi = [0] + list(range(T - 1, 0, -1))            # written out here, independently
    for t in [1, 2, 3, 5, T - 1, T]:
        mask = np.full(n, -np.inf)
        for j in pi[:t]:
            mask[j * bs: min(n, (j + 1) * bs)] = 0.0
        ref = sdpa64(q, K, V, mask)
        np.testing.assert_allclose(r.O[t - 1], ref, rtol=1e-11, atol=1e-13)


def test_all_keys_equal_gives_mean_of_values_closed_form():
    """Equal keys => uniform weights => O^(t) = mean of the processed values.
    With blockwise-constant values (block j rows = u_j) this is
    sum_j n_j u_j / sum_j n_j over processed blocks, evaluated here in exact
    rational arithmetic, including a partial last block.

    Catches: weights not uniform, partial block counted as full, wrong
    prefix bookkeeping."""
    rng = np.random.default_rng(13)
    G, d, bs, n = 2, 16, 8, 8 * 6 - 3
    T = 6
    U = rng.integers(-9, 10, size=(T, d)).astype(np.float64)
    K = np.tile(rng.standard_normal(d), (n, 1))
    V = np.concatenate([np.tile(U[j], (min(bs, n - j * bs), 1)) for j in range(T)])
    q = rng.standard_normal((G, d))
    r = orc.art_unit(q, K, V, n, bs, 1e-3, 1e-4, 2, orc.ORDER_RECENT_FIRST, mode=orc.MODE_FULL)
    pi = [0, 5, 4, 3, 2, 1]
    counts = [min(bs, n - j * bs) for j in range(T)]
    for t in range(1, T + 1):
        num = [sum(Fraction(int(U[j, c])) * counts[j] for j in pi[:t]) for c in range(d)]
        den = sum(counts[j] for j in pi[:t])
        exact = np.array([float(x / den) for x in num])
        for g in range(G):
            np.testing.assert_allclose(r.O[t - 1, g], exact, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# probe and metrics: hand-computed values
# ---------------------------------------------------------------------------
def test_probe_takes_every_fourth_dim_of_each_head():
    """x^(t) = dims 0,4,8,... of head 0, then of head 1, ... (reading R5)."""
    O = np.arange(2 * 3 * 16, dtype=np.float64).reshape(2, 3, 16)
    x = orc.probe(O)
    assert x.shape == (2, 12)
    np.testing.assert_array_equal(x[1], [48, 52, 56, 60, 64, 68, 72, 76, 80, 84, 88, 92])


def test_metrics_hand_computed():
    """d_scale = |b-a|/a with the *previous* norm a; d_dir = 1 - cos.

    x1=(3,4) |5|; x2=(6,8) |10|: d_scale = 1 (would be 0.5 with the current
    norm as denominator), d_dir = 0.  x3=(8,6): d_scale = 0, cos = 0.96,
    d_dir = 0.04.  x4 = 1.0001*x3: d_scale = 1e-4, d_dir = 0.  x5 = 0:
    invalid (reading R11)."""
    x = np.array([[3.0, 4.0], [6.0, 8.0], [8.0, 6.0], [8.0008, 6.0006], [0.0, 0.0]])
    ds, dd, dds, valid = orc.stability_trace(x)
    assert np.isnan(ds[0]) and not valid[0]
    np.testing.assert_allclose(ds[1:4], [1.0, 0.0, 1e-4], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dd[1:4], [0.0, 0.04, 0.0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dds[1:4], [0.0, 0.04, 0.0], rtol=1e-12, atol=1e-15)
    assert list(valid) == [False, True, True, True, False]


def test_direction_forms_agree_on_real_traces():
    """1 - cos and 0.5*|x^_t - x^_{t-1}|^2 agree to 1e-12 in fp64."""
    w = make_workload(scaled(3, "B"))
    _, _, res = orc.art_decode_workload(w, mode=orc.MODE_FULL, keep_results=True)
    for r in res.values():
        m = r.valid
        np.testing.assert_allclose(r.d_dir[m], r.d_dir_stable[m], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# dual threshold + patience
# ---------------------------------------------------------------------------
def test_patience_counting_on_a_hand_trace():
    """Stable pattern over checks t=2..8: S S U S S S S.

    p=1 -> stops at t=2; p=2 -> t=3; p=3 -> t=7 (the unstable check resets
    the counter); p=4 -> t=8; p=5 -> runs to T'=8."""
    lo, hi = 1e-6, 1.0
    ds = np.array([np.nan, lo, lo, hi, lo, lo, lo, lo])
    dd = np.array([np.nan, lo, lo, lo, lo, lo, lo, lo])
    valid = np.array([False] + [True] * 7)
    got = [orc.stop_index(ds, dd, valid, 1e-3, 1e-4, p) for p in (1, 2, 3, 4, 5)]
    assert got == [2, 3, 7, 8, 8]
    # direction alone unstable also resets; both must hold
    dd2 = dd.copy(); dd2[2] = hi
    assert orc.stop_index(ds, dd2, valid, 1e-3, 1e-4, 2) == 6


def test_ablation_switches_on_a_hand_trace():
    """Checks t=2..8 where the scale test fails at t=4 and the direction test
    fails at t=6 (each alone).  Both metrics: p=2 stops at t=3; with p=3 the
    passing runs are {2,3}, {5}, {7,8}, so it runs to T'=8.  Scale test off:
    only t=6 fails, run {2..5} -> p=3 stops at t=4.  Direction test off: only
    t=4 fails, runs {2,3}, {5..8} -> stops at t=7.  Both off: every valid
    check passes -> stops at t=4; an invalid (zero) probe at t=3 still resets
    the counter -> stops at t=6."""
    lo, hi = 1e-6, 1.0
    ds = np.array([np.nan, lo, lo, hi, lo, lo, lo, lo])
    dd = np.array([np.nan, lo, lo, lo, lo, hi, lo, lo])
    valid = np.array([False] + [True] * 7)
    f = orc.stop_index
    assert f(ds, dd, valid, 1e-3, 1e-4, 2) == 3
    assert f(ds, dd, valid, 1e-3, 1e-4, 3) == 8
    assert f(ds, dd, valid, 1e-3, 1e-4, 3, flags=orc.FLAG_NO_SCALE) == 4
    assert f(ds, dd, valid, 1e-3, 1e-4, 3, flags=orc.FLAG_NO_DIR) == 7
    assert f(ds, dd, valid, 1e-3, 1e-4, 3, flags=orc.FLAG_NO_SCALE | orc.FLAG_NO_DIR) == 4
    # a zero-norm probe is still never stable with both tests off
    valid2 = valid.copy(); valid2[2] = False
    assert f(ds, dd, valid2, 1e-3, 1e-4, 3, flags=orc.FLAG_NO_SCALE | orc.FLAG_NO_DIR) == 6


def test_detect_only_reports_the_stop_and_attends_everywhere():
    w = make_workload(scaled(3, "B"))
    eps = dict(eps_scale=5e-2, eps_dir=5e-3)
    out_a, stop_a, _ = orc.art_decode_workload(w, **eps)
    out_d, stop_d, res = orc.art_decode_workload(w, flags=orc.FLAG_DETECT_ONLY, keep_results=True, **eps)
    np.testing.assert_array_equal(stop_d, stop_a)
    out_f, stop_f, _ = orc.art_decode_workload(w, mode=orc.MODE_FULL)
    for (b, h), r in res.items():
        np.testing.assert_array_equal(r.out, r.O[-1])
    # attending to every block is full decode, whatever was detected
    np.testing.assert_allclose(out_d, out_f, rtol=0, atol=1e-12)
    assert np.any(stop_a < stop_f), "the workload should fire somewhere"


def test_ablation_never_stops_later():
    """Taking a test out can only add passing checks."""
    w = make_workload(scaled(3, "B"))
    eps = dict(eps_scale=5e-2, eps_dir=5e-3)
    _, s_both, _ = orc.art_decode_workload(w, **eps)
    _, s_ns, _ = orc.art_decode_workload(w, flags=orc.FLAG_NO_SCALE, **eps)
    _, s_nd, _ = orc.art_decode_workload(w, flags=orc.FLAG_NO_DIR, **eps)
    assert np.all(s_ns <= s_both) and np.all(s_nd <= s_both)
    assert np.any(s_ns < s_both) or np.any(s_nd < s_both), "an ablation should change a stop"


def test_strict_comparison_at_threshold():
    """A metric exactly at its threshold is not stable (reading R3)."""
    tau = orc.threshold(1e-3)
    ds = np.array([np.nan, tau, tau])
    dd = np.array([np.nan, 0.0, 0.0])
    valid = np.array([False, True, True])
    assert orc.stop_index(ds, dd, valid, 1e-3, 1e-4, 1) == 3
    ds2 = np.array([np.nan, np.nextafter(tau, 0), tau])
    assert orc.stop_index(ds2, dd, valid, 1e-3, 1e-4, 1) == 2


def test_eps_zero_never_stops():
    w = make_workload(scaled(3, "B"))
    _, stop, _ = orc.art_decode_workload(w, eps_scale=0.0, eps_dir=0.0)
    np.testing.assert_array_equal(stop, w.traversal_lengths())


@pytest.mark.parametrize("p", [1, 2, 3])
def test_huge_eps_stops_after_p_plus_one_blocks(p):
    w = make_workload(scaled(3, "A"))
    _, stop, _ = orc.art_decode_workload(w, eps_scale=1e30, eps_dir=1e30, patience=p)
    np.testing.assert_array_equal(stop, np.minimum(w.traversal_lengths(), p + 1))


@pytest.mark.parametrize("p", [1, 2, 4])
def test_identical_value_rows_stop_after_p_plus_one(p):
    """All value rows equal => O^(t) constant => both metrics 0 => stop p+1."""
    rng = np.random.default_rng(14)
    q, K, _ = rand_unit(rng, 4, 128, 900)
    V = np.tile(rng.standard_normal(128), (900, 1))
    r = orc.art_unit(q, K, V, 900, 64, 1e-3, 1e-4, p)
    assert r.stop == p + 1
    np.testing.assert_allclose(r.out[0], V[0], rtol=1e-13)


def test_stop_monotone_in_eps_and_patience():
    """The set of passing checks grows with eps, so stop_idx cannot rise;
    a longer patience cannot stop earlier."""
    w = make_workload(scaled(3, "B"))
    _, _, res = orc.art_decode_workload(w, mode=orc.MODE_FULL, keep_results=True)
    for r in res.values():
        prev = None
        for e in [1e-5, 1e-4, 5e-4, 1e-3, 2e-3, 1e-2, 1e-1]:
            s = orc.stop_index(r.d_scale, r.d_dir, r.valid, e, e / 10, 2)
            assert prev is None or s <= prev
            prev = s
        stops = [orc.stop_index(r.d_scale, r.d_dir, r.valid, 2e-3, 2e-4, p) for p in (1, 2, 3, 4, 6)]
        assert stops == sorted(stops)
        assert all(min(r.num_traversal, p + 1) <= s <= r.num_traversal for p, s in zip((1, 2, 3, 4, 6), stops))


# ---------------------------------------------------------------------------
# traversal order, block 0, permutation invariance
# ---------------------------------------------------------------------------
def test_traversal_orders():
    assert orc.traversal(5, None, orc.ORDER_NATURAL) == [0, 1, 2, 3, 4]
    assert orc.traversal(5, None, orc.ORDER_RECENT_FIRST) == [0, 4, 3, 2, 1]
    assert orc.traversal(6, [1, 3, 5], orc.ORDER_RECENT_FIRST) == [5, 3, 1]
    assert orc.traversal(6, [0, 3, 5], orc.ORDER_RECENT_FIRST) == [0, 5, 3]
    assert orc.traversal(6, [3, 0, 5, 1], orc.ORDER_GIVEN) == [0, 3, 5, 1]
    assert orc.traversal(6, [3, 5, 1], orc.ORDER_GIVEN) == [3, 5, 1]
    assert orc.traversal(1, None, orc.ORDER_RECENT_FIRST) == [0]
    assert orc.traversal(0, None, orc.ORDER_RECENT_FIRST) == []


def test_permutation_invariance_of_full_output():
    """Reordering blocks adds no error: O^(T') agrees across orders."""
    rng = np.random.default_rng(15)
    q, K, V = rand_unit(rng, 4, 128, 1300)
    T = (1300 + 63) // 64
    outs = [orc.art_unit(q, K, V, 1300, 64, 0, 0, 1, o, mode=orc.MODE_FULL).out
            for o in (orc.ORDER_NATURAL, orc.ORDER_RECENT_FIRST)]
    perm = list(rng.permutation(T))
    outs.append(orc.art_unit(q, K, V, 1300, 64, 0, 0, 1, orc.ORDER_GIVEN, kept=perm, mode=orc.MODE_FULL).out)
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-12, atol=1e-14)


def test_kept_list_restricts_to_kept_tokens():
    """With a kept list, O^(T') is attention over the kept blocks' tokens."""
    rng = np.random.default_rng(16)
    n, bs = 1000, 64
    q, K, V = rand_unit(rng, 4, 128, n)
    kept = [0, 2, 3, 7, 15]
    r = orc.art_unit(q, K, V, n, bs, 1e-3, 1e-4, 2, orc.ORDER_RECENT_FIRST, kept=kept, mode=orc.MODE_FULL)
    assert r.order_blocks == [0, 15, 7, 3, 2] and r.num_traversal == 5
    mask = np.full(n, -np.inf)
    for j in kept:
        mask[j * bs: min(n, (j + 1) * bs)] = 0
    np.testing.assert_allclose(r.out, sdpa64(q, K, V, mask), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# FlexPrefill Appendix A: exact identity and bound for a truncated set
# ---------------------------------------------------------------------------
def test_truncation_error_identity_and_bound():
    """O_full - O_S = (1 - a_S)(O_{S^c} - O_S) and
    |O_full - O_S| <= (1 - a_S) * sum_j |v_j|, where a_S is the softmax mass
    of the processed tokens; checked at every prefix."""
    rng = np.random.default_rng(17)
    n, bs = 900, 64
    q, K, V = rand_unit(rng, 4, 128, n, spread=1.5)
    r = orc.art_unit(q, K, V, n, bs, 1e-3, 1e-4, 2, mode=orc.MODE_FULL)
    full = r.O[-1]
    vnorm_sum = np.linalg.norm(V, axis=1).sum()
    cum_mass = np.cumsum(r.mass, axis=0)
    for t in range(1, r.num_traversal):
        aS = cum_mass[t - 1]                                   # [G]
        rest = np.ones(n, dtype=bool)
        for j in r.order_blocks[:t]:
            rest[j * bs: min(n, (j + 1) * bs)] = False
        mask = np.where(rest, 0.0, -np.inf)
        O_rest = sdpa64(q, K, V, mask)
        lhs = full - r.O[t - 1]
        rhs = (1 - aS)[:, None] * (O_rest - r.O[t - 1])
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-13)
        assert np.all(np.linalg.norm(lhs, axis=1) <= (1 - aS) * vnorm_sum + 1e-12)


# ---------------------------------------------------------------------------
# brute force on tiny inputs (pure Python loops, independent structure)
# ---------------------------------------------------------------------------
def brute_art(q, K, V, n, bs, eps_s, eps_d, p, order_blocks):
    d = len(q[0])
    tau, phi = float(np.float32(eps_s)), float(np.float32(eps_d))
    xs, outs = [], []
    toks = []
    for j in order_blocks:
        toks += list(range(j * bs, min(n, (j + 1) * bs)))
        # direct softmax over the processed tokens, one head at a time
        o_heads = []
        for qg in q:
            s = [sum(qg[c] * K[i][c] for c in range(d)) / math.sqrt(d) for i in toks]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            o_heads.append([sum(e[k] * V[i][c] for k, i in enumerate(toks)) / z for c in range(d)])
        outs.append(o_heads)
        xs.append([o[c] for o in o_heads for c in range(0, d, 4)])
    count = 0
    for t in range(1, len(xs)):
        a = math.sqrt(sum(v * v for v in xs[t - 1]))
        b = math.sqrt(sum(v * v for v in xs[t]))
        ok = False
        if a > 0 and b > 0:
            cos = sum(u * v for u, v in zip(xs[t], xs[t - 1])) / (a * b)
            ok = abs(b - a) / a < tau and 1 - cos < phi
        count = count + 1 if ok else 0
        if count >= p:
            return t + 1, outs[t]
    return len(xs), outs[-1]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    G, d, bs, n = 2, 8, 3, 20
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d)) * 0.3
    V = np.tile(rng.standard_normal(d), (n, 1)) + 0.02 * rng.standard_normal((n, d))
    for eps in [(0.05, 0.01), (0.02, 0.002), (1e-3, 1e-4)]:
        for p in (1, 2):
            r = orc.art_unit(q, K, V, n, bs, eps[0], eps[1], p, orc.ORDER_RECENT_FIRST)
            T = (n + bs - 1) // bs
            st, out = brute_art(q.tolist(), K.tolist(), V.tolist(), n, bs, eps[0], eps[1], p,
                                [0] + list(range(T - 1, 0, -1)))
            assert r.stop == st
            np.testing.assert_allclose(r.out, np.array(out), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# layouts: paged gather equals contiguous
# ---------------------------------------------------------------------------
def test_paged_and_contiguous_layouts_agree():
    base = scaled(3, "B")
    lens = np.array([700, 1333, 64, 2049], dtype=np.int32)
    wp = make_workload(base, context_lens=lens)
    from dataclasses import replace
    wc = make_workload(replace(base, page_size=0), context_lens=lens)
    op, sp, _ = orc.art_decode_workload(wp)
    oc, sc, _ = orc.art_decode_workload(wc)
    np.testing.assert_array_equal(sp, sc)
    np.testing.assert_array_equal(op, oc)
    assert not np.isnan(op).any()


def test_empty_sequence_gives_zero_blocks():
    r = orc.art_unit(np.ones((2, 8)), np.zeros((0, 8)), np.zeros((0, 8)), 0, 4, 1e-3, 1e-4, 1)
    assert r.stop == 0 and r.num_traversal == 0
    np.testing.assert_array_equal(r.out, 0.0)


# ---------------------------------------------------------------------------
# hand-derived worked example (tests/golden/worked_example_equal_keys.json)
# ---------------------------------------------------------------------------
def test_hand_derived_worked_example():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example_equal_keys.json")
    ex = json.load(open(path))
    st = ex["setup"]
    n, d, bs = st["n_ctx"], st["d"], st["block_size"]
    V = np.concatenate([np.tile(np.array(st["values_by_block"][str(j)], dtype=np.float64),
                                (st["tokens_per_block"][str(j)], 1)) for j in range(4)])
    K = np.ones((n, d))
    q = np.array([[0.3, -1.0, 2.0, 0.5, 0.1, 0.0, -0.7, 1.1]])
    ev = {"sqrt": math.sqrt}
    for case in ex["stops"]:
        r = orc.art_unit(q, K, V, n, bs, case["eps_scale"], case["eps_dir"], case["patience"])
        assert r.order_blocks == ex["traversal"]
        np.testing.assert_allclose(orc.probe(r.O), np.array(ex["probe"], dtype=np.float64), rtol=1e-14, atol=1e-14)
        for t in range(1, 4):
            assert r.d_scale[t] == pytest.approx(eval(ex["d_scale"][t], ev), rel=1e-12, abs=1e-15)
            assert r.d_dir[t] == pytest.approx(eval(ex["d_dir"][t], ev), rel=1e-10, abs=1e-15)
        assert r.stop == case["stop"], case


# ---------------------------------------------------------------------------
# multi-row queries (R28)
# ---------------------------------------------------------------------------
def _rows_case(M, seed=21):
    rng = np.random.default_rng(seed)
    B, Hkv, G, d, n = 2, 2, 2, 64, 700
    q = rng.standard_normal((B, M, Hkv * G, d))
    k = rng.standard_normal((B, Hkv, n, d))
    v = rng.standard_normal((B, Hkv, n, d))
    lens = np.array([700, 455], dtype=np.int32)
    return q, k, v, lens, Hkv


def _rows(q, k, v, lens, Hkv, **kw):
    return orc.art_decode_rows(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), lens, "f32", Hkv,
                               64, kw.get("es", 5e-2), kw.get("ed", 5e-3), 2, orc.ORDER_RECENT_FIRST, orc.MODE_ART)


def test_rows_identical_rows_change_nothing():
    """M identical rows: the concatenated probe is the single-row probe
    repeated, so both metrics (ratios of norms and a cosine) and the stop are
    those of one row, and every row's output is the one-row output."""
    q, k, v, lens, Hkv = _rows_case(1)
    out1, stop1, _ = _rows(q, k, v, lens, Hkv)
    q3 = np.repeat(q, 3, axis=1)
    out3, stop3, _ = _rows(q3, k, v, lens, Hkv)
    np.testing.assert_array_equal(stop3, stop1)
    for i in range(3):
        np.testing.assert_allclose(out3[:, i], out1[:, 0], rtol=1e-12, atol=1e-14)


def test_rows_permutation_invariance():
    """Permuting the rows permutes the outputs and keeps the stop: norms and
    dot products of the concatenated probe do not depend on its order."""
    q, k, v, lens, Hkv = _rows_case(3)
    out, stop, _ = _rows(q, k, v, lens, Hkv)
    perm = [2, 0, 1]
    outp, stopp, _ = _rows(q[:, perm], k, v, lens, Hkv)
    np.testing.assert_array_equal(stopp, stop)
    np.testing.assert_allclose(outp, out[:, perm], rtol=1e-12, atol=1e-14)


def test_rows_full_mode_is_per_row_attention():
    """Full mode: every row's output is plain softmax attention of that row
    over the whole context (a library routine, row by row)."""
    q, k, v, lens, Hkv = _rows_case(2)
    out, stop, _ = orc.art_decode_rows(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), lens, "f32",
                                       Hkv, 64, 1e-3, 1e-4, 2, orc.ORDER_RECENT_FIRST, orc.MODE_FULL)
    G = q.shape[2] // Hkv
    for b in range(2):
        n = int(lens[b])
        for i in range(2):
            for hq in range(q.shape[2]):
                h = hq // G
                qq = q[b, i, hq].astype(np.float32).astype(np.float64)
                K = k[b, h, :n].astype(np.float32).astype(np.float64)
                V = v[b, h, :n].astype(np.float32).astype(np.float64)
                ref = sdpa64(qq[None], K, V, np.zeros(n))[0]
                np.testing.assert_allclose(out[b, i, hq], ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# the parity rule's margin, the exact widening of stored inputs, kept lists
# ---------------------------------------------------------------------------
def test_relative_margin_hand_values():
    """Pins relative_margin, which excuses a stop mismatch when a metric sits
    within a relative 1e-4 of its threshold: |d / eps - 1|, eps as the
    float32 the C ABI carries.  An absolute band |d - eps| would give about
    1e-8 for d = 1.0001 eps and so excuse nearly every check; a margin on
    the wrong side (eps / d) or without the absolute value fails the values
    below."""
    for eps in (1e-4, 2e-4, 1e-3, 2e-3, 5e-2):
        e = float(np.float32(eps))
        m = orc.relative_margin(np.array([1.0001 * e, e, 0.5 * e, 3.0 * e, 0.9999 * e, np.nan]), eps)
        assert abs(m[0] - 1e-4) < 1e-12
        assert m[1] == 0.0
        assert abs(m[2] - 0.5) < 1e-15 and abs(m[3] - 2.0) < 1e-15
        assert abs(m[4] - 1e-4) < 1e-12
        assert np.isnan(m[5])
    # a check 2e-4 above eps_dir = 1e-4 in absolute terms is far (margin 2), not near
    assert orc.relative_margin(np.array([3e-4]), 1e-4)[0] > 1.9


def test_widen_bf16_bit_patterns():
    """Pins widen: bf16 bit patterns are the upper halves of float32 (sign,
    8 exponent bits, 7 mantissa bits), widened exactly; float32 inputs are
    widened exactly."""
    table = {
        0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x3E80: 0.25, 0x0000: 0.0,
        0x7F80: math.inf, 0xFF80: -math.inf,
        0x0001: 2.0 ** -133,            # smallest subnormal
        0x007F: 127 * 2.0 ** -133,      # largest subnormal
        0x0080: 2.0 ** -126,            # smallest normal
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
    }
    bits = np.array(list(table), dtype=np.uint16)
    got = orc.widen(bits, "bf16")
    assert got.dtype == np.float64
    for b, v in zip(table, got):
        assert v == table[b], hex(b)
    neg0 = orc.widen(np.array([0x8000], dtype=np.uint16), "bf16")[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    assert np.isnan(orc.widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")).all()
    f = np.array([0.1, -3.5, 1e-40], dtype=np.float32)
    assert [float(x) for x in orc.widen(f, "f32")] == [float(x) for x in f]


def test_kept_lists_must_be_distinct_blocks_of_the_sequence():
    """A kept list is a set of the sequence's blocks: repeats and blocks
    outside the sequence are refused, in every order."""
    for order in (orc.ORDER_NATURAL, orc.ORDER_RECENT_FIRST, orc.ORDER_GIVEN):
        with pytest.raises(ValueError):
            orc.traversal(10, [1, 3, 3], order)
        with pytest.raises(ValueError):
            orc.traversal(10, [1, 10], order)
        with pytest.raises(ValueError):
            orc.traversal(10, [-1, 2], order)
        assert sorted(orc.traversal(10, [7, 0, 3], order)) == [0, 3, 7]
