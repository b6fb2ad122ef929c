"""The per-unit acceptance rule (oracle.acceptance) on hand-made cases: what
it accepts and what it rejects, so that a loosened rule fails here."""
import numpy as np

import oracle as orc
from oracle.acceptance import MARGIN, MAX_ABS, REL_L2, unit_agreement


def _unit(seed=3, n=64 * 12, G=2, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    return orc.art_unit(q, K, V, n, 64, 1e-3, 1e-4, 2)


def test_exact_result_is_accepted():
    r = _unit()
    a = unit_agreement(r, r.out, r.stop, 1e-3, 1e-4)
    assert a.ok and a.stop_equal and not a.excused and a.rel_l2 == 0 and a.max_abs == 0


def test_output_is_compared_at_the_implementations_stop():
    r = _unit()
    s = r.stop - 1 if r.stop > 1 else r.stop + 1
    # the implementation's output at its own (different) stop is O^(s)
    a = unit_agreement(r, r.O[s - 1], s, 1e-3, 1e-4)
    assert a.output_ok and not a.stop_equal
    # the oracle's own output does not match O^(s)
    b = unit_agreement(r, r.out, s, 1e-3, 1e-4)
    assert not b.output_ok


def test_stop_difference_far_from_thresholds_is_not_excused():
    r = _unit()
    s = r.stop - 1 if r.stop > 1 else r.stop + 1
    a = unit_agreement(r, r.O[s - 1], s, 1e-3, 1e-4)
    assert a.margin > MARGIN and not a.excused and not a.ok


def test_stop_difference_at_a_threshold_is_excused():
    r = _unit()
    s = r.stop - 1 if r.stop > 1 else r.stop + 1
    # put eps_scale exactly on one of the checks' metrics: margin 0 there
    t = 1
    eps = float(r.d_scale[t])
    a = unit_agreement(r, r.O[s - 1], s, eps, 1e-4)
    assert a.margin <= MARGIN and a.excused and a.ok
    # with the scale test switched off, only the direction test can excuse
    b = unit_agreement(r, r.O[s - 1], s, eps, 1e-4, flags=orc.FLAG_NO_SCALE)
    assert not b.excused


def test_tolerances():
    r = _unit()
    ref = r.O[r.stop - 1]
    bump = np.zeros_like(ref)
    bump[0, 0] = MAX_ABS * 1.5
    assert not unit_agreement(r, ref + bump, r.stop, 1e-3, 1e-4).output_ok
    scaled = ref * (1 + 0.5 * REL_L2)
    a = unit_agreement(r, scaled, r.stop, 1e-3, 1e-4)
    assert a.rel_l2 <= REL_L2 and (a.max_abs > MAX_ABS) == (np.abs(ref).max() * 0.5 * REL_L2 > MAX_ABS)
    assert not unit_agreement(r, ref * (1 + 2 * REL_L2), r.stop, 1e-3, 1e-4).output_ok
    nan = ref.copy()
    nan[0, 0] = np.nan
    assert not unit_agreement(r, nan, r.stop, 1e-3, 1e-4).output_ok


def test_stop_out_of_range_is_rejected():
    r = _unit()
    for s in (0, r.num_traversal + 1, -1):
        a = unit_agreement(r, r.out, s, 1e-3, 1e-4)
        assert not a.stop_in_range and not a.ok


def test_detect_only_compares_with_every_block():
    r = orc.art_unit(*[np.random.default_rng(5).standard_normal(s) for s in ((2, 16), (640, 16), (640, 16))],
                     640, 64, 1e-3, 1e-4, 2, flags=orc.FLAG_DETECT_ONLY)
    a = unit_agreement(r, r.O[-1], r.stop, 1e-3, 1e-4, flags=orc.FLAG_DETECT_ONLY)
    assert a.ok
    if r.stop < r.num_traversal:
        assert not unit_agreement(r, r.O[r.stop - 1], r.stop, 1e-3, 1e-4, flags=orc.FLAG_DETECT_ONLY).output_ok
