"""Planted mistakes in the oracle (on the CPU) must each fail some pin.

Every mutation below is a plausible slip when writing ART from its
description: a wrong denominator in the scale metric, a sign slip in the
direction metric, a non-strict threshold, a contiguous probe slice, block 0
not forced first, a dropped 1/sqrt(d), a patience off by one, a prefix off by
one, a dropped ragged tail, an absolute instead of a relative margin band
(or one taken the wrong way round), a mis-shifted bf16 widening, a kept list
whose repeats are accepted.  The test patches the oracle module in place,
runs the pin functions, and requires at least one of them to fail.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.art_oracle as ao
from tests import test_oracle_pins as pins


class _Patch:
    """Patch a name in the oracle module and in the package namespace."""

    def __init__(self, mp):
        self.mp = mp

    def setattr(self, mod, name, value):
        self.mp.setattr(ao, name, value)
        if hasattr(oracle, name):
            self.mp.setattr(oracle, name, value)


def _run_pins():
    """Run the pins once; return the names of those that failed."""
    failed = []
    cases = [
        (pins.test_full_output_is_library_attention, dict(order=ao.ORDER_RECENT_FIRST, G=2, d=64, n=77, bs=16)),
        (pins.test_prefix_outputs_are_restricted_attention, {}),
        (pins.test_all_keys_equal_gives_mean_of_values_closed_form, {}),
        (pins.test_probe_takes_every_fourth_dim_of_each_head, {}),
        (pins.test_metrics_hand_computed, {}),
        (pins.test_patience_counting_on_a_hand_trace, {}),
        (pins.test_strict_comparison_at_threshold, {}),
        (pins.test_huge_eps_stops_after_p_plus_one_blocks, dict(p=2)),
        (pins.test_identical_value_rows_stop_after_p_plus_one, dict(p=2)),
        (pins.test_traversal_orders, {}),
        (pins.test_kept_list_restricts_to_kept_tokens, {}),
        (pins.test_brute_force_tiny, dict(seed=0)),
        (pins.test_hand_derived_worked_example, {}),
        (pins.test_relative_margin_hand_values, {}),
        (pins.test_widen_bf16_bit_patterns, {}),
        (pins.test_kept_lists_must_be_distinct_blocks_of_the_sequence, {}),
    ]
    for fn, kw in cases:
        try:
            fn(**kw)
        except (Exception, pytest.fail.Exception):  # noqa: BLE001 - any failure counts
            failed.append(fn.__name__)
    return failed


def _mut_scale_denominator(mp):
    orig = ao.stability_trace

    def bad(x):
        ds, dd, dds, v = orig(x)
        T = x.shape[0]
        for t in range(1, T):
            a, b = np.linalg.norm(x[t - 1]), np.linalg.norm(x[t])
            if v[t]:
                ds[t] = abs(b - a) / b
        return ds, dd, dds, v
    mp.setattr(ao, "stability_trace", bad)


def _mut_dir_sign(mp):
    orig = ao.stability_trace

    def bad(x):
        ds, dd, dds, v = orig(x)
        return ds, 2.0 - dd, 2.0 - dds, v
    mp.setattr(ao, "stability_trace", bad)


def _mut_nonstrict(mp):
    def bad(ds, dd, valid, es, ed, p, mode=ao.MODE_ART):
        T = len(ds)
        if mode == ao.MODE_FULL or T == 0:
            return T
        c = 0
        for t in range(1, T):
            st = bool(valid[t]) and ds[t] <= ao.threshold(es) and dd[t] <= ao.threshold(ed)
            c = c + 1 if st else 0
            if c >= p:
                return t + 1
        return T
    mp.setattr(ao, "stop_index", bad)


def _mut_contiguous_probe(mp):
    def bad(O):
        T, G, d = O.shape
        return O[:, :, : d // 4].reshape(T, -1)
    mp.setattr(ao, "probe", bad)


def _mut_block0_not_first(mp):
    def bad(nb, kept=None, order=ao.ORDER_RECENT_FIRST):
        cand = list(range(nb)) if kept is None else [int(c) for c in kept]
        if order == ao.ORDER_NATURAL:
            return sorted(cand)
        if order == ao.ORDER_RECENT_FIRST:
            return sorted(cand, reverse=True)
        return cand
    mp.setattr(ao, "traversal", bad)


def _mut_no_scale(mp):
    orig = ao.prefix_outputs

    def bad(q, K, V, n, blocks, bs):
        return orig(q * math.sqrt(q.shape[1]), K, V, n, blocks, bs)
    mp.setattr(ao, "prefix_outputs", bad)


def _mut_patience_off_by_one(mp):
    orig = ao.stop_index

    def bad(ds, dd, valid, es, ed, p, mode=ao.MODE_ART):
        return orig(ds, dd, valid, es, ed, p + 1, mode)
    mp.setattr(ao, "stop_index", bad)


def _mut_prefix_off_by_one(mp):
    orig = ao.prefix_outputs

    def bad(q, K, V, n, blocks, bs):
        O, m = orig(q, K, V, n, blocks, bs)
        if len(O) > 1:
            O = np.concatenate([O[1:], O[-1:]])
        return O, m
    mp.setattr(ao, "prefix_outputs", bad)


def _mut_drop_ragged_tail(mp):
    def bad(j, n, bs):
        hi = (j + 1) * bs
        return np.arange(j * bs, hi) if hi <= n else np.arange(0)
    mp.setattr(ao, "block_tokens", bad)


def _mut_absolute_margin(mp):
    def bad(d, eps):
        with np.errstate(invalid="ignore"):
            return np.abs(np.asarray(d) - ao.threshold(eps))
    mp.setattr(ao, "relative_margin", bad)


def _mut_margin_inverted(mp):
    def bad(d, eps):
        with np.errstate(invalid="ignore", divide="ignore"):
            return np.abs(ao.threshold(eps) / np.asarray(d) - 1.0)
    mp.setattr(ao, "relative_margin", bad)


def _mut_widen_mantissa_shift(mp):
    def bad(arr, dtype):
        if dtype == "bf16":
            bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 15
            return bits.view(np.float32).astype(np.float64)
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    mp.setattr(ao, "widen", bad)


def _mut_kept_duplicates_accepted(mp):
    def bad(nb, kept=None, order=ao.ORDER_RECENT_FIRST):
        cand = list(range(nb)) if kept is None else [int(c) for c in kept]
        head = [0] if 0 in cand else []
        rest = [c for c in cand if c != 0]
        if order == ao.ORDER_NATURAL:
            rest = sorted(rest)
        elif order == ao.ORDER_RECENT_FIRST:
            rest = sorted(rest, reverse=True)
        return head + rest
    mp.setattr(ao, "traversal", bad)


MUTATIONS = {
    "absolute margin band": _mut_absolute_margin,
    "margin inverted (eps / d)": _mut_margin_inverted,
    "bf16 widened with a 15-bit shift": _mut_widen_mantissa_shift,
    "kept list repeats accepted": _mut_kept_duplicates_accepted,
    "scale-metric uses current norm": _mut_scale_denominator,
    "direction metric sign slip": _mut_dir_sign,
    "non-strict thresholds": _mut_nonstrict,
    "contiguous probe slice": _mut_contiguous_probe,
    "block 0 not forced first": _mut_block0_not_first,
    "missing 1/sqrt(d)": _mut_no_scale,
    "patience off by one": _mut_patience_off_by_one,
    "prefix off by one": _mut_prefix_off_by_one,
    "ragged tail dropped": _mut_drop_ragged_tail,
}


def test_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_each_planted_mistake_fails_a_pin(name, monkeypatch):
    MUTATIONS[name](_Patch(monkeypatch))
    failed = _run_pins()
    assert failed, f"no pin caught the planted mistake: {name}"
