"""GPU parity over seeded random combinations of the call's options.

The other GPU tests take one option at a time; here every case draws the
element type, head geometry, ragged lengths, layout and page size, kept
lists, traversal order, generator, thresholds, patience, mode, chunking,
stop-rule switches and wave count together, and checks every unit against
the fp64 oracle with the same acceptance rule (stop equal or margin-excused;
output against the oracle's O^(stop)).  Sizes are small so that the oracle
finishes in a second or two per case.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle as orc
from tests.parity import compare, log, run_gpu
from workloads import config, make_workload

pytestmark = pytest.mark.gpu

CASES = 32


def draw_case(seed):
    """The options of one case (all from numpy's generator with `seed`)."""
    rng = np.random.default_rng([20251203, seed])
    f32 = rng.random() < 0.25
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4]))
    lo = int(rng.integers(1, 2500))
    hi = int(rng.integers(lo, 3200))
    kept = (not f32) and rng.random() < 0.3
    spec = replace(config(3), name=f"random-{seed}", batch=int(rng.integers(1, 4)), num_q_heads=hkv * g,
                   num_kv_heads=hkv, head_dim=64 if f32 else 128, dtype="f32" if f32 else "bf16", ctx=(lo, hi),
                   page_size=int(rng.choice([0, 16, 32, 64])) if not kept else 16,
                   reading=str(rng.choice(["A", "B"])), eps_scale=float(rng.choice([1e-3, 2e-3, 1e-2, 5e-2])),
                   eps_dir=float(rng.choice([1e-4, 2e-4, 1e-3, 1e-2])), patience=int(rng.integers(1, 5)),
                   order=int(rng.choice([orc.ORDER_NATURAL, orc.ORDER_RECENT_FIRST])),
                   kept_frac=0.5 if kept else 0.0, kept_recent=int(rng.integers(2, 9)), seed=seed + 100)
    mode = 0 if rng.random() < 0.2 else 1
    split = int(rng.choice([0, 4, 8, 12, 16, 20, 24, 1 << 20]))
    flags = 0
    if mode == 1 and rng.random() < 0.3:
        flags = int(rng.choice([orc.FLAG_NO_SCALE, orc.FLAG_NO_DIR, orc.FLAG_DETECT_ONLY]))
    # eight waves apply to ART mode with one work item per unit
    waves = 8 if (mode == 1 and split == 1 << 20 and rng.random() < 0.5) else 0
    return spec, mode, split, flags, waves


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("seed", range(CASES))
def test_random_combination(torch_cuda, seed):
    spec, mode, split, flags, waves = draw_case(seed)
    w = make_workload(spec)
    log(f"[case] seed={seed} {spec} mode={mode} split={split} flags={flags} waves={waves}")
    out, stop, issued, err = run_gpu(w, mode=mode, split_blocks=split, flags=flags, waves=waves)
    assert err == 0, f"device error {err}"
    rep, _ = compare(w, out, stop, mode=mode, flags=flags)
    log(f"   {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    assert rep.excused <= -(-rep.units // 100), str(rep)
    tp = w.traversal_lengths()
    assert np.all(stop <= tp) and np.all(issued >= np.minimum(stop, tp)), "stop or blocks_issued out of range"
    if mode == 0 or flags == orc.FLAG_DETECT_ONLY:
        assert np.all(issued >= tp), "full decode and detect-only read every block"
