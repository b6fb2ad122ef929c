"""GPU parity over seeded random combinations of the call's options.

The other GPU tests take one option at a time; here every case draws the
element type, head geometry, ragged lengths, layout and page size, kept
lists (the generator's, or a caller-given traversal), traversal order,
generator, thresholds, patience, mode, chunking, stop-rule switches, wave
count and query rows per unit together, and checks every unit against
the fp64 oracle with the same acceptance rule (stop equal or margin-excused;
output against the oracle's O^(stop)).  Sizes are small so that the oracle
finishes in a second or two per case.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle as orc
from tests.parity import compare, log, run_gpu
from workloads import config, make_workload, multi_row_queries

pytestmark = pytest.mark.gpu

CASES = 96


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
    # query rows per unit, and a caller-given traversal (a kept list in the
    # caller's order) where the generator made no kept list
    rows = 1 if rng.random() < 0.7 else int(rng.choice([2, 4]))
    given = (not kept) and rng.random() < 0.15
    if g * rows > 4:  # split ART and eight waves take at most 4 query vectors per unit
        waves = 0
        if mode == 1 and split not in (0, 1 << 20):
            split = 1 << 20
    return spec, mode, split, flags, waves, rows, given


def given_lists(w, seed):
    """A distinct random subset of each unit's blocks in random order (block 0
    may be absent, or anywhere in the list)."""
    rng = np.random.default_rng([20251203, seed, 1])
    s = w.spec
    T = w.num_blocks
    kb = np.full((s.batch, s.num_kv_heads, max(1, int(T.max()))), -1, dtype=np.int32)
    kc = np.zeros((s.batch, s.num_kv_heads), dtype=np.int32)
    for b in range(s.batch):
        for h in range(s.num_kv_heads):
            if T[b] == 0:
                continue
            n = int(rng.integers(1, T[b] + 1))
            kb[b, h, :n] = rng.choice(T[b], size=n, replace=False)
            kc[b, h] = n
    w.kept_blocks, w.kept_count = kb, kc


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("seed", range(CASES))
def test_random_combination(torch_cuda, seed):
    spec, mode, split, flags, waves, rows, given = draw_case(seed)
    w = make_workload(spec)
    order = spec.order
    if given:
        given_lists(w, seed)
        order = orc.ORDER_GIVEN
    qr = qd = None
    if rows > 1:
        qr = multi_row_queries(w, rows)
        qd = torch_cuda.from_numpy(qr.view(np.int16) if qr.dtype == np.uint16 else qr).to("cuda")
    log(f"[case] seed={seed} {spec} mode={mode} split={split} flags={flags} waves={waves} rows={rows} "
        f"given={given}")
    out, stop, issued, err = run_gpu(w, mode=mode, split_blocks=split, flags=flags, waves=waves, order=order, q=qd)
    assert err == 0, f"device error {err}"
    rep, _ = compare(w, out, stop, mode=mode, flags=flags, order=order, q_rows=qr)
    log(f"   {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    assert rep.excused <= -(-rep.units // 100), str(rep)
    tp = w.traversal_lengths()
    assert np.all(stop <= tp) and np.all(issued >= np.minimum(stop, tp)), "stop or blocks_issued out of range"
    if mode == 0 or flags == orc.FLAG_DETECT_ONLY:
        assert np.all(issued >= tp), "full decode and detect-only read every block"
