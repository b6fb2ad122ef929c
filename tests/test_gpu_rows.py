"""GPU parity for multi-row queries (q [B, M, Hq, d]) against the oracle.

The M * G query vectors of a unit share its traversal and one stop; the
cases span 4 query vectors per unit (the repeated-column layout), 8 and 16
(one MFMA column and one output row per vector), full mode with split-KV
chunks, kept lists, and both dtypes.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle as orc
from tests.parity import compare, log, run_gpu
from workloads import make_workload, multi_row_queries, scaled
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _spec(case):
    if case == "bf16 G4 paged":
        return scaled(3, "B")
    if case == "bf16 G4 contiguous":
        return scaled(2, "B")
    if case == "bf16 G2 paged":
        return replace(scaled(3, "B"), num_q_heads=4)
    if case == "fp32 G1":
        return scaled(1, "B")
    if case == "bf16 G4 kept list":
        return scaled(5, "B")
    raise ValueError(case)


def _run(case, rows, mode, **kw):
    import torch
    w = make_workload(_spec(case))
    qr = multi_row_queries(w, rows)
    dev = to_device(w)
    qd = torch.from_numpy(qr.view(np.int16) if qr.dtype == np.uint16 else qr).to("cuda")
    log(f"[case] rows={rows} {case} mode={mode} {kw}")
    out, stop, issued, err = run_gpu(w, mode=mode, dev=dev, q=qd, **kw)
    assert err == 0, f"device error {err}"
    ckw = {k: v for k, v in kw.items() if k in ("patience", "eps_scale", "eps_dir", "order", "flags")}
    rep, _ = compare(w, out, stop, mode=mode, q_rows=qr, **ckw)
    log(f"   {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    return w, out, stop, issued


ROWS = [("bf16 G4 paged", 2), ("bf16 G4 paged", 4), ("bf16 G4 contiguous", 2), ("bf16 G4 contiguous", 4),
        ("bf16 G2 paged", 2), ("fp32 G1", 4), ("fp32 G1", 8), ("fp32 G1", 16)]


@pytest.mark.parametrize("case,rows", ROWS, ids=[f"{c}-M{m}" for c, m in ROWS])
@pytest.mark.parametrize("mode", [orc.MODE_ART, orc.MODE_FULL])
def test_rows_parity(torch_cuda, case, rows, mode):
    w, _, stop, _ = _run(case, rows, mode, eps_scale=5e-2, eps_dir=5e-3)
    if mode == orc.MODE_FULL:
        np.testing.assert_array_equal(stop, w.traversal_lengths())


@pytest.mark.parametrize("rows", [2, 4])
def test_rows_full_mode_split_kv(torch_cuda, rows):
    """Full mode cut into chunks: the combine kernel writes every row."""
    w, _, stop, issued = _run("bf16 G4 paged", rows, orc.MODE_FULL, split_blocks=5)
    np.testing.assert_array_equal(issued, w.traversal_lengths())


@pytest.mark.parametrize("rows", [2, 4])
def test_rows_kept_list(torch_cuda, rows):
    _run("bf16 G4 kept list", rows, orc.MODE_ART)


def test_rows_forced_stop(torch_cuda):
    w, _, stop, _ = _run("bf16 G4 paged", 4, orc.MODE_ART, eps_scale=1e30, eps_dir=1e30, patience=2)
    np.testing.assert_array_equal(stop, np.minimum(w.traversal_lengths(), 3))


def test_rows_split_art_is_refused_above_four_vectors(torch_cuda):
    from kv_cache_early_amd import ArtError, art
    w = make_workload(scaled(3, "B"))
    with pytest.raises(ArtError) as e:
        _run("bf16 G4 paged", 2, orc.MODE_ART, split_blocks=8)
    assert e.value.status == art.ART_ERR_UNSUPPORTED
