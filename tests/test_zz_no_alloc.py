"""art_decode_static (the library's own per-device workspace, no
allocation by the caller or the library) against art_decode on the same
inputs: two calls in a row, the second on a smaller input, in each
decomposition that uses the workspace (one work item per unit, split-KV
full mode with the combine kernel, ordered split ART).  Stops must be
identical and outputs within the parity bar of the method's target (they
are in fact bitwise equal: same kernels, same inputs); blocks_issued within
its documented bounds.
"""
from dataclasses import replace

import numpy as np
import pytest

from tests.parity import MAX_ABS, REL_L2, log
from workloads import make_workload, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _both(w, mode, split_blocks):
    """The same call through art_decode (own workspace) and art_decode_static."""
    import torch
    from kv_cache_early_amd import art
    from workloads.device import to_device
    s = w.spec
    dev = to_device(w)
    B, Hq, d = dev.q.shape
    Hkv = dev.k.shape[1]
    shape = art.make_shape(B, Hq, Hkv, d, dev.dtype_code, dev.page_size,
                           max_ctx=dev.k.shape[2] if dev.page_size == 0 else 0,
                           max_pages=dev.block_table.shape[1] if dev.block_table is not None else 0,
                           num_pages=dev.k.shape[0] if dev.page_size else 0,
                           max_kept=dev.kept_blocks.shape[2] if dev.kept_blocks is not None else 0)
    params = art.make_params(s.eps_scale, s.eps_dir, s.patience, s.order, mode, 64, split_blocks)
    need = art.workspace_size(shape, params)
    assert 0 < need <= art.ART_STATIC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    stream = torch.cuda.current_stream().cuda_stream
    for static in (False, True):
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        stop = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
        issued = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
        args = (shape, params, dev.q, dev.k, dev.v, dev.context_lens, dev.block_table, dev.kept_blocks,
                dev.kept_count, out, stop, issued)
        st = art.decode_static_raw(*args, stream) if static else art.decode_raw(*args, ws, need, stream)
        assert st == art.ART_OK, art.status_string(st)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy().astype(np.float64), stop.cpu().numpy(), issued.cpu().numpy()))
    if True:
        assert art.last_error(ws, need) == art.ART_OK
    return outs


@pytest.mark.parametrize("mode,split", [(1, 10 ** 6), (0, 3), (1, 8)],
                         ids=["ART one item per unit", "full mode split-KV", "ordered split ART"])
def test_static_workspace_matches_art_decode(torch_cuda, mode, split):
    big = make_workload(scaled(3, "B"))
    small = make_workload(replace(scaled(3, "B"), batch=2), context_lens=np.array([700, 1900], dtype=np.int32))
    for tag, w in (("first call", big), ("second call, smaller input", small)):
        log(f"[case] static workspace mode={mode} split={split}: {tag}")
        (o1, s1, i1), (o2, s2, i2) = _both(w, mode, split)
        Tp = w.traversal_lengths()
        np.testing.assert_array_equal(s2, s1)
        assert np.all((s2 >= 1) & (s2 <= Tp))
        for b in range(w.spec.batch):
            for h in range(w.spec.num_kv_heads):
                G = w.spec.group
                ref, got = o1[b, h * G:(h + 1) * G], o2[b, h * G:(h + 1) * G]
                rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
                assert rel <= REL_L2 and np.abs(got - ref).max() <= MAX_ABS, (b, h, rel)
        assert np.array_equal(o1, o2), "same kernels on the same inputs: expected identical bits"
        if mode == 0:
            np.testing.assert_array_equal(i2, i1)
        assert np.all(i2 >= s2) and np.all(i2 <= Tp + 32)
