"""GPU parity for key-based block selection (through the C ABI) against the
fp64 selection oracle, and importance-first ART end to end.

The kernel scores in fp32, so two blocks whose fp64 scores differ by less
than the fp32 error of a score may be ranked either way.  Where the rule
keeps one of two near-equal blocks, either is correct: the tests check that
every difference from the oracle's list involves only such near-ties, and
that every list is a valid answer.  The end-to-end test uses inputs with no
near-ties, so its lists must match exactly.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle as orc
from tests.parity import compare, log, run_gpu
from workloads import config, make_workload, scaled
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def score_tol(scores):
    """fp32 error bound on a score: 128 products of O(1) terms, rounded."""
    return 1e-5 * (1.0 + float(np.max(np.abs(scores)))) if scores.size else 0.0


def gpu_means(dec, dev, w):
    s = w.spec
    return dec.block_means(dev.k, dev.context_lens, num_q_heads=s.num_q_heads, dtype=dev.dtype_code,
                           page_size=dev.page_size, block_table=dev.block_table)


def gpu_select(dec, dev, w, means, frac, sink, recent, order):
    s = w.spec
    kw = dict(page_size=dev.page_size)
    if dev.page_size:
        kw["max_pages"] = int(dev.block_table.shape[1])
    else:
        kw["max_ctx"] = int(dev.k.shape[2])
    return dec.select_blocks(dev.q, means, dev.context_lens, dtype=dev.dtype_code, keep_frac=frac, sink=sink,
                             recent=recent, order=order, **kw)


@pytest.mark.parametrize("case", ["paged bf16", "contiguous bf16", "fp32 d64", "ragged lengths"])
def test_block_means(torch_cuda, case):
    from kv_cache_early_amd import ArtDecoder
    if case == "paged bf16":
        w = make_workload(scaled(3, "B"))
    elif case == "contiguous bf16":
        w = make_workload(scaled(2, "B"))
    elif case == "fp32 d64":
        w = make_workload(scaled(1, "B"))
    else:
        lens = np.array([0, 1, 63, 64, 65, 127, 129, 1000], dtype=np.int32)
        w = make_workload(replace(scaled(3, "B"), batch=8), context_lens=lens)
    log(f"[case] block means {case}")
    dec = ArtDecoder()
    dev = to_device(w)
    m = gpu_means(dec, dev, w).cpu().numpy().astype(np.float64)
    assert dec.device_error() == 0
    _, _, detail = orc.select_workload(w, 1.0, 0, 0)
    for (b, h), (means, _) in detail.items():
        T = means.shape[0]
        np.testing.assert_allclose(m[b, h, :T], means, rtol=1e-5, atol=1e-6, err_msg=f"unit {(b, h)}")


def unique_list(kept, scores, sink, recent):
    """The importance-ordered list is the same under any score error within
    the tolerance: adjacent kept blocks, and the weakest kept block against
    the strongest dropped one (forced blocks aside), are further apart."""
    tol = 4 * score_tol(scores)
    T, n = scores.shape[0], len(kept)
    n_sink = min(sink, n)
    forced = set(range(n_sink)) | set(range(T - max(0, min(recent, n - n_sink)), T))
    if np.any(np.abs(np.diff(scores[kept])) <= tol):
        return False
    free_kept = [scores[j] for j in kept if j not in forced]
    dropped = [scores[j] for j in range(T) if j not in set(kept.tolist())]
    return not (free_kept and dropped and min(free_kept) - max(dropped) <= tol)


def check_list(got, ref, scores, forced, order, tol):
    """`got` is a valid kept list: same length, same forced blocks, every
    difference from `ref` a near-tie at the selection boundary, and (for
    the importance order) sorted by score within the tolerance."""
    assert len(got) == len(ref)
    assert len(set(got.tolist())) == len(got)
    gs, rs = set(got.tolist()), set(ref.tolist())
    assert forced <= gs
    extra, missing = gs - rs, rs - gs
    if extra:
        # the boundary: the weakest non-forced block the oracle kept
        free = [j for j in rs if j not in forced]
        cut = min(scores[j] for j in free)
        for j in extra | missing:
            assert abs(scores[j] - cut) <= tol, (j, scores[j], cut)
    if order == orc.SELECT_ASCENDING:
        assert np.all(np.diff(got) > 0)
    else:
        assert np.all(np.diff(scores[got]) <= tol)


@pytest.mark.parametrize("order", [orc.SELECT_ASCENDING, orc.SELECT_IMPORTANCE])
@pytest.mark.parametrize("frac,sink,recent", [(0.5, 1, 24), (0.25, 2, 8), (1.0, 1, 0), (0.1, 0, 0)])
def test_select_blocks(torch_cuda, order, frac, sink, recent):
    from kv_cache_early_amd import ArtDecoder
    w = make_workload(scaled(5, "B"))
    log(f"[case] select frac={frac} sink={sink} recent={recent} order={order}")
    dec = ArtDecoder()
    dev = to_device(w)
    means = gpu_means(dec, dev, w)
    kb, kc = gpu_select(dec, dev, w, means, frac, sink, recent, order)
    assert dec.device_error() == 0
    kb, kc = kb.cpu().numpy(), kc.cpu().numpy()
    rkb, rkc, detail = orc.select_workload(w, frac, sink, recent, order)
    np.testing.assert_array_equal(kc, rkc)
    for (b, h), (_, scores) in detail.items():
        T = scores.shape[0]
        n = int(rkc[b, h])
        n_sink = min(sink, n)
        forced = set(range(n_sink)) | set(range(T - max(0, min(recent, n - n_sink)), T))
        check_list(kb[b, h, :n], rkb[b, h, :n], scores, forced, order, score_tol(scores))


def test_select_empty_and_short_sequences(torch_cuda):
    from kv_cache_early_amd import ArtDecoder
    lens = np.array([0, 1, 64, 65, 200, 1000, 3000, 5000], dtype=np.int32)
    w = make_workload(replace(scaled(3, "B"), batch=8), context_lens=lens)
    log("[case] select with empty and short sequences")
    dec = ArtDecoder()
    dev = to_device(w)
    means = gpu_means(dec, dev, w)
    kb, kc = gpu_select(dec, dev, w, means, 0.5, 1, 2, orc.SELECT_ASCENDING)
    assert dec.device_error() == 0
    kb, kc = kb.cpu().numpy(), kc.cpu().numpy()
    rkb, rkc, detail = orc.select_workload(w, 0.5, 1, 2)
    np.testing.assert_array_equal(kc, rkc)
    assert np.all(kc[0] == 0)
    for (b, h), (_, scores) in detail.items():
        n = int(rkc[b, h])
        T = scores.shape[0]
        forced = set(range(min(1, n))) | set(range(T - max(0, min(2, n - min(1, n))), T))
        check_list(kb[b, h, :n], rkb[b, h, :n], scores, forced, orc.SELECT_ASCENDING, score_tol(scores))


def test_bad_page_id_is_reported(torch_cuda):
    from kv_cache_early_amd import ArtDecoder, art
    w = make_workload(scaled(3, "B"))
    w.block_table = w.block_table.copy()
    w.block_table[1, 2] = 10 ** 8
    log("[case] block means with a page id outside the pool")
    dec = ArtDecoder()
    dev = to_device(w)
    gpu_means(dec, dev, w)
    assert dec.device_error() == art.ART_ERR_DEVICE_INPUT


@pytest.mark.parametrize("n", [3, 5])
def test_importance_first_art_end_to_end(torch_cuda, n):
    """Block means -> importance order (every block, or the kept list) ->
    ART walking that order (ART_ORDER_GIVEN), all on the GPU; the oracle
    makes its own selection and runs ART on its own list."""
    from kv_cache_early_amd import ArtDecoder
    w = make_workload(scaled(n, "B"))
    frac, sink, recent = (1.0, 0, 0) if n == 3 else (0.5, 1, 24)
    log(f"[case] importance-first ART scaled cfg{n}")
    rkb, rkc, detail = orc.select_workload(w, frac, sink, recent, orc.SELECT_IMPORTANCE)
    for (b, h), (_, scores) in detail.items():
        assert unique_list(rkb[b, h, :rkc[b, h]], scores, sink, recent), "inputs with near-tied scores"
    dec = ArtDecoder()
    dev = to_device(w)
    means = gpu_means(dec, dev, w)
    kb, kc = gpu_select(dec, dev, w, means, frac, sink, recent, orc.SELECT_IMPORTANCE)
    kb_h, kc_h = kb.cpu().numpy(), kc.cpu().numpy()
    np.testing.assert_array_equal(kc_h, rkc)
    for b in range(w.spec.batch):
        for h in range(w.spec.num_kv_heads):
            np.testing.assert_array_equal(kb_h[b, h, :kc_h[b, h]], rkb[b, h, :rkc[b, h]])
    # ART over the GPU's list, on the GPU; the oracle walks its own list
    dev.kept_blocks, dev.kept_count = kb.contiguous(), kc.contiguous()
    w.kept_blocks, w.kept_count = rkb, rkc
    out, stop, issued, err = run_gpu(w, dev=dev, order=orc.ORDER_GIVEN, eps_scale=5e-2, eps_dir=5e-3, decoder=dec)
    assert err == 0
    rep, _ = compare(w, out, stop, order=orc.ORDER_GIVEN, eps_scale=5e-2, eps_dir=5e-3)
    log(f"   {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    # importance-first reaches the stop in fewer blocks than recency-first on these inputs
    _, stop_rf, _, _ = run_gpu(make_workload(scaled(n, "B")), eps_scale=5e-2, eps_dir=5e-3)
    log(f"   blocks: importance-first {int(stop.sum())}, recency-first {int(stop_rf.sum())}")
