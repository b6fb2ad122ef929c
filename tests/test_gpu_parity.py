"""GPU parity: libart (through the C ABI) against the fp64 oracle.

Every test prints the case it is about to run before touching the GPU.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle as orc
from tests.parity import compare, log, run_gpu, sample_units
from workloads import config, make_workload, scaled

pytestmark = pytest.mark.gpu

SPLIT_MAX = 24  # longest split-ART chunk
SPEC_DEPTH = 16  # split ART: chunks a unit may walk ahead of its resolved stop rule


def EXCUSED_MAX(units):
    """Margin-excused units allowed among `units` compared: 1%, rounded up."""
    return -(-units // 100)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def check(w, mode=1, tag="", **kw):
    log(f"[case] {tag or w.spec.name} reading={w.spec.reading} mode={mode} {kw}")
    out, stop, issued, err = run_gpu(w, mode=mode, **kw)
    assert err == 0, f"device error {err}"
    ckw = {k: v for k, v in kw.items() if k in ("patience", "eps_scale", "eps_dir", "order", "flags")}
    rep, res = compare(w, out, stop, mode=mode, **ckw)
    log(f"   {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    assert rep.excused <= EXCUSED_MAX(rep.units), str(rep)
    Tp = w.traversal_lengths()
    # split ART may re-read up to one chunk to recompute the stop chunk
    assert np.all(issued >= stop) and np.all(issued <= Tp + SPLIT_MAX), "blocks_issued out of range"
    return out, stop, issued, rep


@pytest.mark.parametrize("reading", ["A", "B"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("mode", [0, 1])
def test_scaled_configs(torch_cuda, n, reading, mode):
    """The library's own choice of work decomposition (few units: ordered
    split ART in ART mode)."""
    w = make_workload(scaled(n, reading))
    _, stop, _, _ = check(w, mode=mode, tag=f"scaled cfg{n}")
    if mode == 0:
        np.testing.assert_array_equal(stop, w.traversal_lengths())


@pytest.mark.parametrize("reading", ["A", "B"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_scaled_configs_one_item_per_unit(torch_cuda, n, reading):
    """ART mode with one work item per unit (the stop rule's chain over 4 waves)."""
    w = make_workload(scaled(n, reading))
    _, stop, issued, _ = check(w, tag=f"scaled cfg{n} one item per unit", split_blocks=10 ** 6, waves=4)
    assert np.all(issued <= np.minimum(w.traversal_lengths(), stop + 7))


@pytest.mark.parametrize("p", [1, 2, 3])
def test_forced_stop_after_p_plus_one(torch_cuda, p):
    """eps huge: every check is stable, so the stop is at min(T', p+1)."""
    w = make_workload(scaled(3, "B"))
    # one work item per unit (the chain's stop; split ART is tested below)
    _, stop, issued, _ = check(w, tag="huge eps", eps_scale=1e30, eps_dir=1e30, patience=p, split_blocks=10 ** 6,
                               waves=4)
    Tp = w.traversal_lengths()
    np.testing.assert_array_equal(stop, np.minimum(Tp, p + 1))
    # loads stop: the W positions in flight and their prefetches (W = 4
    # waves per unit) are the most that can be issued past it
    W = 4
    assert np.all(issued <= np.minimum(Tp, stop + 2 * W - 1))


def test_eps_zero_runs_to_the_end(torch_cuda):
    w = make_workload(scaled(3, "B"))
    _, stop, _, _ = check(w, tag="eps 0", eps_scale=0.0, eps_dir=0.0)
    np.testing.assert_array_equal(stop, w.traversal_lengths())


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_criterion_fires_at_real_lengths(torch_cuda, n):
    """Reading B at the configs' own context lengths, few units: ART fires."""
    s = config(n, "B", batch=2, num_q_heads=8, num_kv_heads=2)
    w = make_workload(s)
    _, stop, _, _ = check(w, tag=f"firing cfg{n}")
    assert np.all(stop < w.traversal_lengths()), "expected the criterion to fire on every unit"


@pytest.mark.parametrize("order", [orc.ORDER_NATURAL, orc.ORDER_RECENT_FIRST])
def test_orders(torch_cuda, order):
    w = make_workload(config(2, "B", batch=1, num_q_heads=8, num_kv_heads=2, ctx=(20000, 20000)))
    check(w, tag=f"order {order}", order=order)


def test_given_order_with_block0_moved_first(torch_cuda):
    import torch
    s = scaled(3, "B")
    w = make_workload(s)
    rng = np.random.default_rng(3)
    T = w.num_blocks
    kmax = int(T.max())
    kb = np.full((s.batch, s.num_kv_heads, kmax), -1, dtype=np.int32)
    kc = np.zeros((s.batch, s.num_kv_heads), dtype=np.int32)
    for b in range(s.batch):
        for h in range(s.num_kv_heads):
            n = int(rng.integers(1, T[b] + 1))
            lst = rng.choice(T[b], size=n, replace=False).astype(np.int32)
            kb[b, h, :n] = lst
            kc[b, h] = n
    w.kept_blocks, w.kept_count = kb, kc
    check(w, tag="given order", order=orc.ORDER_GIVEN, eps_scale=5e-2, eps_dir=5e-3)


def test_layout_equivalence_bitwise(torch_cuda):
    """Same logical KV, paged (shuffled pages) vs contiguous: identical bits."""
    base = scaled(3, "B")
    lens = np.array([700, 1333, 64, 2049], dtype=np.int32)
    wp = make_workload(base, context_lens=lens)
    wc = make_workload(replace(base, page_size=0), context_lens=lens)
    log("[case] layout equivalence")
    op, sp, _, e1 = run_gpu(wp, split_blocks=10 ** 6)
    oc, sc, _, e2 = run_gpu(wc, split_blocks=10 ** 6)
    assert e1 == e2 == 0
    np.testing.assert_array_equal(sp, sc)
    np.testing.assert_array_equal(op, oc)


@pytest.mark.parametrize("page", [16, 32, 64, 128])
def test_page_sizes(torch_cuda, page):
    w = make_workload(replace(scaled(3, "B"), page_size=page))
    check(w, tag=f"page {page}", eps_scale=2e-2, eps_dir=2e-3)


def test_edge_lengths(torch_cuda):
    """Empty, one-token, exact-block and ragged sequences in one batch."""
    s = replace(scaled(3, "B"), batch=8)
    lens = np.array([0, 1, 63, 64, 65, 127, 129, 1000], dtype=np.int32)
    w = make_workload(s, context_lens=lens)
    out, stop, issued, _ = check(w, tag="edge lengths", eps_scale=5e-2, eps_dir=5e-3, patience=1)
    assert np.all(stop[0] == 0) and np.all(out[0] == 0) and np.all(issued[0] == 0)
    assert np.all(stop[1] == 1)


@pytest.mark.parametrize("split", [1, 3, 7])
def test_full_mode_split_kv(torch_cuda, split):
    w = make_workload(scaled(3, "A"))
    _, stop, issued, _ = check(w, mode=0, tag=f"full split {split}", split_blocks=split)
    np.testing.assert_array_equal(stop, w.traversal_lengths())
    np.testing.assert_array_equal(issued, w.traversal_lengths())


@pytest.mark.parametrize("batch,hkv", [(1, 1), (1, 4), (2, 8)])
def test_full_mode_few_units_default_decomposition(torch_cuda, batch, hkv):
    """Full mode with fewer units than CUs, library default: about two work
    items per CU, down to 8-block items for one unit (here 1, 4 and 16
    units of up to 16k tokens, ragged), merged by the combine kernel."""
    w = make_workload(config(3, "A", batch=batch, num_q_heads=4 * hkv, num_kv_heads=hkv, ctx=(9000, 16384)))
    _, stop, issued, _ = check(w, mode=0, tag=f"full default {batch}x{hkv}")
    np.testing.assert_array_equal(stop, w.traversal_lengths())
    np.testing.assert_array_equal(issued, w.traversal_lengths())


@pytest.mark.parametrize("mode", [0, 1])
def test_length_ranked_unit_order(torch_cuda, mode):
    """One work item per unit pairs long and short sequences on a CU by
    ranking the lengths in every workgroup: an odd batch with repeated
    lengths still gives every unit exactly once, in place."""
    lens = [1500, 900, 1500, 2900, 700]
    w = make_workload(config(3, "B", batch=5, num_q_heads=8, num_kv_heads=2), context_lens=lens)
    _, stop, issued, _ = check(w, mode=mode, tag=f"ranked unit order mode {mode}", split_blocks=10 ** 6)
    if mode == 0:
        np.testing.assert_array_equal(stop, w.traversal_lengths())


def test_full_mode_more_than_64_chunks(torch_cuda):
    """One block per chunk over 65 blocks: the combine kernel's lanes take
    the chunks 64 at a time, so this unit needs two passes."""
    w = make_workload(scaled(2, "B"))
    assert np.all(w.traversal_lengths() == 65)
    _, stop, issued, _ = check(w, mode=0, tag="full mode, 65 chunks", split_blocks=1)
    np.testing.assert_array_equal(stop, w.traversal_lengths())
    np.testing.assert_array_equal(issued, w.traversal_lengths())


def test_kept_list_out_of_range_is_reported(torch_cuda):
    from kv_cache_early_amd import art
    w = make_workload(scaled(5, "B"))
    w.kept_blocks = w.kept_blocks.copy()
    w.kept_blocks[0, 1, 3] = 10 ** 6
    log("[case] bad kept list")
    out, stop, issued, err = run_gpu(w)
    assert err == art.ART_ERR_DEVICE_INPUT
    assert stop[0, 1] == -1
    good = [(b, h) for b in range(w.spec.batch) for h in range(w.spec.num_kv_heads) if (b, h) != (0, 1)]
    rep, _ = compare(w, out, stop, units=good)
    assert rep.ok(), str(rep)


def test_device_error_is_per_call(torch_cuda):
    """A bad call's device error does not leak into the next call on the same workspace."""
    from kv_cache_early_amd import ArtDecoder, art
    dec = ArtDecoder()
    w = make_workload(scaled(5, "B"))
    bad = make_workload(scaled(5, "B"))
    bad.kept_blocks = bad.kept_blocks.copy()
    bad.kept_blocks[1, 0, 0] = -3
    log("[case] bad kept list, then a good call on the same workspace")
    _, _, _, e1 = run_gpu(bad, decoder=dec)
    assert e1 == art.ART_ERR_DEVICE_INPUT
    out, stop, _, e2 = run_gpu(w, decoder=dec)
    assert e2 == art.ART_OK
    rep, _ = compare(w, out, stop)
    assert rep.ok(), str(rep)


# ---------------------------------------------------------------------------
# full-size configurations: every unit on the GPU, sampled units in the oracle
# ---------------------------------------------------------------------------
FULL = [(2, "A"), (2, "B"), (3, "A"), (3, "B"), (4, "A"), (4, "B"), (5, "A"), (5, "B")]


@pytest.mark.parametrize("n,reading", FULL)
def test_full_size_sampled(torch_cuda, n, reading):
    log(f"[case] full-size cfg{n} reading={reading}: generating")
    w = make_workload(config(n, reading))
    units = sample_units(w, 12, seed=n)
    log(f"[case] full-size cfg{n} reading={reading}: GPU")
    patiences = (1, 2, 4) if n == 4 else (w.spec.patience,)
    from workloads.device import to_device
    dev = to_device(w)
    # few units: the library's choice is split ART; also one work item per unit
    splits = (0, 1 << 20) if n in (2, 5) else (0,)
    for p in patiences:
        for split in splits:
            out, stop, issued, err = run_gpu(w, patience=p, dev=dev, split_blocks=split)
            assert err == 0
            rep, _ = compare(w, out, stop, units=units, patience=p)
            log(f"   p={p} split={split} {rep} skipped={1 - stop.sum() / w.traversal_lengths().sum():.3f}")
            assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
            # a margin excuse needs an fp32-vs-fp64 flip right at a threshold:
            # at most 1% of the compared units (rounded up) may use it
            assert rep.excused <= EXCUSED_MAX(rep.units), str(rep)
            assert np.all((stop >= 1) & (stop <= w.traversal_lengths()))
    # full mode, in the library's own decomposition at this size (split-KV
    # chunks and the combine kernel), on the same sampled units
    out, stop, issued, err = run_gpu(w, mode=0, dev=dev)
    assert err == 0
    rep, _ = compare(w, out, stop, units=units, mode=0)
    log(f"   full mode {rep}")
    assert rep.ok(), (rep.unexcused[:5], rep.bad_outputs[:5])
    np.testing.assert_array_equal(stop, w.traversal_lengths())
    np.testing.assert_array_equal(issued, w.traversal_lengths())
    del dev


# ---------------------------------------------------------------------------
# ordered split ART (chunks with look-back) against the oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [4, 8, 16, 20, 24, 32])
def test_split_art_firing(torch_cuda, split):
    """Few units at long context, forced chunk lengths: the stop is found by
    the look-back replay and the stop chunk is recomputed."""
    w = make_workload(config(2, "B", batch=2, num_q_heads=8, num_kv_heads=2, ctx=(20000, 32768)))
    _, stop, _, _ = check(w, tag=f"split ART {split}", split_blocks=split)
    assert np.all(stop < w.traversal_lengths())


def test_split_art_bounded_speculation(torch_cuda):
    """A chunk starts loading only once the chunk SPEC_DEPTH places before it
    has published its carry, so a unit loads at most the chunks up to
    SPEC_DEPTH - 1 past its stop chunk, plus the stop chunk's recompute.
    With 4-block chunks the calls hand out up to 128 chunks per unit, nearly
    all past the stop."""
    C = 4
    w = make_workload(config(2, "B", batch=2, num_q_heads=8, num_kv_heads=2, ctx=(20000, 32768)))
    _, stop, issued, _ = check(w, tag="split ART bounded speculation", split_blocks=C)
    Tp = w.traversal_lengths()
    assert np.all(stop < Tp)
    stop_chunk = (stop - 1) // C
    bound = np.minimum(Tp, (stop_chunk + SPEC_DEPTH) * C) + C
    log(f"   issued {issued.ravel().tolist()} stop {stop.ravel().tolist()} bound {bound.ravel().tolist()}")
    assert np.all(issued <= bound)


@pytest.mark.parametrize("p", [1, 2, 3])
def test_split_art_stop_in_first_chunk(torch_cuda, p):
    w = make_workload(config(2, "B", batch=1, num_q_heads=8, num_kv_heads=2, ctx=(12000, 12000)))
    _, stop, _, _ = check(w, tag="split ART early stop", split_blocks=8, eps_scale=1e30, eps_dir=1e30, patience=p)
    np.testing.assert_array_equal(stop, np.minimum(w.traversal_lengths(), p + 1))


def test_split_art_no_stop(torch_cuda):
    """eps 0: every chunk passes its carry on; the output is full attention."""
    w = make_workload(config(2, "B", batch=1, num_q_heads=8, num_kv_heads=2, ctx=(9000, 9000)))
    _, stop, issued, _ = check(w, tag="split ART eps 0", split_blocks=8, eps_scale=0.0, eps_dir=0.0)
    np.testing.assert_array_equal(stop, w.traversal_lengths())


@pytest.mark.parametrize("order", [orc.ORDER_NATURAL, orc.ORDER_GIVEN])
def test_split_art_orders(torch_cuda, order):
    s = config(5, "B", batch=1, num_q_heads=8, num_kv_heads=2, ctx=(16384, 16384))
    w = make_workload(s)
    if order == orc.ORDER_GIVEN:
        rng = np.random.default_rng(5)
        kb = w.kept_blocks.copy()
        for h in range(s.num_kv_heads):
            n = int(w.kept_count[0, h])
            kb[0, h, :n] = rng.permutation(kb[0, h, :n])
        w.kept_blocks = kb
    check(w, tag=f"split ART order {order}", order=order, split_blocks=16, eps_scale=2e-2, eps_dir=2e-3)


# ---------------------------------------------------------------------------
# stop-rule switches: ablations and detect-only
# ---------------------------------------------------------------------------
ABLATIONS = [orc.FLAG_NO_SCALE, orc.FLAG_NO_DIR, orc.FLAG_NO_SCALE | orc.FLAG_NO_DIR]


@pytest.mark.parametrize("flags", ABLATIONS)
@pytest.mark.parametrize("split", [0, 8])
def test_ablation_flags(torch_cuda, flags, split):
    """One test of the stability check taken out: the stops follow the
    oracle's ablated rule, in one work item per unit and in split ART."""
    w = make_workload(scaled(3, "B"))
    sb = 10 ** 6 if split == 0 else split
    _, stop, _, _ = check(w, tag=f"ablation flags={flags} split={split}", flags=flags, split_blocks=sb,
                          eps_scale=5e-2, eps_dir=5e-3)
    assert np.all(stop <= w.traversal_lengths())


@pytest.mark.parametrize("split", [0, 4, 8, 32])
def test_detect_only(torch_cuda, split):
    """Detect-only reads every block once: the output is full decode, the stop
    is the one ART mode finds, blocks_issued is T'."""
    w = make_workload(config(2, "B", batch=2, num_q_heads=8, num_kv_heads=2, ctx=(20000, 32768)))
    sb = 10 ** 6 if split == 0 else split
    eps = dict(eps_scale=5e-2, eps_dir=5e-3)
    _, stop_d, issued, _ = check(w, tag=f"detect-only split={split}", flags=orc.FLAG_DETECT_ONLY, split_blocks=sb,
                                 **eps)
    Tp = w.traversal_lengths()
    np.testing.assert_array_equal(issued, Tp)
    _, stop_a, _, _ = check(w, tag=f"ART split={split}", split_blocks=sb, **eps)
    np.testing.assert_array_equal(stop_d, stop_a)
    assert np.any(stop_d < Tp), "the rule should fire somewhere"


def test_detect_only_never_fires(torch_cuda):
    w = make_workload(scaled(3, "B"))
    _, stop, issued, _ = check(w, tag="detect-only eps 0", flags=orc.FLAG_DETECT_ONLY, eps_scale=0.0, eps_dir=0.0)
    np.testing.assert_array_equal(stop, w.traversal_lengths())
    np.testing.assert_array_equal(issued, w.traversal_lengths())


# ---------------------------------------------------------------------------
# the stop rule's chain: 4 or 8 waves per unit, stops at every position
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("p", [1, 2, 3, 4, 5, 6, 7, 8])
def test_chain_forced_stop_at_every_position(torch_cuda, waves, p):
    """eps huge: every check is stable, so the stop is at min(T', p+1).  p
    from 1 to 8 puts the stop on every position modulo 4 and 8, so each
    wave of the chain once holds the stopping position, and the patience
    runs cross from wave to wave.  Loads past the stop: at most 2W - 1."""
    w = make_workload(scaled(3, "B"))
    _, stop, issued, _ = check(w, tag=f"chain W={waves} p={p}", eps_scale=1e30, eps_dir=1e30, patience=p,
                               split_blocks=10 ** 6, waves=waves)
    Tp = w.traversal_lengths()
    np.testing.assert_array_equal(stop, np.minimum(Tp, p + 1))
    assert np.all(issued <= np.minimum(Tp, stop + 2 * waves - 1))


@pytest.mark.parametrize("reading", ["A", "B"])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_eight_waves_per_unit(torch_cuda, n, reading):
    """8 waves per workgroup on every scaled configuration: parity with the
    oracle, and loads past the stop bounded by 2 * 8 - 1."""
    w = make_workload(scaled(n, reading))
    _, stop, issued, _ = check(w, tag=f"scaled cfg{n} 8 waves", split_blocks=10 ** 6, waves=8)
    assert np.all(issued <= np.minimum(w.traversal_lengths(), stop + 15))


@pytest.mark.parametrize("waves", [4, 8])
def test_chain_natural_stops(torch_cuda, waves):
    """Generator B at its own lengths: the criterion fires at data-dependent
    positions; 4 and 8 waves agree with the oracle (and so with each other,
    up to margin-excused units)."""
    w = make_workload(config(2, "B", batch=2, num_q_heads=8, num_kv_heads=2, ctx=(20000, 32768)))
    _, stop, issued, _ = check(w, tag=f"chain natural W={waves}", split_blocks=10 ** 6, waves=waves)
    assert np.all(stop < w.traversal_lengths())
    assert np.all(issued <= np.minimum(w.traversal_lengths(), stop + 2 * waves - 1))


@pytest.mark.parametrize("waves", [4, 8])
def test_chain_detect_only(torch_cuda, waves):
    w = make_workload(config(2, "B", batch=2, num_q_heads=8, num_kv_heads=2, ctx=(20000, 32768)))
    eps = dict(eps_scale=5e-2, eps_dir=5e-3)
    _, stop_d, issued, _ = check(w, tag=f"chain detect-only W={waves}", flags=orc.FLAG_DETECT_ONLY,
                                 split_blocks=10 ** 6, waves=waves, **eps)
    np.testing.assert_array_equal(issued, w.traversal_lengths())
    _, stop_a, _, _ = check(w, tag=f"chain ART W={waves}", split_blocks=10 ** 6, waves=waves, **eps)
    np.testing.assert_array_equal(stop_d, stop_a)


def test_given_order_repeated_block_is_reported(torch_cuda):
    """GIVEN order with a block listed twice: the unit is rejected
    (ART_ERR_DEVICE_INPUT, stop -1, out 0); the other units are unaffected."""
    from kv_cache_early_amd import art
    s = scaled(5, "B")
    w = make_workload(s)
    kb = w.kept_blocks.copy()
    n = int(w.kept_count[1, 0])
    kb[1, 0, n - 1] = kb[1, 0, 2]  # a duplicate inside the used part of the list
    w.kept_blocks = kb
    log("[case] GIVEN order with a repeated block")
    for split in (0, 10 ** 6):
        out, stop, issued, err = run_gpu(w, order=orc.ORDER_GIVEN, split_blocks=split)
        assert err == art.ART_ERR_DEVICE_INPUT
        assert stop[1, 0] == -1 and np.all(out[1, 0:s.group] == 0) and issued[1, 0] == 0
        good = [(b, h) for b in range(s.batch) for h in range(s.num_kv_heads) if (b, h) != (1, 0)]
        rep, _ = compare(w, out, stop, units=good, order=orc.ORDER_GIVEN)
        log(f"   split={split} {rep}")
        assert rep.ok(), str(rep)
