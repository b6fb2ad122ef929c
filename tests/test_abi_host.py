"""C-ABI checks that need no GPU: the library loads, exports every symbol
declared in include/art.h, and rejects bad arguments on the host before
anything is enqueued."""
import ctypes
import math
import os
import re

import pytest

from kv_cache_early_amd import art

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "art.h")

FAKE = 0x10000  # a non-null address; validation fails before any use


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(art_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = art.load()
    names = declared_functions()
    assert set(names) == set(art.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_probe_stride():
    for s in range(7):
        assert art.status_string(s) and art.status_string(s) != "unknown status"
    assert art.status_string(99) == "unknown status"
    assert art.load().art_probe_stride() == 4


def good_shape(**kw):
    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, dtype=art.ART_DT_BF16, page_size=16,
             max_ctx=0, max_pages=64, num_pages=200, max_kept=0, q_rows=1)
    d.update(kw)
    return art.make_shape(**d)


def good_params(**kw):
    d = dict(eps_scale=1e-3, eps_dir=1e-4, patience=2, order=art.ART_ORDER_RECENT_FIRST, mode=art.ART_MODE_ART,
             block_size=64, split_blocks=0, flags=0, waves=0)
    d.update(kw)
    return art.make_params(**d)


def call(shape, params, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, bt=FAKE, kept=None, kc=None, out=FAKE, stop=FAKE,
         issued=None, ws=FAKE * 16, ws_bytes=1 << 30, stream=None, shape_ptr=True, params_ptr=True):
    lib = art.load()
    return lib.art_decode(ctypes.byref(shape) if shape_ptr else None, ctypes.byref(params) if params_ptr else None,
                          q, k, v, lens, bt, kept, kc, out, stop, issued, ws, ws_bytes, stream)


CASES = [
    ("null shape", dict(shape_ptr=False), art.ART_ERR_INVALID_ARG),
    ("null params", dict(params_ptr=False), art.ART_ERR_INVALID_ARG),
    ("Hq % Hkv", dict(shape=good_shape(num_q_heads=6, num_kv_heads=4)), art.ART_ERR_INVALID_ARG),
    ("negative batch", dict(shape=good_shape(batch=-1)), art.ART_ERR_INVALID_ARG),
    ("bad dtype", dict(shape=good_shape(dtype=7)), art.ART_ERR_INVALID_ARG),
    ("head_dim 96", dict(shape=good_shape(head_dim=96)), art.ART_ERR_UNSUPPORTED),
    ("bf16 d64", dict(shape=good_shape(head_dim=64)), art.ART_ERR_UNSUPPORTED),
    ("32 query vectors per unit", dict(shape=good_shape(num_q_heads=16, q_rows=4)), art.ART_ERR_UNSUPPORTED),
    ("group 3", dict(shape=good_shape(num_q_heads=6, num_kv_heads=2)), art.ART_ERR_UNSUPPORTED),
    ("negative q_rows", dict(shape=good_shape(q_rows=-1)), art.ART_ERR_INVALID_ARG),
    ("split ART above 4 query vectors", dict(shape=good_shape(q_rows=2), params=good_params(split_blocks=4)),
     art.ART_ERR_UNSUPPORTED),
    ("block_size 32", dict(params=good_params(block_size=32)), art.ART_ERR_UNSUPPORTED),
    ("block_size 0", dict(params=good_params(block_size=0)), art.ART_ERR_INVALID_ARG),
    ("page 24", dict(shape=good_shape(page_size=24)), art.ART_ERR_INVALID_ARG),
    ("page 48", dict(shape=good_shape(page_size=48)), art.ART_ERR_UNSUPPORTED),
    ("patience 0", dict(params=good_params(patience=0)), art.ART_ERR_INVALID_ARG),
    ("eps negative", dict(params=good_params(eps_scale=-1e-3)), art.ART_ERR_INVALID_ARG),
    ("eps nan", dict(params=good_params(eps_dir=math.nan)), art.ART_ERR_INVALID_ARG),
    ("eps inf", dict(params=good_params(eps_scale=math.inf)), art.ART_ERR_INVALID_ARG),
    ("bad order", dict(params=good_params(order=3)), art.ART_ERR_INVALID_ARG),
    ("bad mode", dict(params=good_params(mode=2)), art.ART_ERR_INVALID_ARG),
    ("given without kept list", dict(params=good_params(order=art.ART_ORDER_GIVEN)), art.ART_ERR_INVALID_ARG),
    ("negative split", dict(params=good_params(split_blocks=-1)), art.ART_ERR_INVALID_ARG),
    ("unknown flag", dict(params=good_params(flags=8)), art.ART_ERR_INVALID_ARG),
    ("bad waves", dict(params=good_params(waves=3)), art.ART_ERR_INVALID_ARG),
    ("8 waves in full mode", dict(params=good_params(waves=8, mode=art.ART_MODE_FULL)), art.ART_ERR_UNSUPPORTED),
    ("8 waves with 8 query vectors", dict(shape=good_shape(q_rows=2), params=good_params(waves=8)),
     art.ART_ERR_UNSUPPORTED),
    ("given order past the repeat check's capacity",
     dict(shape=good_shape(max_pages=(524288 * 64) // 16 + 16, max_kept=8), kept=FAKE, kc=FAKE,
          params=good_params(order=art.ART_ORDER_GIVEN)), art.ART_ERR_UNSUPPORTED),
    ("flags in full mode", dict(params=good_params(mode=art.ART_MODE_FULL, flags=art.ART_FLAG_DETECT_ONLY)),
     art.ART_ERR_INVALID_ARG),
    ("kept without count", dict(shape=good_shape(max_kept=8), kept=FAKE), art.ART_ERR_INVALID_ARG),
    ("count without kept", dict(kc=FAKE), art.ART_ERR_INVALID_ARG),
    ("kept list but max_kept 0", dict(kept=FAKE, kc=FAKE), art.ART_ERR_INVALID_ARG),
    ("null q", dict(q=None), art.ART_ERR_INVALID_ARG),
    ("null out", dict(out=None), art.ART_ERR_INVALID_ARG),
    ("null stop", dict(stop=None), art.ART_ERR_INVALID_ARG),
    ("null lens", dict(lens=None), art.ART_ERR_INVALID_ARG),
    ("paged without table", dict(bt=None), art.ART_ERR_INVALID_ARG),
    ("contiguous with table", dict(shape=good_shape(page_size=0, max_ctx=4096)), art.ART_ERR_INVALID_ARG),
    ("null workspace", dict(ws=None), art.ART_ERR_WORKSPACE),
    ("small workspace", dict(ws_bytes=64), art.ART_ERR_WORKSPACE),
    ("misaligned workspace", dict(ws=FAKE * 16 + 8), art.ART_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,expect", CASES, ids=[c[0] for c in CASES])
def test_host_rejects(name, kw, expect):
    kw = dict(kw)
    shape = kw.pop("shape", good_shape())
    params = kw.pop("params", good_params())
    assert call(shape, params, **kw) == expect


def test_struct_size_mismatch_is_rejected():
    """A caller built against another layout of the structs is refused, not misread."""
    sh, pa = good_shape(), good_params()
    sh.struct_size -= 4
    assert call(sh, pa) == art.ART_ERR_INVALID_ARG
    sh, pa = good_shape(), good_params()
    pa.struct_size = 0
    assert call(sh, pa) == art.ART_ERR_INVALID_ARG
    sh = good_shape()
    sh.struct_size += 4
    assert art.load().art_workspace_size(ctypes.byref(sh), ctypes.byref(good_params())) == 0
    assert art.load().art_select_workspace_size(ctypes.byref(sh)) == 0


def test_abi_version():
    assert art.load().art_abi_version() == art.ART_ABI_VERSION == 2
    text = open(HEADER).read()
    assert re.search(r"#define ART_ABI_VERSION 2\b", text)


def test_empty_batch_is_a_no_op():
    assert call(good_shape(batch=0), good_params(), q=None, k=None, v=None, lens=None, bt=None, out=None,
                stop=None) == art.ART_OK


def test_last_error_rejects_without_touching_the_device():
    lib = art.load()
    assert lib.art_last_error(None, 4096) == art.ART_ERR_INVALID_ARG
    assert lib.art_last_error(FAKE * 16, 64) == art.ART_ERR_INVALID_ARG


def test_workspace_size():
    s, p = good_shape(), good_params()
    n = art.workspace_size(s, p)
    assert n > 0 and n % 256 == 0
    assert art.workspace_size(good_shape(head_dim=96), p) == 0
    full_split = art.workspace_size(s, good_params(mode=art.ART_MODE_FULL, split_blocks=4))
    assert full_split > n  # room for the split partials


@pytest.mark.parametrize("batch,hkv,expect", [
    (16, 8, 128),  # 128 units x 512 blocks, fewer units than CUs: about 512 work items
    (4, 8, 32),    # 32 units: about 512 work items
    (64, 8, 64),   # 512 units: about 4096 work items
    (32, 8, 32),   # 256 units: about 4096 work items, 32 blocks each
    (8, 8, 64),    # 64 units: about 512 work items
    (2, 8, 32),    # 16 units: 32 blocks still give every CU an item
    (1, 4, 8),     # 4 units: shorter items, so that every CU gets one
    (1, 1, 8),     # one unit: at least 8 blocks per item
])
def test_full_mode_default_decomposition(batch, hkv, expect):
    """The workspace holds one partial per work item, so its size shows the
    library's default chunk length: it must equal the size for that chunk
    length given explicitly, and differ from the neighbouring lengths."""
    s = good_shape(batch=batch, num_q_heads=4 * hkv, num_kv_heads=hkv, max_pages=2048, num_pages=4096)  # 512 blocks
    full = lambda sb: art.workspace_size(s, good_params(mode=art.ART_MODE_FULL, split_blocks=sb))
    units, tmax = batch * hkv, 512
    if units < 256:  # two items per CU, not below 32 blocks unless CUs would idle, never below 8
        c = max(-(-tmax * units // 512), min(32, -(-tmax * units // 256)), 8)
    else:
        c = max(32, -(-tmax * units // 4096))
    c = min(-(-c // 4) * 4, tmax)
    assert c == expect
    assert full(0) == full(expect)
    for other in (expect // 2, expect * 2):
        if 1 <= other <= tmax and -(-tmax // other) != -(-tmax // expect):
            assert full(0) != full(other)


@pytest.mark.parametrize("batch,split", [(16, True), (31, True), (32, False), (64, False)])
def test_art_mode_default_decomposition(batch, split):
    """ART mode: split ART in 16-block chunks below 256 units (fewer units
    than compute units), one work item per unit from 256 on.  The workspace
    size shows the choice: it equals the size for that decomposition given
    explicitly."""
    s = good_shape(batch=batch, num_q_heads=32, num_kv_heads=8, max_pages=2048, num_pages=8192)  # 512 blocks
    ws = lambda sb: art.workspace_size(s, good_params(split_blocks=sb))
    assert ws(16) != ws(10 ** 6)
    assert ws(0) == (ws(16) if split else ws(10 ** 6))
    assert ws(32) == ws(24) != ws(16)  # chunks are capped at 24 blocks


# ---------------------------------------------------------------------------
# block selection entry points: host-side rejections (nothing is enqueued)
# ---------------------------------------------------------------------------
def sel_params(**kw):
    d = dict(keep_frac=0.5, sink=1, recent=4, order=art.ART_SELECT_ASCENDING)
    d.update(kw)
    return art.art_select_params(**d)


def call_means(shape=None, k=FAKE, lens=FAKE, bt=FAKE, means=FAKE, max_blocks=1024, ws=FAKE * 16,
               ws_bytes=1 << 30):
    shape = shape or good_shape()
    return art.load().art_block_means(ctypes.byref(shape), k, lens, bt, means, max_blocks, ws, ws_bytes, None)


def call_select(shape=None, params=None, q=FAKE, means=FAKE, max_blocks=1024, lens=FAKE, kb=FAKE, kc=FAKE,
                ws=FAKE * 16, ws_bytes=1 << 30):
    shape = shape or good_shape(max_kept=512)
    params = params or sel_params()
    return art.load().art_select_blocks(ctypes.byref(shape), ctypes.byref(params), q, means, max_blocks, lens, kb, kc,
                                        ws, ws_bytes, None)


MEANS_CASES = [
    ("null k", dict(k=None), art.ART_ERR_INVALID_ARG),
    ("null means", dict(means=None), art.ART_ERR_INVALID_ARG),
    ("max_blocks below capacity", dict(max_blocks=15), art.ART_ERR_INVALID_ARG),
    ("paged without table", dict(bt=None), art.ART_ERR_INVALID_ARG),
    ("bad dtype", dict(shape=good_shape(dtype=7)), art.ART_ERR_INVALID_ARG),
    ("head_dim 96", dict(shape=good_shape(head_dim=96)), art.ART_ERR_UNSUPPORTED),
    ("small workspace", dict(ws_bytes=64), art.ART_ERR_WORKSPACE),
    ("misaligned workspace", dict(ws=FAKE * 16 + 8), art.ART_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,expect", MEANS_CASES, ids=[c[0] for c in MEANS_CASES])
def test_block_means_rejects(name, kw, expect):
    assert call_means(**kw) == expect


SELECT_CASES = [
    ("keep_frac 0", dict(params=sel_params(keep_frac=0.0)), art.ART_ERR_INVALID_ARG),
    ("keep_frac above 1", dict(params=sel_params(keep_frac=1.5)), art.ART_ERR_INVALID_ARG),
    ("keep_frac nan", dict(params=sel_params(keep_frac=math.nan)), art.ART_ERR_INVALID_ARG),
    ("negative sink", dict(params=sel_params(sink=-1)), art.ART_ERR_INVALID_ARG),
    ("bad order", dict(params=sel_params(order=2)), art.ART_ERR_INVALID_ARG),
    ("max_kept too small", dict(shape=good_shape(max_kept=3)), art.ART_ERR_INVALID_ARG),
    ("null kept_count", dict(kc=None), art.ART_ERR_INVALID_ARG),
    ("max_blocks below capacity", dict(max_blocks=15), art.ART_ERR_INVALID_ARG),
    ("more than 4096 blocks", dict(shape=good_shape(max_pages=20000, max_kept=20000), max_blocks=5000),
     art.ART_ERR_UNSUPPORTED),
    ("small workspace", dict(ws_bytes=64), art.ART_ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,expect", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_blocks_rejects(name, kw, expect):
    assert call_select(**kw) == expect


def test_select_workspace_size():
    s = good_shape()  # 2 units, 64 pages of 16 tokens = 16 blocks -> 4 groups per unit
    n = art.select_workspace_size(s)
    assert n >= 256 + 8 * 2 * 4 and n % 256 == 0
    assert art.select_workspace_size(good_shape(dtype=7)) == 0
    assert call_means(shape=good_shape(batch=0)) == art.ART_OK  # empty batch: nothing enqueued
    assert call_select(shape=good_shape(batch=0, max_kept=512)) == art.ART_OK


def test_static_workspace_entry_point_rejects_large_calls_before_launching():
    """art_decode_static refuses, on the host, a call whose workspace would
    not fit the library's per-device buffer (fake pointers: nothing may be
    touched), and validates arguments as art_decode does."""
    lib = art.load()
    sh = good_shape(batch=4096, num_kv_heads=8, num_q_heads=32, max_pages=2048)
    pa = good_params(mode=art.ART_MODE_FULL, split_blocks=1)
    need = art.workspace_size(sh, pa)
    assert need > art.ART_STATIC_SCRATCH_BYTES
    assert lib.art_decode_static(ctypes.byref(sh), ctypes.byref(pa), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                 FAKE, FAKE, None, None) == art.ART_ERR_WORKSPACE
    bad = good_params(patience=0)
    assert lib.art_decode_static(ctypes.byref(good_shape()), ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 None, FAKE, FAKE, None, None) == art.ART_ERR_INVALID_ARG
