"""Thin ctypes binding over libart's C ABI (include/art.h).

Argument marshalling only: every step of the decode runs in the HIP
kernels of libart.so.  torch is used for device memory and streams.  The
library must have been built (``python -m kv_cache_early_amd.build``); there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libart.so")

ART_OK = 0
ART_ERR_INVALID_ARG = 1
ART_ERR_UNSUPPORTED = 2
ART_ERR_WORKSPACE = 3
ART_ERR_HIP = 4
ART_ERR_TIMEOUT = 5
ART_ERR_DEVICE_INPUT = 6

ART_DT_F32 = 0
ART_DT_BF16 = 1
ART_ORDER_NATURAL = 0
ART_ORDER_RECENT_FIRST = 1
ART_ORDER_GIVEN = 2
ART_MODE_FULL = 0
ART_MODE_ART = 1
ART_FLAG_NO_SCALE = 1
ART_FLAG_NO_DIR = 2
ART_FLAG_DETECT_ONLY = 4
ART_SELECT_ASCENDING = 0
ART_SELECT_IMPORTANCE = 1
ART_ABI_VERSION = 2  # include/art.h

EXPORTS = ("art_workspace_size", "art_decode", "art_last_error", "art_status_string", "art_probe_stride",
           "art_select_workspace_size", "art_block_means", "art_select_blocks", "art_abi_version",
           "art_decode_static")
ART_STATIC_SCRATCH_BYTES = 32 << 20  # include/art.h


class art_params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("block_size", ctypes.c_int32), ("eps_scale", ctypes.c_float),
                ("eps_dir", ctypes.c_float), ("patience", ctypes.c_int32), ("order", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("split_blocks", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("waves", ctypes.c_int32)]


class art_shape(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_kept", ctypes.c_int32), ("q_rows", ctypes.c_int32)]


class art_select_params(ctypes.Structure):
    _fields_ = [("keep_frac", ctypes.c_float), ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
                ("order", ctypes.c_int32)]


class ArtError(RuntimeError):
    def __init__(self, status: int, what: str = "art_decode"):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libart.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libart.so not built at {path}; run `python -m kv_cache_early_amd.build`")
    # torch carries its own HIP runtime: loading it first makes libart bind to
    # that one, so the process has a single runtime whatever the import order
    # (a second one, loaded first, does not see the device)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    lib.art_workspace_size.argtypes = [ctypes.POINTER(art_shape), ctypes.POINTER(art_params)]
    lib.art_workspace_size.restype = ctypes.c_size_t
    lib.art_decode.argtypes = [ctypes.POINTER(art_shape), ctypes.POINTER(art_params), vp, vp, vp, vp, vp, vp, vp,
                               vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.art_decode.restype = ctypes.c_int
    lib.art_last_error.argtypes = [vp, ctypes.c_size_t]
    lib.art_last_error.restype = ctypes.c_int
    lib.art_status_string.argtypes = [ctypes.c_int]
    lib.art_status_string.restype = ctypes.c_char_p
    lib.art_probe_stride.argtypes = []
    lib.art_probe_stride.restype = ctypes.c_int32
    lib.art_select_workspace_size.argtypes = [ctypes.POINTER(art_shape)]
    lib.art_select_workspace_size.restype = ctypes.c_size_t
    lib.art_block_means.argtypes = [ctypes.POINTER(art_shape), vp, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_size_t, vp]
    lib.art_block_means.restype = ctypes.c_int
    lib.art_select_blocks.argtypes = [ctypes.POINTER(art_shape), ctypes.POINTER(art_select_params), vp, vp,
                                      ctypes.c_int32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.art_select_blocks.restype = ctypes.c_int
    lib.art_decode_static.argtypes = [ctypes.POINTER(art_shape), ctypes.POINTER(art_params), vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp]
    lib.art_decode_static.restype = ctypes.c_int
    lib.art_abi_version.argtypes = []
    lib.art_abi_version.restype = ctypes.c_int32
    if lib.art_abi_version() != ART_ABI_VERSION:
        raise ImportError(f"libart.so reports ABI version {lib.art_abi_version()}, the binding expects "
                          f"{ART_ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().art_status_string(int(status)).decode()


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, dtype, page_size=0, max_ctx=0, max_pages=0,
               num_pages=0, max_kept=0, q_rows=1) -> art_shape:
    return art_shape(ctypes.sizeof(art_shape), batch, num_q_heads, num_kv_heads, head_dim, dtype, page_size,
                     max_ctx, max_pages, num_pages, max_kept, q_rows)


def make_params(eps_scale=1e-3, eps_dir=1e-4, patience=2, order=ART_ORDER_RECENT_FIRST, mode=ART_MODE_ART,
                block_size=64, split_blocks=0, flags=0, waves=0) -> art_params:
    return art_params(ctypes.sizeof(art_params), block_size, eps_scale, eps_dir, patience, order, mode,
                      split_blocks, flags, waves)


def workspace_size(shape: art_shape, params: art_params) -> int:
    return int(load().art_workspace_size(ctypes.byref(shape), ctypes.byref(params)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def decode_raw(shape: art_shape, params: art_params, q, k, v, context_lens, block_table, kept_blocks, kept_count,
               out, stop_idx, blocks_issued, workspace, workspace_bytes: int, stream: Optional[int]) -> int:
    """Call art_decode with raw device pointers taken from tensors; returns the status."""
    return int(load().art_decode(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(context_lens), _ptr(block_table), _ptr(kept_blocks), _ptr(kept_count),
                                 _ptr(out), _ptr(stop_idx), _ptr(blocks_issued), _ptr(workspace),
                                 workspace_bytes, stream))


def decode_static_raw(shape: art_shape, params: art_params, q, k, v, context_lens, block_table, kept_blocks,
                      kept_count, out, stop_idx, blocks_issued, stream: Optional[int]) -> int:
    """Call art_decode_static (the library's own per-device workspace); returns the status."""
    return int(load().art_decode_static(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(context_lens), _ptr(block_table), _ptr(kept_blocks),
                                        _ptr(kept_count), _ptr(out), _ptr(stop_idx), _ptr(blocks_issued),
                                        stream))


def select_workspace_size(shape: art_shape) -> int:
    return int(load().art_select_workspace_size(ctypes.byref(shape)))


def block_means_raw(shape: art_shape, k, context_lens, block_table, means, max_blocks: int, workspace,
                    workspace_bytes: int, stream: Optional[int]) -> int:
    """Call art_block_means with raw device pointers taken from tensors; returns the status."""
    return int(load().art_block_means(ctypes.byref(shape), _ptr(k), _ptr(context_lens), _ptr(block_table),
                                      _ptr(means), int(max_blocks), _ptr(workspace), workspace_bytes, stream))


def select_blocks_raw(shape: art_shape, params: art_select_params, q, means, max_blocks: int, context_lens,
                      kept_blocks, kept_count, workspace, workspace_bytes: int, stream: Optional[int]) -> int:
    """Call art_select_blocks with raw device pointers taken from tensors; returns the status."""
    return int(load().art_select_blocks(ctypes.byref(shape), ctypes.byref(params), _ptr(q), _ptr(means),
                                        int(max_blocks), _ptr(context_lens), _ptr(kept_blocks), _ptr(kept_count),
                                        _ptr(workspace), workspace_bytes, stream))


def last_error(workspace, workspace_bytes: int) -> int:
    return int(load().art_last_error(_ptr(workspace), int(workspace_bytes)))


@dataclass
class DecodeResult:
    out: object            # fp32 [B, Hq, d]
    stop_idx: object       # int32 [B, Hkv]
    blocks_issued: object  # int32 [B, Hkv]


class ArtDecoder:
    """Owns a workspace and calls art_decode on torch device tensors.

    Tensors: q [B, Hq, d]; k, v contiguous [B, Hkv, max_ctx, d] or paged
    [num_pages, Hkv, page, d]; bf16 data may be passed as torch.bfloat16 or
    as int16/uint16 bit patterns.  All tensors must be contiguous and on the
    same device.
    """

    def __init__(self, device=None):
        import torch
        self.torch = torch
        self.device = torch.device(device or "cuda")
        self._ws = None
        load()

    def workspace(self, nbytes: int):
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = self.torch.empty(max(nbytes, 256), dtype=self.torch.uint8, device=self.device)
        return self._ws

    def decode(self, q, k, v, context_lens, *, dtype: int, page_size: int = 0, block_table=None,
               kept_blocks=None, kept_count=None, eps_scale=1e-3, eps_dir=1e-4, patience=2,
               order=ART_ORDER_RECENT_FIRST, mode=ART_MODE_ART, block_size=64, split_blocks=0, flags=0, waves=0,
               out=None, stop_idx=None, blocks_issued=None, stream=None) -> DecodeResult:
        torch = self.torch
        if q.dim() == 4:  # [B, M, Hq, d]: M query rows per sequence
            B, M, Hq, d = q.shape
        else:
            (B, Hq, d), M = q.shape, 1
        Hkv = k.shape[1]
        for t in (q, k, v, context_lens, block_table, kept_blocks, kept_count):
            if t is not None and not t.is_contiguous():
                raise ValueError("art_decode needs contiguous tensors")
        shape = make_shape(B, Hq, Hkv, d, dtype, page_size,
                           max_ctx=k.shape[2] if page_size == 0 else 0,
                           max_pages=block_table.shape[1] if block_table is not None else 0,
                           num_pages=k.shape[0] if page_size else 0,
                           max_kept=kept_blocks.shape[2] if kept_blocks is not None else 0, q_rows=M)
        params = make_params(eps_scale, eps_dir, patience, order, mode, block_size, split_blocks, flags, waves)
        nbytes = workspace_size(shape, params)
        if nbytes == 0:  # invalid shape or params: art_decode names the reason before using anything
            raise ArtError(decode_raw(shape, params, q, k, v, context_lens, block_table, kept_blocks, kept_count,
                                      q, q, None, None, 0, None))
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.empty(tuple(q.shape), dtype=torch.float32, device=self.device)
        if stop_idx is None:
            stop_idx = torch.empty((B, Hkv), dtype=torch.int32, device=self.device)
        if blocks_issued is None:
            blocks_issued = torch.empty((B, Hkv), dtype=torch.int32, device=self.device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st = decode_raw(shape, params, q, k, v, context_lens, block_table, kept_blocks, kept_count, out, stop_idx,
                        blocks_issued, ws, ws.numel(), stream)
        if st != ART_OK:
            raise ArtError(st)
        return DecodeResult(out, stop_idx, blocks_issued)

    def block_means(self, k, context_lens, *, num_q_heads: int, dtype: int, page_size: int = 0,
                    block_table=None, max_blocks: Optional[int] = None, out=None, stream=None):
        """art_block_means: fp32 [B, Hkv, max_blocks, d] block-mean keys (rows past
        a sequence's blocks are left as they are)."""
        torch = self.torch
        B, Hkv, d = context_lens.shape[0], k.shape[1], k.shape[3]
        max_ctx = k.shape[2] if page_size == 0 else 0
        max_pages = block_table.shape[1] if block_table is not None else 0
        cap = max_ctx if page_size == 0 else max_pages * page_size
        mb = (cap + 63) // 64 if max_blocks is None else max_blocks
        shape = make_shape(B, num_q_heads, Hkv, d, dtype, page_size, max_ctx=max_ctx, max_pages=max_pages,
                           num_pages=k.shape[0] if page_size else 0)
        nbytes = select_workspace_size(shape)
        if nbytes == 0:
            raise ArtError(ART_ERR_INVALID_ARG, "art_select_workspace_size")
        ws = self.workspace(nbytes)
        if out is None:
            out = torch.zeros((B, Hkv, mb, d), dtype=torch.float32, device=self.device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st = block_means_raw(shape, k, context_lens, block_table, out, mb, ws, ws.numel(), stream)
        if st != ART_OK:
            raise ArtError(st, "art_block_means")
        return out

    def select_blocks(self, q, means, context_lens, *, dtype: int, keep_frac: float, sink: int, recent: int,
                      order: int = ART_SELECT_ASCENDING, page_size: int = 0, max_ctx: int = 0, max_pages: int = 0,
                      max_kept: Optional[int] = None, stream=None):
        """art_select_blocks: (kept_blocks int32 [B, Hkv, max_kept], kept_count int32 [B, Hkv])."""
        import math
        torch = self.torch
        B, Hq, d = q.shape
        Hkv, mb = means.shape[1], means.shape[2]
        cap = max_ctx if page_size == 0 else max_pages * page_size
        tmax = (cap + 63) // 64
        if max_kept is None:
            max_kept = max(1, min(tmax, math.ceil(float(ctypes.c_float(keep_frac).value) * tmax)))
        shape = make_shape(B, Hq, Hkv, d, dtype, page_size, max_ctx=max_ctx, max_pages=max_pages,
                           num_pages=1 if page_size else 0, max_kept=max_kept)
        nbytes = select_workspace_size(shape)
        if nbytes == 0:
            raise ArtError(ART_ERR_INVALID_ARG, "art_select_workspace_size")
        ws = self.workspace(nbytes)
        kept_blocks = torch.full((B, Hkv, max_kept), -1, dtype=torch.int32, device=self.device)
        kept_count = torch.empty((B, Hkv), dtype=torch.int32, device=self.device)
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        params = art_select_params(keep_frac, sink, recent, order)
        st = select_blocks_raw(shape, params, q, means, mb, context_lens, kept_blocks, kept_count, ws, ws.numel(),
                               stream)
        if st != ART_OK:
            raise ArtError(st, "art_select_blocks")
        return kept_blocks, kept_count

    def device_error(self) -> int:
        """Device-side status of the last decode (synchronizes the device first)."""
        self.torch.cuda.synchronize(self.device)
        return last_error(self._ws, self._ws.numel()) if self._ws is not None else ART_OK
