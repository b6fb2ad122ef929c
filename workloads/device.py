"""Upload a host ``Workload`` to device tensors (memory movement only)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class DeviceWorkload:
    q: object
    k: object
    v: object
    context_lens: object
    block_table: Optional[object]
    kept_blocks: Optional[object]
    kept_count: Optional[object]
    dtype_code: int          # 0 fp32, 1 bf16 (the C ABI's art_dtype)
    page_size: int


def to_device(w, device="cuda") -> DeviceWorkload:
    import torch

    def t(x, dt=None):
        if x is None:
            return None
        a = np.ascontiguousarray(x)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    return DeviceWorkload(q=t(w.q), k=t(w.k), v=t(w.v), context_lens=t(w.context_lens),
                          block_table=t(w.block_table), kept_blocks=t(w.kept_blocks),
                          kept_count=t(w.kept_count), dtype_code=1 if w.spec.dtype == "bf16" else 0,
                          page_size=w.spec.page_size)
