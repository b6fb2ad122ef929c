"""Parity helpers: run libart on a workload and compare with the fp64 oracle.

The acceptance rule per unit (batch, kv head) is oracle.acceptance's:
  * stop_idx equal to the oracle's, unless the unit is margin-excused: some
    check t <= max(stop_gpu, stop_oracle) has a metric within a relative
    margin of 1e-4 of its threshold (|d / eps - 1| <= 1e-4);
  * the GPU output is compared with the oracle's O^(stop_gpu) (the exact
    truncated attention at the GPU's own stop), or O^(T') in detect-only
    mode, which attends to every block: relative L2 <= 1e-3 and max-abs
    <= 4e-3 per unit.
With a test switched off (ablation flags) only the remaining test's margin
can excuse a stop difference.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np

import oracle as orc
from workloads.device import to_device

from oracle.acceptance import MARGIN, MAX_ABS, REL_L2, unit_agreement  # noqa: F401


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(w, mode=1, patience=None, eps_scale=None, eps_dir=None, order=None, split_blocks=0, dev=None,
            decoder=None, flags=0, waves=0, q=None):
    """Upload (unless ``dev`` is given) and run art_decode; returns numpy arrays."""
    import torch
    from kv_cache_early_amd import ArtDecoder
    s = w.spec
    dev = dev or to_device(w)
    dec = decoder or ArtDecoder()
    r = dec.decode(dev.q if q is None else q, dev.k, dev.v, dev.context_lens, dtype=dev.dtype_code, page_size=dev.page_size,
                   block_table=dev.block_table, kept_blocks=dev.kept_blocks, kept_count=dev.kept_count,
                   eps_scale=s.eps_scale if eps_scale is None else eps_scale,
                   eps_dir=s.eps_dir if eps_dir is None else eps_dir,
                   patience=s.patience if patience is None else patience,
                   order=s.order if order is None else order, mode=mode, split_blocks=split_blocks, flags=flags,
                   waves=waves)
    torch.cuda.synchronize()
    err = dec.device_error()
    return (r.out.cpu().numpy().astype(np.float64), r.stop_idx.cpu().numpy().astype(np.int64),
            r.blocks_issued.cpu().numpy().astype(np.int64), err)


@dataclass
class Report:
    units: int = 0
    stop_equal: int = 0
    excused: int = 0
    unexcused: list = field(default_factory=list)
    worst_rel_l2: float = 0.0
    worst_abs: float = 0.0
    bad_outputs: list = field(default_factory=list)

    def ok(self):
        return not self.unexcused and not self.bad_outputs

    def __str__(self):
        return (f"units={self.units} stop_equal={self.stop_equal} excused={self.excused} "
                f"unexcused={len(self.unexcused)} worst_rel_l2={self.worst_rel_l2:.2e} "
                f"worst_abs={self.worst_abs:.2e} bad_outputs={len(self.bad_outputs)}")


def compare(w, out_gpu, stop_gpu, units=None, mode=1, patience=None, eps_scale=None, eps_dir=None, order=None,
            flags=0, q_rows=None):
    """Compare GPU results with the oracle on ``units`` (default: all).

    ``q_rows`` [B, M, Hq, d] (storage format) compares a multi-row call:
    ``out_gpu`` is then [B, M, Hq, d]."""
    s = w.spec
    es = s.eps_scale if eps_scale is None else eps_scale
    ed = s.eps_dir if eps_dir is None else eps_dir
    if q_rows is None:
        _, _, res = orc.art_decode_workload(w, mode=mode, patience=patience, units=units, keep_results=True,
                                            eps_scale=es, eps_dir=ed, order=order, flags=flags)
    else:
        _, _, res = orc.art_decode_rows(q_rows, w.k, w.v, w.context_lens, s.dtype, s.num_kv_heads, s.block_size,
                                        es, ed, s.patience if patience is None else patience,
                                        s.order if order is None else order, mode, s.page_size, w.block_table,
                                        w.kept_blocks, w.kept_count, units, True, flags)
        M = q_rows.shape[1]
        out_gpu = out_gpu.reshape(s.batch, M, s.num_kv_heads, s.group, -1).transpose(0, 2, 1, 3, 4).reshape(
            s.batch, s.num_kv_heads * M * s.group, -1)
    G = s.group * (1 if q_rows is None else q_rows.shape[1])  # query vectors per unit
    rep = Report()
    for (b, h), r in res.items():
        rep.units += 1
        sg = int(stop_gpu[b, h])
        a = unit_agreement(r, out_gpu[b, h * G:(h + 1) * G], sg, es, ed, flags)
        rep.stop_equal += int(a.stop_equal)
        if a.excused:
            rep.excused += 1
        elif not a.stop_equal:
            rep.unexcused.append(((b, h), sg, int(r.stop), a.margin))
        if not a.stop_in_range:
            rep.bad_outputs.append(((b, h), "stop out of range", sg))
            continue
        rep.worst_rel_l2 = max(rep.worst_rel_l2, a.rel_l2)
        rep.worst_abs = max(rep.worst_abs, a.max_abs)
        if not a.output_ok:
            rep.bad_outputs.append(((b, h), a.rel_l2, a.max_abs))
    return rep, res


def sample_units(w, n, seed=0):
    B, H = w.spec.batch, w.spec.num_kv_heads
    rng = np.random.default_rng(seed)
    allu = [(b, h) for b in range(B) for h in range(H)]
    if n >= len(allu):
        return allu
    idx = rng.choice(len(allu), size=n, replace=False)
    return sorted(allu[i] for i in idx)
