#!/usr/bin/env python3
"""Benchmark: ART decode attention on one MI355X.

A step is one art_decode call (the whole hot path: one kernel in ART mode)
over the whole batch of the large-batch paged decode workload: batch 64,
32 query / 8 KV heads, head_dim 128, bf16 KV in 16-token pages with a
shuffled block table, context lengths uniform in [8192, 32768], 64-token ART
blocks, eps_scale 2e-3, eps_dir 2e-4, patience 3, recency-first traversal.
Inputs are generated once (seeded, synthetic) and are resident in HBM before
the timed region.  Before every timed step an untimed 1 GiB scratch read
evicts the last-level (MALL) and L2 caches.  It is a read on purpose: a
scratch write would leave up to the MALL's size of dirty lines behind, and
their write-back would be charged to the timed kernel (+60 us measured).

Reported (one JSON line on stdout):
  value          KV GB/s on the bytes actually loaded (blocks_issued x block
                 bytes + per-unit q / out / block-table bytes) / step time,
                 ART mode, generator reading "B" (Llama-shaped keys, where
                 the criterion fires)
  roofline       algorithmic bytes (stop_idx x block bytes + per-unit terms)
                 per launch / average decode-kernel time (HIP events on the
                 launch stream around the call, which enqueues only that
                 kernel in ART mode) against the 8 TB/s HBM peak; `traffic`
                 is the HBM bytes per launch measured with rocprofv3 counters
                 (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel),
                 read from the committed counter summary and reported only
                 while the kernel sources still match it
  cpu_baseline   the fp64 numpy oracle over every unit of the same workload,
                 in single-threaded worker processes (cores = workers),
                 with the acceptance rule applied to the GPU's stop and
                 output of every unit (worst rel-L2 / max-abs, excused)
  extra fields   full-attention mode and generator reading "A" on the same
                 shapes, % KV blocks skipped, effective tokens/s;
                 detector_overhead: detect-only (detector on, termination
                 off) against full mode at the same launch shape;
                 ablation: blocks skipped and output error against full
                 decode with the scale test, the direction test or
                 patience taken out;
                 importance_first: block-mean keys and the importance
                 order on the GPU, then ART over that order;
                 multi_row: M = 1, 2, 4 query rows per sequence

Other modes (no timing line):
  --table    every configuration (cfg1..cfg5) in the library's default
        decomposition: full mode, then ART under generator readings A and
        B (cfg4 at patience 1, 2 and 4); one markdown row per measurement
        on stderr and a JSON object on stdout
  --profile-set   every profile case (cfg1..cfg5 in full and ART mode, the
        patience sweep, importance-first selection, a lone unit, a copy
        kernel) in one process, a marker kernel before each case, for
        rocprofv3 runs; prints a manifest line
  --summarize-set LOG TRACE_DIR [PMC_DIR ...]   per-case kernel times,
        algorithmic GB/s, copy-calibrated HBM traffic and other counters of
        such runs, into OUT.md and OUT.json
  --summarize-trace TRACE_DIR BENCH_LOG  turn a rocprofv3 --kernel-trace
        --stats run into a markdown summary next to the events timing
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BLOCK = 64
KERNEL_SOURCES = ("kv_cache_early_amd/csrc/art_kernels.hip", "kv_cache_early_amd/csrc/art_internal.h",
                  "kv_cache_early_amd/csrc/art_api.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "art_kernels_all_configs.json")
WORKLOAD = ("cfg3 large-batch paged decode: B=64, Hq=32, Hkv=8, d=128, ctx U[8192,32768], page 16 shuffled, "
            "block 64, eps (2e-3, 2e-4), patience 3, recent-first")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reading", default="B", choices=["A", "B"])
    ap.add_argument("--only", choices=["art", "full"], default=None,
                    help="time only this mode (for profiling runs); the line then reports it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=0, help="oracle sample size (0 = every unit)")
    ap.add_argument("--skip-extra", action="store_true", help="only the headline measurement")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0, choices=[0, 4, 8],
                    help="waves per workgroup in ART mode (0 = the library's choice)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-evicting read between steps")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run an elementwise copy of this many MiB `steps` times (counter calibration)")
    ap.add_argument("--table", action="store_true", help="measure every configuration (no timing line)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"))
    ap.add_argument("--profile-set", action="store_true",
                    help="run every profile case in one process, a marker kernel before each (no timing line)")
    ap.add_argument("--cases", default="", help="comma-separated profile cases (default: all)")
    ap.add_argument("--summarize-set", nargs="+", metavar="PATH",
                    help="LOG TRACE_DIR [PMC_DIR ...] of a --profile-set run; writes OUT.md and OUT.json")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--out", default="", help="summary output path")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def accounting(w, stop, issued):
    """Bytes moved per call: KV of the blocks counted + once-per-unit terms."""
    s = w.spec
    es = 2 if s.dtype == "bf16" else 4
    d, G = s.head_dim, s.group
    lens = w.context_lens.astype(np.int64)

    def kv_bytes(count):
        # valid tokens in the first `count` blocks of each unit's recency-first
        # traversal [0, T-1, T-2, ...]; only block T-1 can be partial
        tot = 0
        for b in range(s.batch):
            n = int(lens[b])
            T = (n + BLOCK - 1) // BLOCK
            partial = BLOCK - (n - (T - 1) * BLOCK)
            for h in range(s.num_kv_heads):
                c = int(count[b, h])
                if c > 0:
                    tot += c * BLOCK - (partial if (T == 1 or c >= 2) else 0)
        return tot * d * 2 * es

    units = s.batch * s.num_kv_heads
    per_unit = units * (G * d * es + G * d * 4 + 8)          # q, out, stop + issued
    pages = 0
    if s.page_size:
        pages = int(np.sum(np.minimum(issued, 10 ** 9))) * (BLOCK // s.page_size) * 4
    return kv_bytes(issued) + per_unit + pages, kv_bytes(stop) + per_unit + pages, kv_bytes


WAVES = 0  # art_params.waves for ART-mode calls (set from --waves)


def decode_kwargs(dev, w, mode, split_blocks, stream, flags=0, patience=None, order=None):
    s = w.spec
    return dict(dtype=dev.dtype_code, page_size=dev.page_size, block_table=dev.block_table,
                kept_blocks=dev.kept_blocks, kept_count=dev.kept_count, eps_scale=s.eps_scale, eps_dir=s.eps_dir,
                patience=s.patience if patience is None else patience, order=s.order if order is None else order,
                mode=mode, split_blocks=split_blocks, flags=flags, stream=stream.cuda_stream,
                waves=WAVES if mode == 1 else 0)


def eviction_buffer():
    """1 GiB of device memory, written once here (untimed, outside every
    timed loop) and only read afterwards."""
    import torch
    return torch.ones(1 << 28, dtype=torch.float32, device="cuda")


def write_eviction_buffer():
    import torch
    return torch.empty(1 << 30, dtype=torch.uint8, device="cuda")


def evict(buf):
    """Read all of `buf` (a sum): evicts the MALL (256 MB) and the L2s
    without leaving dirty lines for the next kernel to write back."""
    import torch
    torch.sum(buf)


def time_steps(dec, dev, w, mode, steps, warmup, split_blocks, flush, flags=0, order=None):
    import torch
    stream = torch.cuda.current_stream()
    kw = decode_kwargs(dev, w, mode, split_blocks, stream, flags, order=order)
    scratch = (write_eviction_buffer() if flush == "write" else eviction_buffer()) if flush else None
    r = dec.decode(dev.q, dev.k, dev.v, dev.context_lens, **kw)
    for _ in range(warmup):
        dec.decode(dev.q, dev.k, dev.v, dev.context_lens, out=r.out, stop_idx=r.stop_idx,
                   blocks_issued=r.blocks_issued, **kw)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        if scratch is not None:  # untimed: evicts the MALL and the L2s
            if flush == "write":
                scratch.fill_(1)
            else:
                evict(scratch)
        a.record(stream)
        dec.decode(dev.q, dev.k, dev.v, dev.context_lens, out=r.out, stop_idx=r.stop_idx,
                   blocks_issued=r.blocks_issued, **kw)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in evs]
    err = dec.device_error()
    if err != 0:
        raise RuntimeError(f"device error {err}")
    return dict(ms_mean=float(np.mean(ms)), ms_min=float(np.min(ms)), ms_median=float(np.median(ms)),
                wall_ms=wall * 1e3 / steps, out=r.out.cpu().numpy(), stop=r.stop_idx.cpu().numpy().astype(np.int64),
                issued=r.blocks_issued.cpu().numpy().astype(np.int64))


def measure(dec, w, mode, args, dev=None, flags=0, split_blocks=None, order=None):
    from workloads.device import to_device
    dev = dev or to_device(w)
    sb = args.split_blocks if split_blocks is None else split_blocks
    t = time_steps(dec, dev, w, mode, args.steps, args.warmup, sb, not args.no_flush, flags, order)
    loaded, algo, _ = accounting(w, t["stop"], t["issued"])
    sec = t["ms_mean"] * 1e-3
    Tp = w.traversal_lengths()
    res = dict(ms=t["ms_mean"], ms_min=t["ms_min"], ms_median=t["ms_median"], wall_ms=t["wall_ms"],
               gbs_loaded=loaded / sec / 1e9, gbs_algorithmic=algo / sec / 1e9,
               bytes_loaded=loaded, bytes_algorithmic=algo,
               pct_blocks_skipped=float(1 - t["stop"].sum() / Tp.sum()),
               wasted_frac=float((t["issued"].sum() - t["stop"].sum()) / Tp.sum()),
               effective_tokens_per_s=w.spec.batch / sec,
               context_tokens_per_s=float(w.context_lens.astype(np.int64).sum()) / sec)
    res["pct_of_peak"] = res["gbs_loaded"] / HBM_PEAK_GBS
    return res, t, dev


def ablation_report(dec, dev, w, split_blocks, full_out):
    """Stop-rule variants on the same workload, one call each: KV blocks
    skipped and the output error against full decode per (batch, kv head)
    unit (relative L2 over the unit's query heads)."""
    import torch
    from kv_cache_early_amd import ART_FLAG_NO_DIR, ART_FLAG_NO_SCALE
    s = w.spec
    Tp = w.traversal_lengths()
    ref = full_out.astype(np.float64).reshape(s.batch, s.num_kv_heads, -1)
    ref_n = np.linalg.norm(ref, axis=2)
    rows = {}
    for name, flags, p in (("art", 0, None), ("no_scale_test", ART_FLAG_NO_SCALE, None),
                           ("no_direction_test", ART_FLAG_NO_DIR, None), ("no_patience", 0, 1)):
        r = dec.decode(dev.q, dev.k, dev.v, dev.context_lens,
                       **decode_kwargs(dev, w, 1, split_blocks, torch.cuda.current_stream(), flags, p))
        torch.cuda.synchronize()
        if dec.device_error() != 0:
            raise RuntimeError(f"device error {dec.device_error()} in ablation {name}")
        out = r.out.cpu().numpy().astype(np.float64).reshape(s.batch, s.num_kv_heads, -1)
        stop = r.stop_idx.cpu().numpy().astype(np.int64)
        rel = np.linalg.norm(out - ref, axis=2) / np.maximum(ref_n, 1e-30)
        rows[name] = dict(patience=s.patience if p is None else p,
                          pct_blocks_skipped=round(float(1 - stop.sum() / Tp.sum()), 4),
                          rel_l2_mean=float(f"{rel.mean():.3e}"), rel_l2_max=float(f"{rel.max():.3e}"),
                          frac_units_rel_l2_over_1e_2=round(float((rel > 1e-2).mean()), 4))
    return rows


def time_call(fn, steps, flush):
    """Mean ms of `fn()` over `steps` calls (HIP events on the current
    stream, the caches evicted before each call unless `flush` is false)."""
    import torch
    scratch = eviction_buffer() if flush else None
    fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        if scratch is not None:
            evict(scratch)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.mean(ms)), r


def importance_report(dec, dev, w, args, head, full_out):
    """Importance-first traversal on the same workload: block-mean keys and
    the importance order of every block, both on the GPU, then ART walking
    that order (ART_ORDER_GIVEN), against recency-first ART (`head`)."""
    from dataclasses import replace as dc_replace
    from kv_cache_early_amd import ART_DT_BF16, ART_ORDER_GIVEN, ART_SELECT_IMPORTANCE
    s = w.spec
    mp = int(dev.block_table.shape[1])
    steps = max(3, args.steps // 3)
    means_ms, means = time_call(lambda: dec.block_means(dev.k, dev.context_lens, num_q_heads=s.num_q_heads,
                                                        dtype=dev.dtype_code, page_size=dev.page_size,
                                                        block_table=dev.block_table), steps, not args.no_flush)
    sel_ms, (kb, kc) = time_call(lambda: dec.select_blocks(dev.q, means, dev.context_lens, dtype=dev.dtype_code,
                                                           keep_frac=1.0, sink=0, recent=0,
                                                           order=ART_SELECT_IMPORTANCE, page_size=dev.page_size,
                                                           max_pages=mp), steps, not args.no_flush)
    if dec.device_error() != 0:
        raise RuntimeError("device error in block selection")
    k_bytes = int(w.context_lens.astype(np.int64).sum()) * s.num_kv_heads * s.head_dim * (2 if dev.dtype_code == ART_DT_BF16 else 4)
    dev_imp = dc_replace(dev, kept_blocks=kb, kept_count=kc)
    imp, imp_t, _ = measure(dec, w, 1, args, dev=dev_imp, order=ART_ORDER_GIVEN)
    ref = full_out.astype(np.float64).reshape(s.batch, s.num_kv_heads, -1)
    got = imp_t["out"].astype(np.float64).reshape(s.batch, s.num_kv_heads, -1)
    rel = np.linalg.norm(got - ref, axis=2) / np.maximum(np.linalg.norm(ref, axis=2), 1e-30)
    return dict(block_means_ms=round(means_ms, 4), block_means_gbs=round(k_bytes / (means_ms * 1e-3) / 1e9, 1),
                select_ms=round(sel_ms, 4), art_ms=round(imp["ms"], 4),
                pct_blocks_skipped=round(imp["pct_blocks_skipped"], 4),
                recency_first_pct_blocks_skipped=round(head["pct_blocks_skipped"], 4),
                rel_l2_vs_full_mean=float(f"{rel.mean():.3e}"),
                note="block means read every key once (meant for when blocks are written); the selection and "
                     "the ART call are per decode step")


def multi_row_report(dec, dev, w, args):
    """Multi-row queries on the same workload (M query rows per sequence,
    seeded draft-like rows): ART time and query rows per second for M = 1,
    2, 4; the M * 4 query vectors of a unit share its K/V loads."""
    import torch
    from workloads import multi_row_queries
    rows = {}
    for M in (1, 2, 4):
        if M == 1:
            q = dev.q
        else:
            qr = multi_row_queries(w, M)
            q = torch.from_numpy(qr.view(np.int16) if qr.dtype == np.uint16 else qr).to("cuda")
        stream = torch.cuda.current_stream()
        kw = decode_kwargs(dev, w, 1, args.split_blocks, stream)
        r = dec.decode(q, dev.k, dev.v, dev.context_lens, **kw)
        ms, _ = time_call(lambda: dec.decode(q, dev.k, dev.v, dev.context_lens, out=r.out, stop_idx=r.stop_idx,
                                             blocks_issued=r.blocks_issued, **kw), max(3, args.steps // 3),
                          not args.no_flush)
        if dec.device_error() != 0:
            raise RuntimeError(f"device error in multi-row M={M}")
        stop = r.stop_idx.cpu().numpy()
        rows[f"M{M}"] = dict(ms=round(ms, 4), query_rows_per_s=round(w.spec.batch * M / (ms * 1e-3), 1),
                             pct_blocks_skipped=round(float(1 - stop.sum() / w.traversal_lengths().sum()), 4))
    return rows


def copy_leg(mib, steps):
    """Elementwise copy (y = x * 1) of `mib` MiB: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.mul(x, 1.0, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        torch.mul(x, 1.0, out=y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return dict(bytes_read=n * 4, bytes_written=n * 4, ms=ms, gbs=2 * n * 4 / (ms * 1e-3) / 1e9)


CPU_WORKERS_MAX = 12  # with the bench process itself, at most 13 processes that a profiler may attach to the GPU


def _oracle_worker(conn, spec, units, outs, stops, mode):
    """One worker of the cpu_baseline leg, in a spawned interpreter.

    Draws its units' inputs from the workload's seeds (the same generator
    calls that built the GPU's arrays), reports ready with a digest of its
    first unit, waits for "go", then runs the oracle and the acceptance rule
    on each unit and sends back per-unit figures and its compute time."""
    from threadpoolctl import threadpool_limits

    import oracle as orc
    from oracle.acceptance import unit_agreement
    from workloads.gen import draw_context_lens, draw_unit, select_kept_blocks
    try:
        with threadpool_limits(1):
            lens = draw_context_lens(spec)
            data = []
            for (b, h) in units:
                n = int(lens[b])
                q, K, V = draw_unit(spec, b, h, n)
                kept = select_kept_blocks(spec, q, K, n) if spec.kept_frac > 0 else None
                data.append((q, K, V, n, kept))
            q, K, V = data[0][:3]
            conn.send(("ready", hashlib.sha256(q.tobytes() + K.tobytes() + V.tobytes()).hexdigest()))
            conn.recv()
            t0 = time.perf_counter()
            rows = []
            for (b, h), (q, K, V, n, kept), out_u, sg in zip(units, data, outs, stops):
                r = orc.art_unit(orc.widen(q, spec.dtype), orc.widen(K, spec.dtype), orc.widen(V, spec.dtype), n,
                                 spec.block_size, spec.eps_scale, spec.eps_dir, spec.patience, spec.order, kept,
                                 mode, 0)
                a = unit_agreement(r, out_u, int(sg), spec.eps_scale, spec.eps_dir)
                rows.append((b, h, int(r.stop), bool(a.stop_equal), bool(a.excused), bool(a.output_ok),
                             float(a.rel_l2), float(a.max_abs)))
            conn.send(("done", rows, time.perf_counter() - t0))
    except BaseException as e:  # noqa: BLE001 - reported to the parent, which raises
        conn.send(("error", repr(e)))
    finally:
        conn.close()


def cpu_baseline(w, n_units, stop_gpu, out_gpu, kv_bytes, mode=1):
    """The fp64 oracle as it stands over the workload's units (all, or a
    bounded sample), in a pool of single-threaded spawned workers, each of
    which also applies the acceptance rule to the GPU's stop and output."""
    import multiprocessing as mp

    from oracle import gather_unit
    s = w.spec
    G = s.group
    allu = [(b, h) for b in range(s.batch) for h in range(s.num_kv_heads)]
    if n_units and n_units < len(allu):
        rng = np.random.default_rng(0)
        pick = sorted(allu[i] for i in rng.choice(len(allu), size=n_units, replace=False))
    else:
        pick = allu
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    nw = max(1, min(CPU_WORKERS_MAX, avail, len(pick)))
    # longest context first onto the least loaded worker (the oracle's cost
    # grows with the context length)
    shares = [[] for _ in range(nw)]
    load = [0] * nw
    for u in sorted(pick, key=lambda u: -int(w.context_lens[u[0]])):
        i = int(np.argmin(load))
        shares[i].append(u)
        load[i] += int(w.context_lens[u[0]])
    ctx = mp.get_context("spawn")
    procs, conns = [], []
    try:
        for sh in shares:
            parent, child = ctx.Pipe()
            outs = [np.asarray(out_gpu[b, h * G:(h + 1) * G], dtype=np.float64) for (b, h) in sh]
            stops = [int(stop_gpu[b, h]) for (b, h) in sh]
            p = ctx.Process(target=_oracle_worker, args=(child, s, sh, outs, stops, mode), daemon=True)
            p.start()
            child.close()
            procs.append(p)
            conns.append(parent)
        for sh, c in zip(shares, conns):
            msg = c.recv()
            if msg[0] != "ready":
                raise RuntimeError(f"oracle worker failed: {msg[1]}")
            # the worker's inputs are the GPU's: same bytes for its first unit
            b, h = sh[0]
            n = int(w.context_lens[b])
            K, V = gather_unit(w.k, w.v, b, h, n, s.page_size, w.block_table)
            q = np.ascontiguousarray(w.q[b, h * G:(h + 1) * G])
            dig = hashlib.sha256(q.tobytes() + np.ascontiguousarray(K).tobytes()
                                 + np.ascontiguousarray(V).tobytes()).hexdigest()
            if dig != msg[1]:
                raise RuntimeError(f"oracle worker drew different inputs for unit {(b, h)}")
        t0 = time.perf_counter()
        for c in conns:
            c.send("go")
        rows, busy = [], []
        for c in conns:
            msg = c.recv()
            if msg[0] != "done":
                raise RuntimeError(f"oracle worker failed: {msg[1]}")
            rows += msg[1]
            busy.append(msg[2])
        el = time.perf_counter() - t0
    finally:
        for c in conns:
            c.close()
        for p in procs:
            p.join(timeout=30)
            if p.is_alive():
                p.kill()
    count = np.zeros((s.batch, s.num_kv_heads), dtype=np.int64)
    for (b, h, so, *_rest) in rows:
        count[b, h] = so
    kv = kv_bytes(count)
    n_eq = sum(r[3] for r in rows)
    n_exc = sum(r[4] for r in rows)
    n_out = sum(r[5] for r in rows)
    unexcused = len(rows) - n_eq - n_exc
    what = "every" if len(pick) == len(allu) else f"{len(pick)} of {len(allu)}"
    return dict(value=round(kv / el / 1e9, 4), unit="GB/s", cores=nw, kind="oracle",
                sample=f"{what} (batch, kv head) units of the same workload ({len(allu)} units) in {nw} "
                       f"single-threaded worker processes (each draws its units from the workload's seeds; the "
                       f"first unit of each is checked byte for byte against the GPU's inputs); fp64 numpy "
                       f"oracle: all prefix outputs and the stop rule; {el:.2f} s wall "
                       f"({sum(busy):.1f} worker-seconds); GB/s on the KV bytes of the blocks up to its stop",
                seconds=round(el, 3), worker_seconds=round(sum(busy), 2),
                parity=dict(units=len(rows), stop_equal=int(n_eq), excused=int(n_exc), unexcused=int(unexcused),
                            outputs_ok=int(n_out), worst_rel_l2=float(max(r[6] for r in rows)),
                            worst_abs=float(max(r[7] for r in rows)),
                            rule="stop equal or within 1e-4 of a threshold; out vs oracle O^(stop_gpu): "
                                 "rel-L2 <= 1e-3, max-abs <= 4e-3"))


def traffic_from_summary(tag):
    """HBM bytes per launch of profile case `tag` from the committed counter
    summary, if it was taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash():
        return None
    for c in t.get("cases", []):
        if c.get("tag") == tag:
            return c.get("traffic_bytes_per_launch")
    return None


# ---------------------------------------------------------------------------
# summaries of rocprofv3 runs
# ---------------------------------------------------------------------------
def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for p in files:
        with open(p) as f:
            rows += list(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter, name_pred):
    """Mean over dispatches of the counter (summed over its instances per dispatch)."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not name_pred(r.get("Kernel_Name", "")):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for the kernel")
    return float(np.mean(list(per.values()))), len(per)


def summarize_trace(args):
    """Markdown summary of a kernel-trace run of `bench.py --only art --skip-extra ...`.

    The average over the last `steps` decode dispatches (the timed, cache-cold
    calls) is set beside the HIP-events time of the same run."""
    trace_dir, log = args.summarize_trace
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    with open(stats) as f:
        rows = list(csv.DictReader(f))
    with open(trace) as f:
        tr = [r for r in csv.DictReader(f) if "art_decode_kernel" in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    line = None
    with open(log) as f:
        for l in f:
            l = l.strip()
            if l.startswith("{") and '"metric"' in l:
                line = json.loads(l)
    steps = line["steps"] if line else len(tr)
    timed = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr[-steps:]]
    mode = line["config"].get("mode", "ART") if line else "ART"
    md = ["# rocprofv3 kernel trace: art_decode_kernel (bf16, G=4, paged), " + WORKLOAD + f", generator B, {mode} mode",
          "", "Command (repository root):", "", "```", args.command, "```", "",
          "## --stats summary (all dispatches of the run)", "",
          "| kernel | calls | average us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['Name'][:100]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    md += ["", f"## The {len(timed)} timed decode dispatches (cache-cold; the earlier ones are warmup)", "",
           f"- kernel-trace average: {np.mean(timed):.1f} us (min {np.min(timed):.1f}, max {np.max(timed):.1f})"]
    if line:
        md += [f"- HIP events around the same calls (bench.py, launch stream): {line['ms_per_step'] * 1e3:.1f} us "
               f"mean",
               f"- value: {line['value']} {line['unit']} on loaded bytes; roofline achieved "
               f"{line['roofline']['achieved']} GB/s on algorithmic bytes ({line['roofline']['frac']:.3f} of 8 TB/s)",
               f"- blocks skipped: {line.get('pct_blocks_skipped')}"]
    md += ["", "The reduction kernels are the untimed 1 GiB cache-evicting read between timed calls (a sum); "
           "the FillFunctor kernel writes that buffer once before the loop; __amd_rocclr_fillBufferAligned entries clear the "
           "sum's 4-byte output; __amd_rocclr_copyBuffer entries are host-device copies of inputs and results."]
    with open(args.out, "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


# ---------------------------------------------------------------------------
# profile set: every configuration in one process, cases split by markers
# ---------------------------------------------------------------------------
# (tag, config, generator reading, mode 0 full / 1 ART, patience or None, spec overrides, kind)
PROFILE_CASES = (
    ("cfg1-full", 1, "A", 0, None, {}, "decode"),
    ("cfg1-A", 1, "A", 1, None, {}, "decode"),
    ("cfg1-B", 1, "B", 1, None, {}, "decode"),
    ("cfg2-full", 2, "A", 0, None, {}, "decode"),
    ("cfg2-A", 2, "A", 1, None, {}, "decode"),
    ("cfg2-B", 2, "B", 1, None, {}, "decode"),
    ("cfg3-full", 3, "A", 0, None, {}, "decode"),
    ("cfg3-A", 3, "A", 1, None, {}, "decode"),
    ("cfg3-B", 3, "B", 1, None, {}, "decode"),
    ("cfg3-B-importance", 3, "B", 1, None, {}, "select"),
    ("cfg4-full", 4, "A", 0, None, {}, "decode"),
    ("cfg4-A-p2", 4, "A", 1, 2, {}, "decode"),
    ("cfg4-B-p1", 4, "B", 1, 1, {}, "decode"),
    ("cfg4-B-p2", 4, "B", 1, 2, {}, "decode"),
    ("cfg4-B-p4", 4, "B", 1, 4, {}, "decode"),
    ("cfg5-full", 5, "A", 0, None, {}, "decode"),
    ("cfg5-A", 5, "A", 1, None, {}, "decode"),
    ("cfg5-B", 5, "B", 1, None, {}, "decode"),
    ("lone-B", 2, "B", 1, None, dict(batch=1, num_q_heads=4, num_kv_heads=1), "decode"),
    # the same unit walked by one workgroup (split_blocks >= its traversal)
    ("lone-B-1item", 2, "B", 1, None, dict(batch=1, num_q_heads=4, num_kv_heads=1), "decode", 1 << 20),
)
MARKER_KERNEL = "spin_kernel"  # torch.cuda._sleep's kernel: one before each case


def _marker():
    import torch
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()


def profile_set(args):
    """Run the profile cases in one process (for rocprofv3 runs): a marker
    kernel, then the case's calls (1 + warmup + steps, the last `steps` timed
    with the caches evicted before each); prints one JSON manifest line."""
    import dataclasses

    import torch
    from kv_cache_early_amd import ART_ORDER_GIVEN, ART_SELECT_IMPORTANCE, ArtDecoder
    from workloads import config, make_workload
    from workloads.device import to_device

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    dec = ArtDecoder()
    want = set(args.cases.split(",")) if args.cases else None
    cases = [c for c in PROFILE_CASES if want is None or c[0] in want]
    if want is not None and len(cases) != len(want):
        raise SystemExit(f"unknown cases: {sorted(want - {c[0] for c in cases})}")
    manifest, key, w, dev = [], None, None, None
    for tag, n, reading, mode, patience, over, kind, *split in cases:
        k = (n, reading, tuple(sorted(over.items())))
        if k != key:
            del w, dev
            torch.cuda.empty_cache()
            w = make_workload(config(n, reading, **over))
            dev = to_device(w)
            key = k
        base = w.spec
        if patience is not None:
            w.spec = dataclasses.replace(base, patience=patience)
        print(f"[profile] {tag}", file=sys.stderr, flush=True)
        _marker()
        rec = dict(tag=tag, workload=w.spec.name, reading=reading, mode="full" if mode == 0 else "ART",
                   patience=w.spec.patience, kind=kind, calls=1 + args.warmup + args.steps, steps=args.steps,
                   split_blocks=split[0] if split else 0)
        if kind == "select":
            s = w.spec
            mp = int(dev.block_table.shape[1])
            rec["calls_block_means"] = rec["calls_select"] = 1 + args.steps
            mms, means = time_call(lambda: dec.block_means(dev.k, dev.context_lens, num_q_heads=s.num_q_heads,
                                                           dtype=dev.dtype_code, page_size=dev.page_size,
                                                           block_table=dev.block_table), args.steps,
                                   not args.no_flush)
            sms, (kb, kc) = time_call(lambda: dec.select_blocks(dev.q, means, dev.context_lens,
                                                                dtype=dev.dtype_code, keep_frac=1.0, sink=0,
                                                                recent=0, order=ART_SELECT_IMPORTANCE,
                                                                page_size=dev.page_size, max_pages=mp),
                                      args.steps, not args.no_flush)
            k_bytes = int(w.context_lens.astype(np.int64).sum()) * s.num_kv_heads * s.head_dim * 2
            rec.update(block_means_ms=mms, select_ms=sms, block_means_bytes=k_bytes
                       + s.batch * s.num_kv_heads * int(w.num_blocks.max()) * s.head_dim * 4)
            dv = dataclasses.replace(dev, kept_blocks=kb, kept_count=kc)
            r, t, _ = measure(dec, w, mode, args, dev=dv, order=ART_ORDER_GIVEN)
            del dv, means, kb, kc
        else:
            r, t, _ = measure(dec, w, mode, args, dev=dev, split_blocks=split[0] if split else None)
        if dec.device_error() != 0:
            raise RuntimeError(f"device error in {tag}")
        rec.update(ms=r["ms"], bytes_algorithmic=int(r["bytes_algorithmic"]), bytes_loaded=int(r["bytes_loaded"]),
                   pct_blocks_skipped=r["pct_blocks_skipped"], wasted_frac=r["wasted_frac"],
                   units=int(w.spec.batch * w.spec.num_kv_heads), blocks_traversal=int(w.traversal_lengths().sum()),
                   blocks_stop=int(t["stop"].sum()), blocks_issued=int(t["issued"].sum()))
        manifest.append(rec)
        w.spec = base
        print(f"[profile] {tag}: {r['ms'] * 1e3:.1f} us, skipped {r['pct_blocks_skipped']:.3f}", file=sys.stderr,
              flush=True)
    if args.copy_mib:
        _marker()
        cp = copy_leg(args.copy_mib, args.steps)
        manifest.append(dict(tag="copy", kind="copy", calls=1 + args.steps, steps=args.steps, ms=cp["ms"],
                             copy_bytes_each_way=args.copy_mib * (1 << 20)))
    print(json.dumps({"profile_set": manifest, "steps": args.steps, "warmup": args.warmup,
                      "source_sha256": source_hash()}), flush=True)


def _dispatches(rows, time_key):
    """Group per-dispatch rows into cases, split at the marker kernel."""
    by = {}
    for r in rows:
        key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        by.setdefault(key, dict(name=r["Kernel_Name"], order=int(r[time_key]) if time_key else key, rows=[]))
        by[key]["rows"].append(r)
    seq = sorted(by.values(), key=lambda x: x["order"])
    cases, cur = [], None
    for d in seq:
        if MARKER_KERNEL in d["name"]:
            cur = []
            cases.append(cur)
        elif cur is not None:
            cur.append(d)
    return cases


_FAMILIES = (("art_decode_kernel", "decode"), ("art_combine_kernel", "combine"),
             ("block_means_kernel", "block_means"), ("select_kernel", "select"))


def _family(name):
    for pat, fam in _FAMILIES:
        if pat in name:
            return fam
    if "MulFunctor" in name or ("elementwise" in name.lower() and "mul" in name.lower()):
        return "copy"
    return None


def _timed(case_disp, rec, fam):
    """The timed dispatches of one kernel family in a case: its last `steps`."""
    ds = [d for d in case_disp if _family(d["name"]) == fam]
    return ds[-rec["steps"]:] if ds else []


def summarize_set(args):
    """Markdown + JSON summary of `bench.py --profile-set` under rocprofv3:
    argument 1 the run's log (its last JSON line is the manifest), argument 2
    a --kernel-trace directory, then any --pmc directories."""
    man_log, trace_dir, *pmc_dirs = args.summarize_set
    man = None
    with open(man_log) as f:
        for l in f:
            if l.startswith("{") and '"profile_set"' in l:
                man = json.loads(l)
    if man is None:
        raise SystemExit(f"no manifest line in {man_log}")
    recs = man["profile_set"]
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not trace:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    with open(trace[0]) as f:
        tcases = _dispatches(list(csv.DictReader(f)), "Start_Timestamp")
    if len(tcases) != len(recs):
        raise SystemExit(f"{len(tcases)} marked cases in the trace, {len(recs)} in the manifest")
    counters = {}  # (case index, family, counter) -> mean per dispatch
    for d in pmc_dirs:
        pcases = _dispatches(_counter_rows(d), None)
        if len(pcases) != len(recs):
            raise SystemExit(f"{len(pcases)} marked cases in {d}, {len(recs)} in the manifest")
        for i, (rec, cd) in enumerate(zip(recs, pcases)):
            for fam in ("decode", "combine", "block_means", "select", "copy"):
                ds = _timed(cd, rec, fam)
                if not ds:
                    continue
                names = {r["Counter_Name"] for dd in ds for r in dd["rows"]}
                for c in names:
                    vals = [sum(float(r["Counter_Value"]) for r in dd["rows"] if r["Counter_Name"] == c) for dd in ds]
                    counters[(i, fam, c)] = float(np.mean(vals))
    copy_i = next((i for i, r in enumerate(recs) if r["kind"] == "copy"), None)
    fs = ws = None
    if copy_i is not None and (copy_i, "copy", "FETCH_SIZE") in counters and (copy_i, "copy", "WRITE_SIZE") in counters:
        cb = recs[copy_i]["copy_bytes_each_way"]
        fs = cb / (counters[(copy_i, "copy", "FETCH_SIZE")] * 1024.0)
        ws = cb / (counters[(copy_i, "copy", "WRITE_SIZE")] * 1024.0)
    out = dict(source_sha256=man["source_sha256"], commands=args.command, steps=man["steps"],
               warmup=man["warmup"], fetch_scale=fs, write_scale=ws, cases=[])
    title = ("over every configuration" if len(recs) >= len(PROFILE_CASES)
             else "on " + ", ".join(r["tag"] for r in recs if r["kind"] != "copy"))
    md = [f"# rocprofv3: ART decode kernels {title}", "",
          "Each case: one untimed call, the warmup calls, then the timed calls, each after an untimed 1 GiB "
          "cache-evicting read. Kernel durations are the kernel-trace averages of the timed calls. "
          "`alg GB/s` is the algorithmic bytes (stop_idx x block bytes + per-unit q, out, stop and page-table "
          "bytes) per launch over that duration; `traffic` is FETCH_SIZE + WRITE_SIZE per launch scaled by what "
          "the same counters read for a copy kernel of known size.", "",
          "Commands (repository root):", "", "```", args.command, "```", ""]
    if fs is not None:
        md += [f"Copy calibration: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f} (bytes per KiB counted / 1024).", ""]
    md += ["| case | workload | mode | p | decode us (trace) | events us | alg GB/s | frac of 8 TB/s | "
           "traffic MB | alg MB | skipped | wasted | other kernels us |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    extra_counter_rows = []
    for i, (rec, cd) in enumerate(zip(recs, tcases)):
        if rec["kind"] == "copy":
            ds = _timed(cd, rec, "copy")
            dur = float(np.mean([(int(d["rows"][0]["End_Timestamp"]) - int(d["rows"][0]["Start_Timestamp"])) / 1e3
                                 for d in ds]))
            out["cases"].append(dict(tag="copy", kernel_us=dur, bytes_each_way=rec["copy_bytes_each_way"]))
            md.append(f"| copy | y = x * 1, {rec['copy_bytes_each_way'] >> 20} MiB | - | - | {dur:.1f} | "
                      f"{rec['ms'] * 1e3:.1f} | {2 * rec['copy_bytes_each_way'] / dur / 1e3:.0f} | "
                      f"{2 * rec['copy_bytes_each_way'] / dur / 1e3 / HBM_PEAK_GBS:.3f} | - | - | - | - | - |")
            continue
        fam_us = {}
        for fam in ("decode", "combine", "block_means", "select"):
            ds = _timed(cd, rec, fam)
            if ds:
                fam_us[fam] = float(np.mean([(int(d["rows"][0]["End_Timestamp"])
                                              - int(d["rows"][0]["Start_Timestamp"])) / 1e3 for d in ds]))
        dec_us = fam_us["decode"]
        alg = rec["bytes_algorithmic"]
        traffic = None
        if fs is not None and (i, "decode", "FETCH_SIZE") in counters and (i, "decode", "WRITE_SIZE") in counters:
            traffic = counters[(i, "decode", "FETCH_SIZE")] * 1024.0 * fs + counters[(i, "decode", "WRITE_SIZE")] * 1024.0 * ws
        kern_name = next(d["name"] for d in cd if _family(d["name"]) == "decode")
        c = dict(tag=rec["tag"], workload=rec["workload"], mode=rec["mode"], patience=rec["patience"],
                 kernel=kern_name, decode_kernel_us=dec_us, events_us=rec["ms"] * 1e3, bytes_algorithmic=alg,
                 bytes_loaded=rec["bytes_loaded"], gbs_algorithmic=alg / dec_us / 1e3,
                 frac_of_peak=alg / dec_us / 1e3 / HBM_PEAK_GBS, traffic_bytes_per_launch=traffic,
                 pct_blocks_skipped=rec["pct_blocks_skipped"], wasted_frac=rec["wasted_frac"],
                 other_kernels_us={k: v for k, v in fam_us.items() if k != "decode"})
        if rec["kind"] == "select":
            c.update(block_means_bytes=rec["block_means_bytes"],
                     block_means_gbs=rec["block_means_bytes"] / fam_us["block_means"] / 1e3)
            for fam in ("block_means", "select"):
                if fs is not None and (i, fam, "FETCH_SIZE") in counters and (i, fam, "WRITE_SIZE") in counters:
                    c[f"{fam}_traffic_bytes"] = (counters[(i, fam, "FETCH_SIZE")] * 1024.0 * fs
                                                 + counters[(i, fam, "WRITE_SIZE")] * 1024.0 * ws)
        sq = {cn: v for (j, fam, cn), v in counters.items() if j == i and fam == "decode"
              and cn not in ("FETCH_SIZE", "WRITE_SIZE")}
        if sq:
            c["counters_per_dispatch"] = sq
            extra_counter_rows.append((rec["tag"], sq))
        out["cases"].append(c)
        others = ", ".join(f"{k} {v:.1f}" for k, v in c["other_kernels_us"].items()) or "-"
        md.append(f"| {rec['tag']} | {rec['workload']} | {rec['mode']} | {rec['patience']} | {dec_us:.1f} | "
                  f"{rec['ms'] * 1e3:.1f} | {c['gbs_algorithmic']:.0f} | {c['frac_of_peak']:.3f} | "
                  f"{'-' if traffic is None else f'{traffic / 1e6:.1f}'} | {alg / 1e6:.1f} | "
                  f"{100 * rec['pct_blocks_skipped']:.1f}% | {100 * rec['wasted_frac']:.1f}% | {others} |")
    md += ["", "Decode kernel instance per case:", ""]
    md += [f"- {c['tag']}: `{c['kernel']}`" for c in out["cases"] if "kernel" in c]
    sel = [c for c in out["cases"] if "block_means_gbs" in c]
    for c in sel:
        md += ["", f"Block means ({c['tag']}): {c['other_kernels_us']['block_means']:.1f} us, "
                   f"{c['block_means_bytes'] / 1e6:.1f} MB algorithmic (every key once + the means), "
                   f"{c['block_means_gbs']:.0f} GB/s; select: {c['other_kernels_us']['select']:.1f} us"
               + (f"; traffic block means {c['block_means_traffic_bytes'] / 1e6:.1f} MB, select "
                  f"{c['select_traffic_bytes'] / 1e6:.1f} MB" if "select_traffic_bytes" in c else "")]
    if extra_counter_rows:
        names = sorted({k for _, sq in extra_counter_rows for k in sq})
        md += ["", "## Other counters, decode kernel, mean per dispatch", "",
               "| case | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for tag, sq in extra_counter_rows:
            md.append(f"| {tag} | " + " | ".join(f"{sq[n]:.4g}" if n in sq else "-" for n in names) + " |")
    with open(args.out + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    with open(args.out + ".json", "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(md))


def config_table(args):
    """Every configuration in the library's default decomposition."""
    import dataclasses

    import torch
    from kv_cache_early_amd import ArtDecoder
    from workloads import config, make_workload
    from workloads.device import to_device

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    dec = ArtDecoder()
    rows = []

    def row(n, reading, mode, r, patience):
        rec = dict(config=n, reading=reading, mode="full" if mode == 0 else "ART", patience=patience,
                   **{k: round(float(r[k]), 4) for k in ("ms", "ms_median", "gbs_loaded", "gbs_algorithmic",
                                                          "pct_blocks_skipped", "wasted_frac")})
        rows.append(rec)
        print(f"| cfg{n} | {rec['mode']} | {reading} | {patience} | {rec['ms'] * 1e3:.0f} µs | "
              f"{rec['gbs_loaded']:.0f} GB/s | {rec['gbs_algorithmic']:.0f} GB/s | "
              f"{100 * rec['pct_blocks_skipped']:.1f}% | {100 * rec['wasted_frac']:.1f}% |", file=sys.stderr, flush=True)

    print("| config | mode | generator | patience | time | loaded | useful | skipped | wasted |\n"
          "|---|---|---|---|---|---|---|---|---|", file=sys.stderr, flush=True)
    for n in (1, 2, 3, 4, 5):
        for reading in ("A", "B"):
            w = make_workload(config(n, reading))
            dev = to_device(w)
            if reading == "A":  # full mode reads every block whatever the keys
                r, _, _ = measure(dec, w, 0, args, dev=dev)
                row(n, "-", 0, r, "-")
            for p in ((1, 2, 4) if n == 4 else (w.spec.patience,)):
                w.spec = dataclasses.replace(w.spec, patience=p)
                r, _, _ = measure(dec, w, 1, args, dev=dev)
                row(n, reading, 1, r, p)
            del dev, w
            torch.cuda.empty_cache()
    print(json.dumps({"table": rows, "steps": args.steps, "warmup": args.warmup,
                      "cache_eviction": "untimed 1 GiB read before each timed call"}))


def main():
    global WAVES
    args = parse()
    WAVES = args.waves
    if args.table:
        return config_table(args)
    if args.summarize_trace:
        return summarize_trace(args)
    if args.summarize_set:
        return summarize_set(args)
    if args.profile_set:
        return profile_set(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this build runs on one GPU; ART units are independent, so --gpus > 1 "
                                   "would shard (batch, kv head) units across devices with no exchange "
                                   "(not built)"}))
        sys.exit(2)
    import torch
    from kv_cache_early_amd import ArtDecoder
    from workloads import config, make_workload

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    dec = ArtDecoder()
    spec = config(3, args.reading)
    t0 = time.perf_counter()
    w = make_workload(spec)
    gen_s = time.perf_counter() - t0
    print(f"[bench] generated {spec.name} reading {args.reading}: {w.kv_bytes_resident() / 1e9:.2f} GB KV "
          f"in {gen_s:.1f} s", file=sys.stderr, flush=True)

    head_mode = 0 if args.only == "full" else 1
    head, head_t, dev = measure(dec, w, head_mode, args)
    print(f"[bench] {'full' if head_mode == 0 else 'ART'}: {head['ms']:.3f} ms {head['gbs_loaded']:.0f} GB/s "
          f"skip {head['pct_blocks_skipped']:.3f}", file=sys.stderr, flush=True)
    extra = {}
    if head_mode == 1 and not args.no_flush and not args.skip_extra:
        # the headline call once more with the caches evicted by a 1 GiB write
        # instead: the write's dirty lines are written back during the call
        tw = time_steps(dec, dev, w, 1, args.steps, args.warmup, args.split_blocks, "write")
        extra["eviction_check"] = {"ms_after_1GiB_read": round(head["ms"], 4),
                                   "ms_after_1GiB_write": round(tw["ms_mean"], 4),
                                   "note": "headline uses the read; a write leaves dirty lines whose write-back "
                                           "lands in the timed call"}
        print(f"[bench] ART after a write eviction: {tw['ms_mean']:.3f} ms", file=sys.stderr, flush=True)
    if not args.skip_extra and args.only is None:
        full_res, full_t, _ = measure(dec, w, 0, args, dev=dev)
        extra["full_mode"] = {k: round(full_res[k], 4) for k in ("ms", "gbs_loaded", "pct_of_peak",
                                                                 "effective_tokens_per_s")}
        print(f"[bench] full: {full_res['ms']:.3f} ms {full_res['gbs_loaded']:.0f} GB/s", file=sys.stderr, flush=True)
        if head_mode == 1:
            from kv_cache_early_amd import ART_FLAG_DETECT_ONLY
            # same launch shape on both sides (one work item per unit, as ART
            # mode runs here): the difference is the detector alone
            one = 10 ** 9
            f1, _, _ = measure(dec, w, 0, args, dev=dev, split_blocks=one)
            det, det_t, _ = measure(dec, w, 1, args, dev=dev, flags=ART_FLAG_DETECT_ONLY, split_blocks=one)
            extra["detector_overhead"] = dict(
                full_one_item_ms=round(f1["ms"], 4), detect_only_ms=round(det["ms"], 4),
                overhead=round(det["ms"] / f1["ms"] - 1, 4),
                stops_equal_art=bool(np.array_equal(det_t["stop"], head_t["stop"])),
                note="detector on, termination off (every block read) against full mode, both one work item "
                     "per (batch, kv head) unit")
            print(f"[bench] detect-only: {det['ms']:.3f} ms vs full one-item {f1['ms']:.3f} ms "
                  f"(overhead {det['ms'] / f1['ms'] - 1:+.3%})", file=sys.stderr, flush=True)
            extra["ablation"] = ablation_report(dec, dev, w, args.split_blocks, full_t["out"])
            print(f"[bench] ablation: {extra['ablation']}", file=sys.stderr, flush=True)
            extra["importance_first"] = importance_report(dec, dev, w, args, head, full_t["out"])
            print(f"[bench] importance-first: {extra['importance_first']}", file=sys.stderr, flush=True)
            extra["multi_row"] = multi_row_report(dec, dev, w, args)
            print(f"[bench] multi-row: {extra['multi_row']}", file=sys.stderr, flush=True)
    traffic = traffic_from_summary(f"cfg3-{args.reading}" if head_mode == 1 else "cfg3-full")
    roof = dict(bound="hbm", achieved=round(head["gbs_algorithmic"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(head["gbs_algorithmic"] / HBM_PEAK_GBS, 4),
                traffic=None if traffic is None else round(traffic),
                traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                algorithmic_bytes=int(head["bytes_algorithmic"]), kernel="art_decode_kernel",
                kernel_ms=round(head["ms"], 4))

    if args.copy_mib:
        cp = copy_leg(args.copy_mib, args.steps)
        extra["copy_kernel"] = cp
        print(f"[bench] copy {args.copy_mib} MiB: {cp['ms']:.3f} ms {cp['gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        _, _, kv_bytes = accounting(w, head_t["stop"], head_t["issued"])
        cpu = cpu_baseline(w, args.cpu_units, head_t["stop"], head_t["out"], kv_bytes, head_mode)
        print(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s over {cpu['seconds']:.2f} s on {cpu['cores']} workers; "
              f"parity {cpu['parity']}", file=sys.stderr, flush=True)

    if not args.skip_extra and args.only is None:
        other = "A" if args.reading == "B" else "B"
        del dev
        w2 = make_workload(config(3, other))
        r2, _, _ = measure(dec, w2, 1, args)
        extra[f"reading_{other}"] = {k: round(r2[k], 4) for k in ("ms", "gbs_loaded", "pct_of_peak",
                                                                  "pct_blocks_skipped", "effective_tokens_per_s")}

    line = {
        "metric": "decode-attn KV GB/s achieved (% of HBM peak) + effective tokens/s; % KV blocks skipped",
        "value": round(head["gbs_loaded"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Llama-shaped keys with recency bias, sinks and low-score/high-value tokens)",
        "config": {"workload": WORKLOAD, "generator": args.reading, "mode": "full" if head_mode == 0 else "ART",
                   "global_batch": spec.batch, "seq_len": "8192-32768", "parallelism": "single GPU",
                   "cache_flush_between_steps": not args.no_flush,
                   "cache_eviction": "untimed 1 GiB read (sum) before each timed step" if not args.no_flush else None},
        "pct_of_peak": round(head["pct_of_peak"], 4),
        "effective_tokens_per_s": round(head["effective_tokens_per_s"], 1),
        "context_tokens_per_s": round(head["context_tokens_per_s"], 1),
        "pct_blocks_skipped": round(head["pct_blocks_skipped"], 4),
        "wasted_block_frac": round(head["wasted_frac"], 4),
        "ms_min": round(head["ms_min"], 4),
        "ms_median": round(head["ms_median"], 4),
        "wall_ms_per_step": round(head["wall_ms"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
