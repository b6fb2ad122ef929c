#!/usr/bin/env python3
"""Benchmark: ART decode attention on one MI355X.

A step is one art_decode call (all kernels of the hot path) over the whole
batch of the large-batch paged decode workload: batch 64, 32 query / 8 KV
heads, head_dim 128, bf16 KV in 16-token pages with a shuffled block table,
context lengths uniform in [8192, 32768], 64-token ART blocks,
eps_scale 2e-3, eps_dir 2e-4, patience 3, recency-first traversal.  Inputs
are generated once (seeded, synthetic) and are resident in HBM before the
timed region.

Reported (one JSON line on stdout):
  value          KV GB/s on the bytes actually loaded (blocks_issued x block
                 bytes + per-unit q / out / block-table bytes) / step time,
                 ART mode, generator reading "B" (Llama-shaped keys, where
                 the criterion fires)
  roofline       algorithmic bytes (stop_idx x block bytes + per-unit terms)
                 per launch / average launch time (HIP events on the
                 decode stream) against the 8 TB/s HBM peak
  cpu_baseline   the fp64 numpy oracle on a bounded sample of the same units
  extra fields   full-attention mode and generator reading "A" on the same
                 shapes, % KV blocks skipped, effective tokens/s
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BLOCK = 64


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reading", default="B", choices=["A", "B"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=0, help="oracle sample size (0 = sized to ~15 s)")
    ap.add_argument("--skip-extra", action="store_true", help="only the headline measurement")
    ap.add_argument("--split-blocks", type=int, default=0)
    return ap.parse_args()


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
    return kv_bytes(issued) + per_unit + pages, kv_bytes(stop) + per_unit + pages


def time_steps(dec, dev, w, mode, steps, warmup, split_blocks):
    import torch
    s = w.spec
    stream = torch.cuda.current_stream()
    kw = dict(dtype=dev.dtype_code, page_size=dev.page_size, block_table=dev.block_table,
              kept_blocks=dev.kept_blocks, kept_count=dev.kept_count, eps_scale=s.eps_scale, eps_dir=s.eps_dir,
              patience=s.patience, order=s.order, mode=mode, split_blocks=split_blocks,
              stream=stream.cuda_stream)
    r = dec.decode(dev.q, dev.k, dev.v, dev.context_lens, **kw)
    for _ in range(warmup):
        dec.decode(dev.q, dev.k, dev.v, dev.context_lens, out=r.out, stop_idx=r.stop_idx,
                   blocks_issued=r.blocks_issued, **kw)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
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


def measure(dec, w, mode, steps, warmup, split_blocks, dev=None):
    from workloads.device import to_device
    dev = dev or to_device(w)
    t = time_steps(dec, dev, w, mode, steps, warmup, split_blocks)
    loaded, algo = accounting(w, t["stop"], t["issued"])
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


def cpu_baseline(w, n_units, stop_gpu):
    """The fp64 oracle as it stands on a bounded sample of the workload's units."""
    import oracle as orc
    from threadpoolctl import threadpool_info
    s = w.spec
    rng = np.random.default_rng(0)
    allu = [(b, h) for b in range(s.batch) for h in range(s.num_kv_heads)]
    pick = sorted(allu[i] for i in rng.choice(len(allu), size=min(n_units, len(allu)), replace=False))
    t0 = time.perf_counter()
    out, stop, res = orc.art_decode_workload(w, units=pick, keep_results=True)
    el = time.perf_counter() - t0
    es = 2 if s.dtype == "bf16" else 4
    kv = 0
    rel = []
    agree = 0
    for (b, h), r in res.items():
        kv += min(int(r.stop) * BLOCK, int(w.context_lens[b])) * s.head_dim * 2 * es
        full = r.O[-1]
        rel.append(float(np.linalg.norm(r.out - full) / np.linalg.norm(full)))
        agree += int(r.stop == stop_gpu[b, h])
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return dict(value=kv / el / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{len(pick)} of {len(allu)} (batch, kv head) units of the same workload, fp64 numpy, "
                       f"all prefix outputs and the stop rule; {el:.1f} s wall",
                seconds=el, rel_l2_vs_full_median=float(np.median(rel)), stop_agree=f"{agree}/{len(pick)}")


def main():
    args = parse()
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

    art_res, art_t, dev = measure(dec, w, 1, args.steps, args.warmup, args.split_blocks)
    print(f"[bench] ART: {art_res['ms']:.3f} ms {art_res['gbs_loaded']:.0f} GB/s "
          f"skip {art_res['pct_blocks_skipped']:.3f}", file=sys.stderr, flush=True)
    extra = {}
    if not args.skip_extra:
        full_res, _, _ = measure(dec, w, 0, args.steps, args.warmup, args.split_blocks, dev=dev)
        extra["full_mode"] = {k: full_res[k] for k in ("ms", "gbs_loaded", "pct_of_peak", "effective_tokens_per_s")}
        print(f"[bench] full: {full_res['ms']:.3f} ms {full_res['gbs_loaded']:.0f} GB/s", file=sys.stderr, flush=True)
    roof = dict(bound="hbm", achieved=round(art_res["gbs_algorithmic"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(art_res["gbs_algorithmic"] / HBM_PEAK_GBS, 4), traffic=None)

    cpu = None
    if not args.no_cpu_baseline:
        n = args.cpu_units or 256
        cpu = cpu_baseline(w, n, art_t["stop"])
        print(f"[bench] cpu oracle: {cpu['value']:.2f} GB/s over {cpu['seconds']:.1f} s", file=sys.stderr, flush=True)

    if not args.skip_extra:
        other = "A" if args.reading == "B" else "B"
        del dev
        w2 = make_workload(config(3, other))
        r2, _, _ = measure(dec, w2, 1, args.steps, args.warmup, args.split_blocks)
        extra[f"reading_{other}"] = {k: r2[k] for k in ("ms", "gbs_loaded", "pct_of_peak", "pct_blocks_skipped",
                                                        "effective_tokens_per_s")}

    line = {
        "metric": "decode-attn KV GB/s achieved (% of HBM peak) + effective tokens/s; % KV blocks skipped",
        "value": round(art_res["gbs_loaded"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(art_res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Llama-shaped keys with recency bias, sinks and low-score/high-value tokens)",
        "config": {"workload": "cfg3 large-batch paged decode: B=64, Hq=32, Hkv=8, d=128, ctx U[8192,32768], "
                               "page 16 shuffled, block 64, eps (2e-3, 2e-4), patience 3, recent-first",
                   "generator": args.reading, "mode": "ART", "global_batch": spec.batch, "seq_len": "8192-32768",
                   "parallelism": "single GPU"},
        "pct_of_peak": round(art_res["pct_of_peak"], 4),
        "effective_tokens_per_s": round(art_res["effective_tokens_per_s"], 1),
        "context_tokens_per_s": round(art_res["context_tokens_per_s"], 1),
        "pct_blocks_skipped": round(art_res["pct_blocks_skipped"], 4),
        "wasted_block_frac": round(art_res["wasted_frac"], 4),
        "ms_min": round(art_res["ms_min"], 4),
        "wall_ms_per_step": round(art_res["wall_ms"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
