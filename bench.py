#!/usr/bin/env python3
"""Benchmark: NVFP4 sparse-MLA decode on one MI355X.

One step = the whole hot path for one decode step of the workload: the
quantize-append of the step's new rows (one per token) plus one sparse
decode launch over every token's selected rows.  Inputs are synthetic and
seeded (synth/), resident in HBM before timing starts.

Default workload: 15 query tokens (one per sequence), 32 heads, top-2048
distinct picks from each sequence's 146,000 rows, 2.2M-row NVFP4 pool.

Timing: W untimed warm-up steps, then K timed steps.  By default the caches
are cold for every step: a 1 GiB read sweep runs between steps (outside the
per-step events) so neither the 256 MB Infinity Cache nor L2 holds the
gathered rows; the step's small inputs (q, index lists, block table, new
rows), which the kernels before attention have just written in a real decode
step, are read once after the sweep (--cold-inputs leaves them cold).  Every step is bracketed by HIP events on the stream the
kernels run on, with no event inside a step; `value` and `us_per_step`
come from that pass.  A second pass puts an event between the append and
the decode (`append_us`, `decode_us`).  A third pass repeats the steps with
the library's kernel timing on
(hipExtLaunchKernel events at each kernel's own start and end): those
durations give `decode_kernel_us`, the roofline figure and the comparators'
`*_kernel_us`.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--warm] [--no-comparators] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode µs/step + gathered HBM GB/s (NVFP4 KV, top-2048)"
HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 352
FP8_ROW_BYTES = 576

DESCRIPTIONS = {
    "tiny": "1 token x 16 heads, 256 picks of a 4,096-row NVFP4 pool",
    "decode15": "15 tokens (1 per sequence) x 32 heads, top-2048 of 146,000 rows each, 2.2M-row NVFP4 pool",
    "padded35": "35 tokens x 32 heads, contexts 256..8192 rows, 2048-slot lists padded with -1",
    "batch128": "128 tokens x 32 heads, top-2048 of 140K-146K rows via a 64-row block table, 1.63M-row pool",
    "prefill4k": "4096 tokens from 4 sequences x 32 heads, causal top-2048 (128 recent + 1920 older)",
}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode15")
    ap.add_argument("--warm", action="store_true", help="no cache flush between steps")
    ap.add_argument("--cold-inputs", action="store_true",
                    help="leave q, index lists and block table cold too (default: only the gathered rows)")
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0 = launch sizer)")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def _copy_calibration(mib: int, reps: int = 10):
    """A plain device-to-device copy of known size, for scaling HBM byte counters."""
    import torch

    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": reps}), flush=True)


def _copy_peak(torch, dev, mib: int = 512, reps: int = 5) -> float:
    """Device-to-device copy bandwidth on this machine (GB/s of bytes read + written)."""
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return round(2 * n / (best * 1e-3) / 1e9, 1)


class Timer:
    """Per-launch HIP events on torch's current stream (the stream the library uses)."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]

    def mark(self, i, k):
        self.ev[i][k].record()

    def spans(self, a, b):
        return [e[a].elapsed_time(e[b]) for e in self.ev]


def _gpu_run(args):
    import torch

    import nvfp4_compressed_sparse_mla_amd as mla
    from synth import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = make_workload(args.workload, dev)
    T, H, K = w.tokens, w.heads, w.topk
    rows = w.pool_rows
    cache = torch.empty((rows, ROW_BYTES), dtype=torch.uint8, device=dev)
    mla.quantize_append(w.latent, w.rope, torch.arange(rows, dtype=torch.int64, device=dev), cache)
    keep = w.append_slots >= 0
    app_slots = w.append_slots.clone()
    app_idx = torch.where(keep, w.append_slots, torch.zeros_like(w.append_slots))
    app_lat = w.latent[app_idx].contiguous()      # each token's own row, same values: the step is repeatable
    app_rope = w.rope[app_idx].contiguous()
    splits = args.splits or mla.num_splits(T, H, K)
    ws = mla.make_workspace(T, H, K, dev, splits)
    out = torch.empty((T, H, 512), dtype=w.q.dtype, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    flush = None if args.warm else torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    if flush is not None:
        flush.fill_(1.0)
    valid = w.valid_slots()
    gathered = valid * ROW_BYTES
    copy_gbs = _copy_peak(torch, dev)

    # The step's own small inputs (q, index lists, block table, the new rows)
    # are written by the kernels that precede attention in a decode step, so
    # after the sweep they are read once more to leave them in cache; only
    # the gathered cache rows stay cold.  --cold-inputs skips that.
    step_inputs = [w.q, w.indices, app_lat, app_rope, app_slots]
    if w.block_table is not None:
        step_inputs += [w.block_table, w.token_seq]

    def do_flush():
        if flush is not None:
            flush.sum()
            if not args.cold_inputs:
                for x in step_inputs:
                    x.sum()

    def step(tm=None, i=0, split=False):
        if tm:
            tm.mark(i, 0)
        mla.quantize_append(app_lat, app_rope, app_slots, cache)
        if tm and split:
            tm.mark(i, 1)
        mla.sparse_decode(w.q, cache, w.indices, w.sm_scale, block_table=w.block_table,
                          token_seq=w.token_seq, block_size=w.block_size, workspace=ws,
                          num_splits=splits, out=out, lse=lse)
        if tm:
            tm.mark(i, 2)

    for _ in range(args.warmup):
        do_flush()
        step()
    torch.cuda.synchronize()
    # pass A, the timed region: K steps, each bracketed by HIP events, no
    # instrumentation inside a step
    tm = Timer(torch, args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        do_flush()
        step(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # pass A2: the same steps with an event between the append and the decode
    # (the split into append_us and decode_us; that event costs the step time)
    tm2 = Timer(torch, max(20, args.steps // 2))
    for i in range(len(tm2.ev)):
        do_flush()
        step(tm2, i, split=True)
    torch.cuda.synchronize()
    # pass B: the same steps with the library's kernel timing on (each kernel's own
    # start/end events), for the roofline and the per-kernel figures
    # (the decode follows its append on the GPU with no host round trip in
    # between, as in pass A; the append's own duration is taken in a loop of
    # its own)
    kern_ms, app_kern_ms = [], []
    mla.kernel_timing(True)
    try:
        for i in range(max(20, args.steps // 2)):
            do_flush()
            mla.quantize_append(app_lat, app_rope, app_slots, cache)
            mla.sparse_decode(w.q, cache, w.indices, w.sm_scale, block_table=w.block_table,
                              token_seq=w.token_seq, block_size=w.block_size, workspace=ws,
                              num_splits=splits, out=out, lse=lse)
            kern_ms.append(mla.last_kernel_ms())
        for i in range(max(10, args.steps // 4)):
            do_flush()
            mla.quantize_append(app_lat, app_rope, app_slots, cache)
            app_kern_ms.append(mla.last_kernel_ms())
    finally:
        mla.kernel_timing(False)
    step_ms = tm.spans(0, 2)
    dec_ms = tm2.spans(1, 2)
    app_ms = tm2.spans(0, 1)
    res = {
        "T": T, "H": H, "K": K, "rows": rows, "splits": splits, "valid": valid, "gathered": gathered,
        "step_ms": statistics.mean(step_ms), "decode_ms": statistics.mean(dec_ms),
        "decode_ms_median": statistics.median(dec_ms),
        "decode_ms_p10": sorted(dec_ms)[len(dec_ms) // 10],
        "decode_ms_p90": sorted(dec_ms)[(9 * len(dec_ms)) // 10],
        "step_ms_median": statistics.median(step_ms),
        "step_ms_p10": sorted(step_ms)[len(step_ms) // 10],
        "step_ms_p90": sorted(step_ms)[(9 * len(step_ms)) // 10],
        "append_ms": statistics.mean(app_ms), "wall_ms_per_iter": 1e3 * wall / args.steps,
        "kernel_ms": statistics.mean(kern_ms), "kernel_ms_median": statistics.median(kern_ms),
        "append_kernel_ms": statistics.mean(app_kern_ms),
        "copy_gbs": copy_gbs,
        "append_bytes": int(app_lat.numel() * app_lat.element_size() + app_rope.numel() * app_rope.element_size()
                            + app_slots.numel() * 8 + int((app_slots >= 0).sum()) * ROW_BYTES),
    }

    if not args.no_comparators:
        res["comparators"] = _comparators(args, torch, mla, w, cache, dev, splits, do_flush)
    return res, w


def _comparators(args, torch, mla, w, cache, dev, splits, do_flush):
    """FP8-576 rows (same values, 576-byte rows) and the staged path
    (gather-dequant the selected NVFP4 rows into an FP8 buffer, then FP8 decode)."""
    T, H, K = w.tokens, w.heads, w.topk
    n = max(10, args.steps // 2)
    c8 = torch.empty((w.pool_rows, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    mla.fp8_quantize_append(w.latent, w.rope, torch.arange(w.pool_rows, device=dev), c8, 1.0)
    ws = mla.make_workspace(T, H, K, dev, splits)
    staged_rows = torch.empty((T * K, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    staged_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=w.q.dtype, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)

    def fp8_decode():
        mla.sparse_decode(w.q, c8, w.indices, w.sm_scale, fmt="fp8", block_table=w.block_table,
                          token_seq=w.token_seq, block_size=w.block_size, workspace=ws,
                          num_splits=splits, out=out, lse=lse)

    def staged(tm=None, i=0):
        mla.gather_dequant_fp8(cache, w.indices, 1.0, block_table=w.block_table, token_seq=w.token_seq,
                               block_size=w.block_size, rows=staged_rows, staged_indices=staged_idx)
        if tm:
            tm.mark(i, 1)
        mla.sparse_decode(w.q, staged_rows, staged_idx, w.sm_scale, fmt="fp8", workspace=ws,
                          num_splits=splits, out=out, lse=lse)

    r = {}
    for _ in range(3):
        do_flush(); fp8_decode(); do_flush(); staged()
    torch.cuda.synchronize()
    tm = Timer(torch, n)
    for i in range(n):
        do_flush()
        tm.mark(i, 0)
        fp8_decode()
        tm.mark(i, 2)
    torch.cuda.synchronize()
    r["fp8_576_decode_us"] = 1e3 * statistics.mean(tm.spans(0, 2))
    tm = Timer(torch, n)
    for i in range(n):
        do_flush()
        tm.mark(i, 0)
        staged(tm, i)
        tm.mark(i, 2)
    torch.cuda.synchronize()
    r["staged_total_us"] = 1e3 * statistics.mean(tm.spans(0, 2))
    r["staged_gather_dequant_us"] = 1e3 * statistics.mean(tm.spans(0, 1))
    r["staged_fp8_decode_us"] = 1e3 * statistics.mean(tm.spans(1, 2))
    # the same launches with kernel timing on: each kernel's own duration
    k_fp8, k_gather, k_sfp8 = [], [], []
    mla.kernel_timing(True)
    try:
        for i in range(n):
            do_flush()
            fp8_decode()
            k_fp8.append(mla.last_kernel_ms())
            do_flush()
            mla.gather_dequant_fp8(cache, w.indices, 1.0, block_table=w.block_table, token_seq=w.token_seq,
                                   block_size=w.block_size, rows=staged_rows, staged_indices=staged_idx)
            k_gather.append(mla.last_kernel_ms())
            mla.sparse_decode(w.q, staged_rows, staged_idx, w.sm_scale, fmt="fp8", workspace=ws,
                              num_splits=splits, out=out, lse=lse)
            k_sfp8.append(mla.last_kernel_ms())
    finally:
        mla.kernel_timing(False)
    r["fp8_576_decode_kernel_us"] = 1e3 * statistics.mean(k_fp8)
    r["staged_gather_dequant_kernel_us"] = 1e3 * statistics.mean(k_gather)
    r["staged_fp8_decode_kernel_us"] = 1e3 * statistics.mean(k_sfp8)
    r["staged_total_kernel_us"] = r["staged_gather_dequant_kernel_us"] + r["staged_fp8_decode_kernel_us"]
    return r


def _cpu_baseline(w, seconds):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: per pass, decode the sampled tokens' selected rows from
    their 352-byte encodings and run the FP64 attention."""
    import numpy as np

    from oracle import attention, codec

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    idx = w.indices.cpu().numpy().astype(np.int64)
    bt = None if w.block_table is None else w.block_table.cpu().numpy().astype(np.int64)
    seq = None if w.token_seq is None else w.token_seq.cpu().numpy().astype(np.int64)
    q = w.q.float().cpu().numpy().astype(np.float64)
    tokens = list(range(w.tokens))
    # the encoded rows the sample touches (setup, not timed): the pool is already encoded
    per_tok = []
    for t in tokens:
        v = idx[t][idx[t] >= 0]
        rows = attention.physical_rows(v, None if seq is None else int(seq[t]), bt, w.block_size,
                                       w.pool_rows)
        rows = rows[rows >= 0]
        sel = __import__("torch").from_numpy(rows).to(w.latent.device)
        lat16 = w.latent.index_select(0, sel).cpu().numpy().astype(np.float64)
        rope16 = w.rope.index_select(0, sel).cpu().numpy().astype(np.float64)
        per_tok.append(codec.nvfp4_encode_rows(lat16, rope16))
    def run(limit):
        done_bytes = 0
        n_tok = 0
        t0 = time.perf_counter()
        while True:
            for t in tokens:
                enc = per_tok[t]
                lat, rope = codec.nvfp4_decode_rows(enc)
                attention.sparse_mla_token(q[t], lat, rope, w.sm_scale)
                done_bytes += enc.shape[0] * ROW_BYTES
                n_tok += 1
                if time.perf_counter() - t0 > limit:
                    break
            if time.perf_counter() - t0 > limit:
                break
        return done_bytes, n_tok, time.perf_counter() - t0

    done_bytes, n_tok, el = run(seconds)
    out = {
        "value": done_bytes / el / 1e9, "unit": "GB/s", "cores": blas_threads,
        "kind": "oracle",
        "sample": f"{n_tok} token-passes of the {w.name} workload ({n_tok / max(1, len(tokens)):.1f} steps), "
                  f"NVFP4 row decode + FP64 attention, {el:.1f} s; host os.cpu_count()={os.cpu_count()}, "
                  f"affinity {len(os.sched_getaffinity(0))} cores",
        "us_per_step": 1e6 * el * len(tokens) / max(1, n_tok),
    }
    # the same with the BLAS pool limited to one thread (half the time budget)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            b1, n1, e1 = run(seconds / 2)
        out["single_thread"] = {"value": b1 / e1 / 1e9, "unit": "GB/s", "cores": 1,
                                "us_per_step": 1e6 * e1 * len(tokens) / max(1, n1),
                                "sample": f"{n1} token-passes, {e1:.1f} s"}
    except Exception:  # pragma: no cover
        pass
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_decode_nvfp4_hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "nvfp4_compressed_sparse_mla_amd", "csrc", f)
                  for f in ("decode.hip", "mla_device.h", "mla_launch.h")]


def _kernel_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(workload: str, splits: int):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, only if it was taken on the current kernel sources
    and the same workload and split count; otherwise None."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    sha = next((l.split()[1] for l in lines if l.startswith("kernel_sources_sha256 ")), None)
    if sha != _kernel_sources_sha256():
        return None
    for l in lines:
        f = l.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == workload and f[2] == f"splits={splits}":
            r, wr = int(f[3].split("=")[1]), int(f[4].split("=")[1])
            return {"read": r, "write": wr, "total": r + wr}
    return None


def main():
    args = _parse()
    if args.calibrate_copy:
        _copy_calibration(args.calibrate_copy)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this implementation runs on one GPU only; the decode path shards "
                                   "by token/sequence or by head with no exchange, and no multi-GPU "
                                   "figure is produced", "n_gpus": args.gpus}))
        sys.exit(2)
    res, w = _gpu_run(args)
    # roofline: algorithmic bytes of one launch over the kernel's own duration
    # (HIP events recorded at kernel start and end by hipExtLaunchKernel)
    achieved = res["gathered"] / (res["kernel_ms"] * 1e-3) / 1e9
    # scores (576) and values (512) per valid slot and head, 2 flops per multiply-add
    mfma_flops = 2.0 * res["H"] * (576 + 512) * res["valid"]
    traffic = None if (args.splits or args.warm) else _traffic(args.workload, res["splits"])
    line = {
        "metric": METRIC,
        "value": round(res["gathered"] / (res["step_ms"] * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["step_ms"], 5),
        "us_per_step": round(1e3 * res["step_ms"], 3),
        "us_per_step_median": round(1e3 * res["step_ms_median"], 3),
        "us_per_step_p10_p90": [round(1e3 * res["step_ms_p10"], 3), round(1e3 * res["step_ms_p90"], 3)],
        "decode_kernel_us": round(1e3 * res["kernel_ms"], 3),
        "decode_kernel_us_median": round(1e3 * res["kernel_ms_median"], 3),
        "decode_us": round(1e3 * res["decode_ms"], 3),
        "decode_us_median": round(1e3 * res["decode_ms_median"], 3),
        "decode_us_p10_p90": [round(1e3 * res["decode_ms_p10"], 3), round(1e3 * res["decode_ms_p90"], 3)],
        "append_us": round(1e3 * res["append_ms"], 3),
        "append_kernel_us": round(1e3 * res["append_kernel_ms"], 3),
        "append_kernel_gbs": round(res["append_bytes"] / (res["append_kernel_ms"] * 1e-3) / 1e9, 2),
        "mfma_tflops": round(mfma_flops / (res["kernel_ms"] * 1e-3) / 1e12, 2),
        "mfma_frac_of_fp16_peak": round(mfma_flops / (res["kernel_ms"] * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "cache_state": "warm" if args.warm else (
            "cold (1 GiB sweep between steps, inputs included)" if args.cold_inputs else
            "cold rows (1 GiB sweep between steps; q, index lists, block table and new rows re-read after it)"),
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS.get(args.workload, '')}",
                   "tokens": res["T"], "heads": res["H"], "topk": res["K"], "pool_rows": res["rows"],
                   "valid_slots": res["valid"], "gathered_bytes": res["gathered"],
                   "splits": res["splits"], "cache": "nvfp4-352"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "copy_peak_measured": res["copy_gbs"],
                     "frac_of_copy_peak": round(achieved / res["copy_gbs"], 4),
                     "traffic": traffic["total"] if traffic else None,
                     "traffic_read_write": [traffic["read"], traffic["write"]] if traffic else None,
                     "kernel": "sparse_decode_kernel", "bytes_per_launch": res["gathered"],
                     "kernel_us": round(1e3 * res["kernel_ms"], 3)},
    }
    if "comparators" in res:
        line["comparators"] = {k: round(v, 3) for k, v in res["comparators"].items()}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
