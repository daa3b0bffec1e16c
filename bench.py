#!/usr/bin/env python3
"""Benchmark: NVFP4 sparse-MLA decode on one MI355X.

One step = the whole hot path for one decode step of a workload: the
quantize-append of the step's new rows plus one sparse decode launch over
every token's selected rows.  Inputs are synthetic and seeded (synth/),
resident in HBM before timing starts.

The headline workload (default ``batch128``, the largest decode batch: 128
tokens x 32 heads, top-2048 of 140K-146K rows through a 64-row block table
in a 1.63M-row pool) gives `value`, `roofline` and `cpu_baseline`.  Every
other workload (tiny, decode15, padded35, prefill4k) is timed in the same
run with the same protocol and reported under `configs`, next to the
headline's own entry.

Timing, per workload: W untimed warm-up steps, then K timed steps.  The
caches are cold for every step: a 1 GiB read sweep runs between steps
(outside the per-step events) so neither the 256 MB Infinity Cache nor L2
holds the gathered rows; the step's small inputs (q, index lists, block
table, new rows), which the kernels before attention have just written in
a real decode step, are read once after the sweep (--cold-inputs leaves
them cold).  Pass A brackets each step with HIP events on the stream the
kernels run on, with nothing inside a step (`us_per_step`, `value`).  Pass
A2 puts an event between the append and the decode (`append_us`,
`decode_us`).  Pass B repeats the launches with the library's kernel timing
on (hipExtLaunchKernel events at each kernel's own start and end), which
gives `decode_kernel_us`, `append_kernel_us`, the roofline figure and the
comparators' kernel times.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--configs a,b,...] [--warm] [--no-comparators]
                    [--no-cpu-baseline]
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
ALL_CONFIGS = ("tiny", "decode15", "padded35", "batch128", "prefill4k")
# the pages' comparison trio (native / FP8-576 / staged) is reported at these
TRIO_CONFIGS = ("decode15", "padded35", "batch128")
# the sparse indexer (the step before the decode) is timed at the decode batches;
# at the prefill chunk every token would rescan its whole sequence
INDEXER_CONFIGS = ("tiny", "decode15", "padded35", "batch128")
INDEXER_KEY_BYTES = 128
# two-level NVFP4 rows (per-tensor latent scale) are timed at these
TWO_LEVEL_CONFIGS = ("decode15", "batch128")

DESCRIPTIONS = {
    "tiny": "1 token x 16 heads, 256 picks of a 4,096-row NVFP4 pool",
    "decode15": "15 tokens (1 per sequence) x 32 heads, top-2048 of 146,000 rows each, 2.2M-row NVFP4 pool",
    "padded35": "35 tokens x 32 heads, contexts 256..8192 rows, 2048-slot lists padded with -1",
    "batch128": "128 tokens x 32 heads, top-2048 of 140K-146K rows via a 64-row block table, 1.63M-row pool",
    "prefill4k": "4096 tokens from 4 sequences x 32 heads, causal top-2048 (128 recent + 1920 older)",
}


def _parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch128", help="headline workload")
    ap.add_argument("--configs", default=",".join(ALL_CONFIGS),
                    help="comma-separated workloads timed besides the headline ('' = none)")
    ap.add_argument("--warm", action="store_true", help="no cache flush between steps")
    ap.add_argument("--cold-inputs", action="store_true",
                    help="leave q, index lists and block table cold too (default: only the gathered rows)")
    ap.add_argument("--splits", type=int, default=0, help="force the split count (0 = launch sizer)")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args(argv)


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
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]

    def mark(self, i, k):
        self.ev[i][k].record()

    def spans(self, a, b):
        return [e[a].elapsed_time(e[b]) for e in self.ev]


def _stats_us(ms):
    s = sorted(ms)
    return {"mean": round(1e3 * statistics.mean(ms), 3), "median": round(1e3 * statistics.median(ms), 3),
            "p10": round(1e3 * s[len(s) // 10], 3), "p90": round(1e3 * s[(9 * len(s)) // 10], 3)}


class Case:
    """One workload, prepared on the device: the encoded pool, the step's new
    rows, workspace and outputs."""

    def __init__(self, torch, mla, name, dev, q_dtype, splits, flush, cold_inputs):
        from synth import make_workload

        self.torch, self.mla, self.name = torch, mla, name
        w = make_workload(name, dev, q_dtype=q_dtype)
        self.w = w
        T, H, K = w.tokens, w.heads, w.topk
        self.cache = torch.empty((w.pool_rows, ROW_BYTES), dtype=torch.uint8, device=dev)
        mla.quantize_append(w.latent, w.rope, torch.arange(w.pool_rows, dtype=torch.int64, device=dev),
                            self.cache)
        keep = w.append_slots >= 0
        self.app_slots = w.append_slots.clone()
        app_idx = torch.where(keep, w.append_slots, torch.zeros_like(w.append_slots))
        # each token's own row with the same values: the step is repeatable
        self.app_lat = w.latent[app_idx].contiguous()
        self.app_rope = w.rope[app_idx].contiguous()
        self.splits = splits or mla.num_splits(T, H, K)
        self.ws = mla.make_workspace(T, H, K, dev, self.splits)
        self.out = torch.empty((T, H, 512), dtype=w.q.dtype, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.valid = w.valid_slots()
        self.gathered = self.valid * ROW_BYTES
        self.app_rows = int(keep.sum().item())
        self.app_bytes = (self.app_lat.numel() * self.app_lat.element_size()
                          + self.app_rope.numel() * self.app_rope.element_size()
                          + self.app_slots.numel() * 8 + self.app_rows * ROW_BYTES)
        inputs = [w.q, w.indices, self.app_lat, self.app_rope, self.app_slots]
        if w.block_table is not None:
            inputs += [w.block_table, w.token_seq]
        self._flush, self._inputs, self._cold = flush, inputs, cold_inputs

    def flush(self):
        """The cache sweep between steps (see the module docstring)."""
        if self._flush is not None:
            self._flush.sum()
            if not self._cold:
                for x in self._inputs:
                    x.sum()

    def append(self):
        self.mla.quantize_append(self.app_lat, self.app_rope, self.app_slots, self.cache)

    def decode(self, cache=None, indices=None, fmt="nvfp4", block=True):
        w = self.w
        self.mla.sparse_decode(w.q, self.cache if cache is None else cache,
                               w.indices if indices is None else indices, w.sm_scale, fmt=fmt,
                               block_table=w.block_table if block else None,
                               token_seq=w.token_seq if block else None, block_size=w.block_size,
                               workspace=self.ws, num_splits=self.splits, out=self.out, lse=self.lse)

    def step(self, tm=None, i=0, split=False):
        if tm:
            tm.mark(i, 0)
        self.append()
        if tm and split:
            tm.mark(i, 1)
        self.decode()
        if tm:
            tm.mark(i, 2)


def _kernel_ms(mla, fn, n, flush):
    """Durations (ms) of the last library kernel `fn` launches, each after a sweep."""
    out = []
    mla.kernel_timing(True)
    try:
        for _ in range(n):
            flush()
            fn()
            out.append(mla.last_kernel_ms())
    finally:
        mla.kernel_timing(False)
    return out


def _measure(torch, mla, c: Case, steps: int, warmup: int, comparators: bool):
    """Passes A, A2 and B (module docstring) plus the comparators for one workload."""
    for _ in range(warmup):
        c.flush()
        c.step()
    torch.cuda.synchronize()
    tm = Timer(torch, steps)
    for i in range(steps):
        c.flush()
        c.step(tm, i)
    torch.cuda.synchronize()
    tm2 = Timer(torch, max(10, steps // 2))
    for i in range(len(tm2.ev)):
        c.flush()
        c.step(tm2, i, split=True)
    torch.cuda.synchronize()
    n = max(10, steps // 2)

    def append_then_decode():
        # the decode follows its append on the GPU, as in pass A; only the
        # decode's own duration is read back
        c.append()
        c.decode()

    kern = _kernel_ms(mla, append_then_decode, n, c.flush)
    app_kern = _kernel_ms(mla, c.append, max(10, steps // 4), c.flush)
    step_ms, dec_ms, app_ms = tm.spans(0, 2), tm2.spans(1, 2), tm2.spans(0, 1)
    k_mean = statistics.mean(kern)
    w = c.w
    flops = 2.0 * w.heads * (576 + 512) * c.valid
    r = {
        "workload": DESCRIPTIONS[c.name], "tokens": w.tokens, "heads": w.heads, "topk": w.topk,
        "q_dtype": str(w.q.dtype).replace("torch.", ""), "pool_rows": w.pool_rows,
        "valid_slots": c.valid, "gathered_bytes": c.gathered, "splits": c.splits,
        "us_per_step": _stats_us(step_ms),
        "decode_us": _stats_us(dec_ms),
        "decode_kernel_us": _stats_us(kern),
        "gathered_gbs_per_step": round(c.gathered / (statistics.mean(step_ms) * 1e-3) / 1e9, 2),
        "gathered_gbs_kernel": round(c.gathered / (k_mean * 1e-3) / 1e9, 2),
        "frac_of_8tbs_kernel": round(c.gathered / (k_mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_tflops": round(flops / (k_mean * 1e-3) / 1e12, 2),
        "mfma_frac_of_fp16_peak": round(flops / (k_mean * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
        "append_rows": c.app_rows,
        "append_us": round(1e3 * statistics.mean(app_ms), 3),
        "append_kernel_us": round(1e3 * statistics.mean(app_kern), 3),
        "append_kernel_gbs": round(c.app_bytes / (statistics.mean(app_kern) * 1e-3) / 1e9, 2),
    }
    r["gather_ceiling"] = _gather_ceiling(torch, mla, c, n, k_mean)
    if comparators and c.name in TRIO_CONFIGS:
        r["trio"] = _comparators(torch, mla, c, n)
    if c.name in INDEXER_CONFIGS:
        r["indexer"] = _indexer(torch, mla, c, n)
    if c.name in TWO_LEVEL_CONFIGS:
        r["two_level"] = _two_level(torch, mla, c, n)
    return r, kern


def _physical_rows(torch, w):
    """The cache rows the decode reads (valid slots, in list order), int32."""
    idx = w.indices.long()
    keep = idx >= 0
    if w.block_table is not None:
        bs = w.block_size
        bt = w.block_table.long()[w.token_seq.long()]                 # [T, blocks]
        blk = torch.where(keep, idx // bs, torch.zeros_like(idx))
        rows = torch.gather(bt, 1, blk) * bs + idx % bs
    else:
        rows = idx
    return rows[keep].to(torch.int32).contiguous()


def _gather_ceiling(torch, mla, c: Case, n: int, decode_ms: float):
    """The same rows read by a kernel that does nothing else (cold, like the
    decode), and as many rows read contiguously: the HBM ceilings of the
    decode's gather on this machine."""
    rows = _physical_rows(torch, c.w)
    seq = torch.arange(rows.numel(), dtype=torch.int32, device=rows.device)
    sink = torch.zeros(1, dtype=torch.int32, device=rows.device)
    out = {}
    for name, rl in (("selected_rows", rows), ("contiguous_rows", seq)):
        ms = _kernel_ms(mla, lambda: mla.gather_probe(c.cache, rl, sink), n, c.flush)
        m = statistics.mean(ms)
        out[name] = {"kernel_us": round(1e3 * m, 3), "row_gbs": round(c.gathered / (m * 1e-3) / 1e9, 1),
                     "frac_of_8tbs": round(c.gathered / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    out["decode_vs_selected_rows"] = round(out["selected_rows"]["kernel_us"] / (1e3 * decode_ms), 4)
    return out


def _two_level(torch, mla, c: Case, n: int):
    """The same decode over two-level NVFP4 rows (global scale amax / 2688),
    and the two-level quantize-append of the step's new rows."""
    w = c.w
    g = float(w.latent.float().abs().max().item()) / 2688.0
    cache2 = torch.empty_like(c.cache)
    mla.quantize_append_2level(w.latent, w.rope, torch.arange(w.pool_rows, dtype=torch.int64, device=c.cache.device),
                               cache2, g)

    def dec():
        mla.sparse_decode(w.q, cache2, w.indices, w.sm_scale, kv_scale=g, block_table=w.block_table,
                          token_seq=w.token_seq, block_size=w.block_size, workspace=c.ws, num_splits=c.splits,
                          out=c.out, lse=c.lse)

    def app():
        mla.quantize_append_2level(c.app_lat, c.app_rope, c.app_slots, cache2, g)

    for _ in range(3):
        c.flush()
        dec()
    torch.cuda.synchronize()
    kd = _kernel_ms(mla, dec, n, c.flush)
    ka = _kernel_ms(mla, app, max(10, n // 2), c.flush)
    del cache2
    return {"global_scale": g, "decode_kernel_us": _stats_us(kd),
            "gathered_gbs_kernel": round(c.gathered / (statistics.mean(kd) * 1e-3) / 1e9, 2),
            "append_kernel_us": round(1e3 * statistics.mean(ka), 3)}


def _indexer(torch, mla, c: Case, n: int):
    """The sparse indexer over every token's visible positions (kernel time of
    its three kernels, from the first one's start to the last one's end)."""
    from synth import indexer_inputs

    w = c.w
    ix = indexer_inputs(w)
    out = torch.empty((w.tokens, w.topk), dtype=torch.int32, device=ix.keys.device)
    ws = mla.indexer_workspace(w.tokens, ix.max_ctx, ix.keys.device)
    kw = dict(key_base=ix.base, out=out, workspace=ws)
    if w.block_table is not None:
        kw = dict(block_table=w.block_table, token_seq=w.token_seq, block_size=w.block_size, out=out,
                  workspace=ws)

    def run():
        mla.indexer_topk(ix.q, ix.keys, ix.ctx, w.topk, ix.max_ctx, **kw)

    for _ in range(3):
        c.flush()
        run()
    torch.cuda.synchronize()
    ms = _kernel_ms(mla, run, n, c.flush)
    positions = int(ix.ctx.sum().item())
    key_bytes = positions * INDEXER_KEY_BYTES
    m = statistics.mean(ms)
    del ix, out, ws
    return {"kernel_us": _stats_us(ms), "positions_scored": positions, "key_bytes": key_bytes,
            "key_gbs": round(key_bytes / (m * 1e-3) / 1e9, 1),
            "frac_of_8tbs": round(key_bytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def _comparators(torch, mla, c: Case, n: int):
    """The pages' comparison at the same shapes: FP8-576 rows (same values,
    576-byte rows) and the staged path (gather-dequant the selected NVFP4
    rows into an FP8 buffer, then FP8 decode); kernel times in µs."""
    w = c.w
    T, K = w.tokens, w.topk
    dev = c.cache.device
    c8 = torch.empty((w.pool_rows, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    mla.fp8_quantize_append(w.latent, w.rope, torch.arange(w.pool_rows, device=dev), c8, 1.0)
    staged_rows = torch.empty((T * K, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    staged_idx = torch.empty((T, K), dtype=torch.int32, device=dev)

    def gather():
        mla.gather_dequant_fp8(c.cache, w.indices, 1.0, block_table=w.block_table, token_seq=w.token_seq,
                               block_size=w.block_size, rows=staged_rows, staged_indices=staged_idx)

    for _ in range(3):
        c.flush(); c.decode(cache=c8, fmt="fp8"); c.flush(); gather(); c.decode(staged_rows, staged_idx, "fp8", False)
    torch.cuda.synchronize()
    native = _kernel_ms(mla, c.decode, n, c.flush)
    fp8 = _kernel_ms(mla, lambda: c.decode(cache=c8, fmt="fp8"), n, c.flush)
    k_gather, k_sfp8 = [], []
    mla.kernel_timing(True)
    try:
        for _ in range(n):
            c.flush()
            gather()
            k_gather.append(mla.last_kernel_ms())
            c.decode(staged_rows, staged_idx, "fp8", False)
            k_sfp8.append(mla.last_kernel_ms())
    finally:
        mla.kernel_timing(False)
    del c8, staged_rows, staged_idx
    g, s8 = statistics.mean(k_gather), statistics.mean(k_sfp8)
    return {"native_nvfp4_kernel_us": round(1e3 * statistics.mean(native), 3),
            "fp8_576_kernel_us": round(1e3 * statistics.mean(fp8), 3),
            "staged_gather_dequant_kernel_us": round(1e3 * g, 3),
            "staged_fp8_decode_kernel_us": round(1e3 * s8, 3),
            "staged_total_kernel_us": round(1e3 * (g + s8), 3)}


def _cpu_baseline(w, seconds, tokens=None):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: per pass, decode the sampled tokens' selected rows from
    their 352-byte encodings and run the FP64 attention."""
    import numpy as np
    import torch

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
    tokens = list(range(w.tokens)) if tokens is None else list(tokens)
    # the encoded rows the sample touches (setup, not timed): the pool is already encoded
    per_tok = {}
    for t in tokens:
        v = idx[t][idx[t] >= 0]
        rows = attention.physical_rows(v, None if seq is None else int(seq[t]), bt, w.block_size,
                                       w.pool_rows)
        sel = torch.from_numpy(rows[rows >= 0]).to(w.latent.device)
        lat16 = w.latent.index_select(0, sel).cpu().numpy().astype(np.float64)
        rope16 = w.rope.index_select(0, sel).cpu().numpy().astype(np.float64)
        per_tok[t] = codec.nvfp4_encode_rows(lat16, rope16)

    def run(limit):
        done_bytes = 0
        n_tok = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 <= limit:
            for t in tokens:
                enc = per_tok[t]
                lat, rope = codec.nvfp4_decode_rows(enc)
                attention.sparse_mla_token(q[t], lat, rope, w.sm_scale)
                done_bytes += enc.shape[0] * ROW_BYTES
                n_tok += 1
                if time.perf_counter() - t0 > limit:
                    break
        return done_bytes, n_tok, time.perf_counter() - t0

    done_bytes, n_tok, el = run(seconds)
    out = {
        "value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": blas_threads,
        "kind": "oracle",
        "sample": f"{n_tok} token-passes over {len(tokens)} tokens of the {w.name} workload, "
                  f"NVFP4 row decode + FP64 attention, {el:.1f} s; host os.cpu_count()={os.cpu_count()}, "
                  f"affinity {len(os.sched_getaffinity(0))} cores",
        "us_per_step": round(1e6 * el * w.tokens / max(1, n_tok), 1),
    }
    # the same with the BLAS pool limited to one thread (half the time budget)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            b1, n1, e1 = run(seconds / 2)
        out["single_thread"] = {"value": round(b1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "us_per_step": round(1e6 * e1 * w.tokens / max(1, n1), 1),
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


def _gpu_run(args):
    import torch

    import nvfp4_compressed_sparse_mla_amd as mla

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = None if args.warm else torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    if flush is not None:
        flush.fill_(1.0)
    copy_gbs = _copy_peak(torch, dev)
    names = [n for n in (args.configs.split(",") if args.configs else []) if n]
    for n in names + [args.workload]:
        if n not in ALL_CONFIGS:
            raise SystemExit(f"unknown workload {n!r}; known: {ALL_CONFIGS}")
    order = [args.workload] + [n for n in names if n != args.workload]
    head = None
    configs = {}
    for name in order:
        dtypes = [torch.float16, torch.bfloat16] if name == "prefill4k" else [torch.float16]
        for qdt in dtypes:
            c = Case(torch, mla, name, dev, qdt, args.splits, flush, args.cold_inputs)
            r, kern = _measure(torch, mla, c, args.steps, args.warmup, not args.no_comparators)
            key = name if qdt == torch.float16 else f"{name}_bf16q"
            configs[key] = r
            print(f"[bench] {key}: kernel {r['decode_kernel_us']['mean']} us, "
                  f"step {r['us_per_step']['mean']} us", file=sys.stderr, flush=True)
            if name == args.workload and head is None:
                head = (c, r, kern)
                if not args.no_cpu_baseline:
                    r["cpu_baseline"] = _cpu_baseline(c.w, args.cpu_seconds)
            elif name == "prefill4k" and qdt == torch.float16 and not args.no_cpu_baseline:
                # the oracle once at the prefill chunk, on 12 of its tokens
                r["cpu_baseline"] = _cpu_baseline(c.w, min(6.0, args.cpu_seconds),
                                                  tokens=[b * 1024 + j for b in range(4) for j in (0, 511, 1023)])
            if head is None or c is not head[0]:
                del c
                torch.cuda.empty_cache()
    return head, configs, copy_gbs


def main(argv=None):
    args = _parse(argv)
    if args.calibrate_copy:
        _copy_calibration(args.calibrate_copy)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this implementation runs on one GPU only; the decode path shards "
                                   "by token/sequence or by head with no exchange, and no multi-GPU "
                                   "figure is produced", "n_gpus": args.gpus}))
        sys.exit(2)
    (c, r, kern), configs, copy_gbs = _gpu_run(args)
    k_ms = statistics.mean(kern)
    # roofline: algorithmic bytes of one launch over the kernel's own mean
    # duration (HIP events recorded at kernel start and end by hipExtLaunchKernel)
    achieved = c.gathered / (k_ms * 1e-3) / 1e9
    traffic = None if (args.splits or args.warm) else _traffic(args.workload, c.splits)
    step_s = r["us_per_step"]["mean"] * 1e-6
    line = {
        "metric": METRIC,
        "value": round(c.gathered / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "us_per_step": r["us_per_step"]["mean"],
        "decode_kernel_us": r["decode_kernel_us"]["mean"],
        "append_kernel_us": r["append_kernel_us"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "cache_state": "warm" if args.warm else (
            "cold (1 GiB sweep between steps, inputs included)" if args.cold_inputs else
            "cold rows (1 GiB sweep between steps; q, index lists, block table and new rows re-read after it)"),
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
                   "tokens": c.w.tokens, "heads": c.w.heads, "topk": c.w.topk, "pool_rows": c.w.pool_rows,
                   "valid_slots": c.valid, "gathered_bytes": c.gathered, "splits": c.splits,
                   "cache": "nvfp4-352"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "copy_peak_measured": copy_gbs,
                     "frac_of_copy_peak": round(achieved / copy_gbs, 4),
                     "gather_ceiling_measured": r["gather_ceiling"]["selected_rows"]["row_gbs"],
                     "frac_of_gather_ceiling": round(achieved / r["gather_ceiling"]["selected_rows"]["row_gbs"], 4),
                     "traffic": traffic["total"] if traffic else None,
                     "traffic_read_write": [traffic["read"], traffic["write"]] if traffic else None,
                     "kernel": "sparse_decode_kernel", "bytes_per_launch": c.gathered,
                     "kernel_us": round(1e3 * k_ms, 3)},
        "configs": configs,
    }
    if "cpu_baseline" in r:
        line["cpu_baseline"] = r["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
