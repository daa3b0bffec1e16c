"""Seeded synthetic workloads (inputs only; see the package docstring).

Value distributions (one recipe for every workload):

* latent row  = z * r, z ~ N(0,1)^512, r ~ LogNormal(0, 0.5) drawn once per
  row, cast to fp16;
* rope row    ~ N(0,1)^64, cast to fp16;
* q           ~ N(0,1)^(H x 576), fp16 (or bf16 where asked);
* index lists: distinct uniform picks without replacement, per token.

Pool values are drawn on the target device in 65,536-row chunks, chunk c
from a torch generator seeded with (seed, c), so a chunk can be drawn again
on its own.  Index lists and block tables are drawn on the host from numpy
PCG64 streams seeded with [seed, 10**6] and [seed, 2*10**6].

Named workloads (sizes as the decode path sees them):

* ``tiny``      1 token, 16 heads, 4,096-row pool, 256 distinct picks.
* ``decode15``  15 tokens (one per sequence), 32 heads, 15 sequences of
                146,000 rows each in a 2,200,000-row pool, 2,048 picks each.
* ``padded35``  35 tokens, 32 heads, contexts uniform in 256..8192 rows
                (one sequence has none), 2,048-slot lists padded with -1.
* ``batch128``  128 tokens, 32 heads, contexts 140,000..146,000 rows, a
                1,629,952-row pool of 64-row blocks reached through a block
                table, 2,048 picks each over logical positions.
* ``prefill4k`` 4,096 tokens from 4 sequences of 140,000 cached rows plus
                1,024 new rows each, 32 heads, causal lists made of the 128
                most recent positions plus 1,920 distinct older picks.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

LATENT_DIM = 512
ROPE_DIM = 64
QK_DIM = LATENT_DIM + ROPE_DIM
CHUNK_ROWS = 65536
# softmax scale 1/sqrt(576) as the float32 value handed to the kernel
SM_SCALE = float(np.float32(1.0 / 24.0))

WORKLOAD_NAMES = ("tiny", "decode15", "padded35", "batch128", "prefill4k")


@dataclass
class Workload:
    name: str
    pool_rows: int
    heads: int
    topk: int
    latent: torch.Tensor            # [R, 512] fp16 source values of every pool row
    rope: torch.Tensor              # [R, 64]  fp16
    q: torch.Tensor                 # [T, H, 576] fp16 or bf16
    indices: torch.Tensor           # [T, K] int32, -1 = masked
    sm_scale: float = SM_SCALE
    block_table: Optional[torch.Tensor] = None   # [B, max_blocks] int32 or None
    token_seq: Optional[torch.Tensor] = None     # [T] int32 or None
    block_size: int = 64
    # rows written by quantize-append inside one step: token t's own row
    append_slots: Optional[torch.Tensor] = None  # [N] int64 physical rows (-1 = skip)
    meta: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return int(self.q.shape[0])

    def valid_slots(self) -> int:
        return int((self.indices >= 0).sum().item())


def _torch_gen(device, seed: int, chunk: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(chunk)) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def pool_values(rows: int, seed: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Latent [rows, 512] and rope [rows, 64] fp16 source values of a pool."""
    device = torch.device(device)
    lat = torch.empty((rows, LATENT_DIM), dtype=torch.float16, device=device)
    rope = torch.empty((rows, ROPE_DIM), dtype=torch.float16, device=device)
    for c, r0 in enumerate(range(0, rows, CHUNK_ROWS)):
        n = min(CHUNK_ROWS, rows - r0)
        g = _torch_gen(device, seed, c)
        z = torch.randn((n, LATENT_DIM), generator=g, device=device, dtype=torch.float32)
        r = torch.exp(0.5 * torch.randn((n, 1), generator=g, device=device, dtype=torch.float32))
        lat[r0:r0 + n] = (z * r).to(torch.float16)
        rope[r0:r0 + n] = torch.randn((n, ROPE_DIM), generator=g, device=device,
                                      dtype=torch.float32).to(torch.float16)
    return lat, rope


def _queries(t: int, h: int, seed: int, device, dtype) -> torch.Tensor:
    g = _torch_gen(device, seed, 10**6)
    return torch.randn((t, h, QK_DIM), generator=g, device=device,
                       dtype=torch.float32).to(dtype)


def _distinct(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """k distinct uniform picks from range(n), in draw order."""
    return rng.choice(n, size=k, replace=False).astype(np.int64)


def _index_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng([seed, 10**6])


def make_custom(rows: int, tokens: int, heads: int, topk: int, seed: int, device,
                valid_per_token=None, pad_random: bool = False,
                q_dtype=torch.float16, name: str = "custom") -> Workload:
    """A small single-pool workload: every token picks from the whole pool.

    valid_per_token: optional list of valid counts per token (<= topk);
    remaining slots are -1, trailing unless pad_random.
    """
    lat, rope = pool_values(rows, seed, device)
    q = _queries(tokens, heads, seed, device, q_dtype)
    rng = _index_rng(seed)
    idx = np.full((tokens, topk), -1, dtype=np.int64)
    for t in range(tokens):
        v = topk if valid_per_token is None else int(valid_per_token[t])
        v = min(v, rows)
        picks = _distinct(rng, rows, v)
        if pad_random:
            pos = np.sort(rng.choice(topk, size=v, replace=False))
            idx[t, pos] = picks
        else:
            idx[t, :v] = picks
    append = torch.full((tokens,), -1, dtype=torch.int64, device=device)
    return Workload(name=name, pool_rows=rows, heads=heads, topk=topk, latent=lat,
                    rope=rope, q=q, indices=torch.from_numpy(idx.astype(np.int32)).to(device),
                    append_slots=append, meta={"seed": seed})


def _tiny(device, q_dtype):
    w = make_custom(4096, 1, 16, 256, seed=0, device=device, q_dtype=q_dtype, name="tiny")
    w.append_slots = torch.tensor([4095], dtype=torch.int64, device=device)
    return w


def _decode15(device, q_dtype):
    seed, seqs, ctx, pool = 1, 15, 146_000, 2_200_000
    lat, rope = pool_values(pool, seed, device)
    q = _queries(seqs, 32, seed, device, q_dtype)
    rng = _index_rng(seed)
    idx = np.stack([_distinct(rng, ctx, 2048) + b * ctx for b in range(seqs)])
    append = torch.tensor([b * ctx + ctx - 1 for b in range(seqs)], dtype=torch.int64,
                          device=device)
    return Workload("decode15", pool, 32, 2048, lat, rope, q,
                    torch.from_numpy(idx.astype(np.int32)).to(device),
                    append_slots=append, meta={"seed": seed, "ctx": ctx, "seqs": seqs})


def _padded35(device, q_dtype, pad_random=False):
    seed, seqs = 2, 35
    rng = _index_rng(seed)
    ctx = rng.integers(256, 8192, size=seqs, endpoint=True)
    ctx[rng.integers(seqs)] = 0
    base = np.concatenate([[0], np.cumsum(ctx)[:-1]])
    pool = int(ctx.sum())
    lat, rope = pool_values(pool, seed, device)
    q = _queries(seqs, 32, seed, device, q_dtype)
    idx = np.full((seqs, 2048), -1, dtype=np.int64)
    for b in range(seqs):
        k = int(min(ctx[b], 2048))
        picks = _distinct(rng, int(ctx[b]), k) + base[b]
        if pad_random:
            pos = np.sort(rng.choice(2048, size=k, replace=False))
            idx[b, pos] = picks
        else:
            idx[b, :k] = picks
    append = torch.tensor([int(base[b] + ctx[b] - 1) if ctx[b] > 0 else -1 for b in range(seqs)],
                          dtype=torch.int64, device=device)
    return Workload("padded35", pool, 32, 2048, lat, rope, q,
                    torch.from_numpy(idx.astype(np.int32)).to(device),
                    append_slots=append,
                    meta={"seed": seed, "ctx": ctx.tolist(), "pad_random": pad_random})


def _batch128(device, q_dtype):
    seed, seqs, bs = 3, 128, 64
    n_blocks = 25_468
    pool = n_blocks * bs                                         # 1,629,952 rows
    rng = _index_rng(seed)
    ctx = rng.integers(140_000, 146_000, size=seqs, endpoint=True)
    max_blocks = int(-(-146_000 // bs))                           # 2282
    bt = np.full((seqs, max_blocks), -1, dtype=np.int64)
    brng = np.random.default_rng([seed, 2 * 10**6])
    for b in range(seqs):
        nb = int(-(-int(ctx[b]) // bs))
        bt[b, :nb] = _distinct(brng, n_blocks, nb)               # blocks alias across sequences
    lat, rope = pool_values(pool, seed, device)
    q = _queries(seqs, 32, seed, device, q_dtype)
    idx = np.stack([_distinct(rng, int(ctx[b]), 2048) for b in range(seqs)])
    last = ctx - 1
    append = torch.tensor([int(bt[b, last[b] // bs] * bs + last[b] % bs) for b in range(seqs)],
                          dtype=torch.int64, device=device)
    return Workload("batch128", pool, 32, 2048, lat, rope, q,
                    torch.from_numpy(idx.astype(np.int32)).to(device),
                    block_table=torch.from_numpy(bt.astype(np.int32)).to(device),
                    token_seq=torch.arange(seqs, dtype=torch.int32, device=device),
                    block_size=bs, append_slots=append,
                    meta={"seed": seed, "ctx": ctx.tolist(), "n_blocks": n_blocks})


def _prefill4k(device, q_dtype):
    seed, seqs, cached, new, window = 4, 4, 140_000, 1024, 128
    span = cached + new                                          # rows per sequence
    pool = seqs * span                                           # 564,096 rows
    lat, rope = pool_values(pool, seed, device)
    t_count = seqs * new
    q = _queries(t_count, 32, seed, device, q_dtype)
    rng = _index_rng(seed)
    idx = np.empty((t_count, 2048), dtype=np.int64)
    append = np.empty(t_count, dtype=np.int64)
    for b in range(seqs):
        for j in range(new):
            t = b * new + j
            p = cached + j
            recent = np.arange(p - window + 1, p + 1)
            older = _distinct(rng, p - window + 1, 2048 - window)
            idx[t] = np.concatenate([recent, older]) + b * span
            append[t] = b * span + p
    return Workload("prefill4k", pool, 32, 2048, lat, rope, q,
                    torch.from_numpy(idx.astype(np.int32)).to(device),
                    append_slots=torch.from_numpy(append).to(device),
                    meta={"seed": seed, "cached": cached, "new": new, "window": window})


@dataclass
class IndexerInputs:
    keys: torch.Tensor              # [R, 128] uint8 E4M3 bytes, one key per pool row
    q: torch.Tensor                 # [T, 128] uint8 E4M3 bytes
    ctx: torch.Tensor               # [T] int32 visible positions per token
    base: Optional[torch.Tensor]    # [T] int64 first row of each token's sequence (no block table)
    max_ctx: int


def fp8_values(shape, seed: int, chunk: int, device) -> torch.Tensor:
    """E4M3 bytes of N(0,1) draws (torch's cast to float8_e4m3fn)."""
    g = _torch_gen(device, seed, chunk)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)


def indexer_inputs(w: Workload) -> IndexerInputs:
    """Indexer keys of every pool row and one indexer query per token, N(0,1)
    values stored as E4M3, with each token's visible context: its whole
    sequence for the decode workloads, the positions up to and including its
    own for the prefill chunk."""
    dev = w.q.device
    seed = int(w.meta.get("seed", 0))
    keys = torch.empty((w.pool_rows, 128), dtype=torch.uint8, device=dev)
    for c, r0 in enumerate(range(0, w.pool_rows, CHUNK_ROWS)):
        n = min(CHUNK_ROWS, w.pool_rows - r0)
        keys[r0:r0 + n] = fp8_values((n, 128), seed, 3 * 10**6 + c, dev)
    q = fp8_values((w.tokens, 128), seed, 4 * 10**6, dev)
    T = w.tokens
    if w.name == "decode15":
        ctx = [w.meta["ctx"]] * T
        base = [b * w.meta["ctx"] for b in range(T)]
    elif w.name == "padded35":
        ctx = list(w.meta["ctx"])
        base = list(np.concatenate([[0], np.cumsum(ctx)[:-1]]))
    elif w.name == "batch128":
        ctx, base = list(w.meta["ctx"]), None
    elif w.name == "prefill4k":
        span = w.meta["cached"] + w.meta["new"]
        ctx = [w.meta["cached"] + j + 1 for b in range(4) for j in range(w.meta["new"])]
        base = [b * span for b in range(4) for j in range(w.meta["new"])]
    else:                                              # one sequence over the whole pool
        ctx, base = [w.pool_rows] * T, [0] * T
    return IndexerInputs(keys=keys, q=q, ctx=torch.tensor(ctx, dtype=torch.int32, device=dev),
                         base=None if base is None else torch.tensor([int(b) for b in base],
                                                                     dtype=torch.int64, device=dev),
                         max_ctx=int(max(ctx)) if ctx else 0)


def make_workload(name: str, device, q_dtype=torch.float16, pad_random: bool = False) -> Workload:
    if name == "tiny":
        return _tiny(device, q_dtype)
    if name == "decode15":
        return _decode15(device, q_dtype)
    if name == "padded35":
        return _padded35(device, q_dtype, pad_random=pad_random)
    if name == "batch128":
        return _batch128(device, q_dtype)
    if name == "prefill4k":
        return _prefill4k(device, q_dtype)
    raise ValueError(f"unknown workload {name!r}; known: {WORKLOAD_NAMES}")
