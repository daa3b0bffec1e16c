"""Oracle sparse indexer: exact scores and the per-token top-k position list.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the
product path may import this module.

What the pages fix (Prime Inference write-up, section "A native NVFP4
sparse-MLA decode kernel"; wireai.ir article, 4-bit-caches section, third
decision): a sparse indexer selects, for each query token, the cache
positions its attention reads; the selection is a fixed-width list of up to
2048 positions whose unused slots are padded; the indexer keeps state of its
own per cached position next to the compressed row ("Making room for
low-latency decode": the indexer state is left unchanged when the rows
shrink).

The pages give no formula for the indexer's score, its state's format, or
the order of the list.  Readings taken:

* X1  Each cached position holds an indexer key of 128 values and each query
      token an indexer query of 128 values, both stored as FP8 E4M3 (the FP8
      type the pages use for stored state; codec reading R2).
* X2  The score of position p for token t is the dot product
      q_idx[t] . key[p], computed exactly.  Every E4M3 value is a multiple of
      2^-9 below 2^9 in magnitude, so every product is a multiple of 2^-18
      and the sum of 128 of them is below 2^25: FP64 holds every partial sum
      exactly, in any order.
* X3  Token t sees positions 0 .. ctx[t]-1 of its sequence (causal: the
      positions cached before it, plus its own where the caller counts it).
* X4  The list holds the min(k, n) positions with the largest scores, n the
      number of candidate positions (X3, X6);
      equal scores go to the smaller position.  It is written in ascending
      position order and padded with -1 to width k (any negative index is a
      masked pad for the attention, reading A2).
* X5  Positions are sequence positions.  Without a block table the list
      holds physical rows (base[t] + p: each sequence's keys are contiguous
      from base[t]), as the decode's index lists do for contiguous pools;
      with a block table it holds logical positions, and key p of sequence b
      lives at row block_table[b, p // bs] * bs + p % bs (reading A4).
* X6  A position that names no key row (a negative or past-the-pool row, a
      block past the table's width, an unassigned block entry, a sequence
      id outside the table) is not a candidate, as such a slot is masked in
      the attention (reading A8).
"""

from __future__ import annotations

import numpy as np

from .codec import e4m3_decode

KEY_DIM = 128


def key_rows(positions, seq, base, block_table, block_size, n_rows):
    """Physical key rows of a sequence's positions, -1 where none (X5, X6)."""
    p = np.asarray(positions, dtype=np.int64)
    rows = np.full(p.shape, -1, dtype=np.int64)
    if block_table is None:
        r = base + p
        ok = (r >= 0) & (r < n_rows)
        rows[ok] = r[ok]
        return rows
    bt = np.asarray(block_table, dtype=np.int64)
    if seq is None or not 0 <= int(seq) < bt.shape[0]:
        return rows
    blk = p // block_size
    entry = np.full(p.shape, -1, dtype=np.int64)
    inside = blk < bt.shape[1]
    entry[inside] = bt[int(seq), blk[inside]]
    r = entry * block_size + p % block_size
    ok = (entry >= 0) & (r < n_rows)
    rows[ok] = r[ok]
    return rows


def scores(q_code, key_codes):
    """Exact scores (X2): q_code [128] E4M3 bytes, key_codes [n, 128] E4M3 bytes."""
    q = e4m3_decode(np.asarray(q_code, dtype=np.uint8))
    k = e4m3_decode(np.asarray(key_codes, dtype=np.uint8))
    return k @ q                                    # FP64, exact for these operands


def topk_positions(s, k):
    """Positions of the min(k, n) largest scores, equal scores to the smaller
    position (X4), in ascending order."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    # a stable sort on -score keeps equal scores in position order
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:k])


def indexer_topk(q_codes, keys, ctx, k, base=None, block_table=None, token_seq=None,
                 block_size=64):
    """The indexer's lists for every token.

    q_codes:  [T, 128] uint8 E4M3 indexer queries
    keys:     [R, 128] uint8 E4M3 indexer keys of every cached row
    ctx:      [T] visible positions per token (X3)
    k:        list width (top-k)
    base:     [T] first key row of each token's sequence (no block table)
    block_table, token_seq, block_size: logical -> physical rows (X5)

    Returns [T, k] int64: physical rows (no block table) or logical
    positions (block table), ascending, padded with -1.
    """
    q_codes = np.asarray(q_codes, dtype=np.uint8)
    keys = np.asarray(keys, dtype=np.uint8)
    t_count = q_codes.shape[0]
    out = np.full((t_count, k), -1, dtype=np.int64)
    for t in range(t_count):
        n = int(ctx[t])
        if n <= 0:
            continue
        seq = None if token_seq is None else int(token_seq[t])
        b = 0 if base is None else int(base[t])
        rows = key_rows(np.arange(n), seq, b, block_table, block_size, keys.shape[0])
        cand = np.nonzero(rows >= 0)[0]                            # X6
        sel = cand[topk_positions(scores(q_codes[t], keys[rows[cand]]), k)]
        out[t, :sel.shape[0]] = sel if block_table is not None else sel + b
    return out
