"""Oracle for the paged cache pool: capacity arithmetic, the 64-row block
allocator's block tables, and the copy descriptors a request's blocks need
under the layer-major and block-major layouts.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the
product path may import this module.

What the pages fix (Prime Inference write-up, "Making room for low-latency
decode"): shrinking each MLA row from 576 to 352 bytes, with the indexer and
other per-token state unchanged, raised the cache capacity per decoder from
about 1.09 M to 1.63 M tokens at the same memory budget.  "Changing the
layout to reduce fragmentation" (and the mo.ai.kr article's KV-transfer
section): a block-major layout puts one block's data from every layer
together, so a request's cache moves in fewer, larger copies; it used
64-token blocks, against 1,024-token blocks for the layer-major layout.

Readings taken where the pages are silent:

* P1  Capacity: every cached token costs, in each of L layers, its cache row
      plus a fixed amount of other per-token state (the indexer's and the
      rest).  Capacity = floor(budget / (L * block_rows * (row + other)))
      whole blocks of block_rows tokens.
* P2  Allocation: a request grows by whole blocks; each new block is the
      lowest-numbered free block (so a request on an unfragmented pool gets
      consecutive blocks); a request that cannot get every block it asks
      for gets none; releasing a request frees all its blocks.
* P3  Layouts: layer-major holds layer l's rows of block b at
      (l * n_blocks + b) * B, block-major at (b * L + l) * B, with B =
      block_rows * row the bytes of one (layer, block) region.  A copy
      descriptor is one maximal run of contiguous bytes holding the
      request's regions, when the request's blocks are visited in table
      order.
"""

from __future__ import annotations

import numpy as np


def capacity_blocks(budget_bytes, layers, row_bytes, other_bytes, block_rows):
    """Whole blocks a budget holds (P1)."""
    per_block = layers * block_rows * (row_bytes + other_bytes)
    return budget_bytes // per_block


class Pool:
    """The block allocator (P2): block tables of up to max_seqs sequences."""

    def __init__(self, n_blocks, block_rows, max_seqs, max_blocks_per_seq):
        self.n_blocks = n_blocks
        self.block_rows = block_rows
        self.max_blocks = max_blocks_per_seq
        self.free = [True] * n_blocks
        self.tables = [[] for _ in range(max_seqs)]

    def reserve(self, seq, tokens):
        """Grow sequence `seq` to hold `tokens` positions; False if it cannot."""
        need = -(-tokens // self.block_rows) - len(self.tables[seq])
        if need <= 0:
            return True
        if len(self.tables[seq]) + need > self.max_blocks:
            return False
        picks = [b for b in range(self.n_blocks) if self.free[b]][:need]
        if len(picks) < need:
            return False
        for b in picks:
            self.free[b] = False
        self.tables[seq].extend(picks)
        return True

    def release(self, seq):
        for b in self.tables[seq]:
            self.free[b] = True
        self.tables[seq] = []

    def table(self, seq):
        return list(self.tables[seq]) + [-1] * (self.max_blocks - len(self.tables[seq]))

    def slot(self, seq, pos):
        """Physical row of position `pos` of sequence `seq`."""
        return self.tables[seq][pos // self.block_rows] * self.block_rows + pos % self.block_rows


def descriptors(blocks, layers, n_blocks, region_bytes, layout):
    """(copy descriptors, bytes) of a request whose blocks are `blocks`, in
    table order, under layout "layer" or "block" (P3)."""
    starts = []
    if layout == "layer":
        for l in range(layers):
            for b in blocks:
                starts.append((l * n_blocks + b) * region_bytes)
    elif layout == "block":
        for b in blocks:
            for l in range(layers):
                starts.append((b * layers + l) * region_bytes)
    else:
        raise ValueError(layout)
    runs = 0
    end = None
    for s in starts:
        if s != end:
            runs += 1
        end = s + region_bytes
    return runs, len(starts) * region_bytes


def _regions(pool_bytes, layout, n_blocks, layers, region):
    """View of a pool's bytes as [layer, block, region] (P3)."""
    a = np.asarray(pool_bytes, dtype=np.uint8)[:n_blocks * layers * region]
    if layout == "layer":
        return a.reshape(layers, n_blocks, region)
    return a.reshape(n_blocks, layers, region).transpose(1, 0, 2)


def pack(pool_bytes, layout, n_blocks, layers, region, block_ids):
    """Staging bytes [n][layers][region] of the request's blocks, in order."""
    v = _regions(pool_bytes, layout, n_blocks, layers, region)
    ids = np.asarray(block_ids, dtype=np.int64)
    out = np.zeros((ids.shape[0], layers, region), dtype=np.uint8)
    for i, b in enumerate(ids):
        if 0 <= b < n_blocks:
            out[i] = v[:, b, :]
    return out.reshape(-1)


def unpack(staging, block_ids, pool_bytes, layout, n_blocks, layers, region):
    """The pool after writing staging entry i to block block_ids[i] (in
    order: a later entry naming the same block wins)."""
    pool = np.array(pool_bytes, dtype=np.uint8, copy=True)
    v = _regions(pool, layout, n_blocks, layers, region)
    st = np.asarray(staging, dtype=np.uint8).reshape(-1, layers, region)
    for i, b in enumerate(np.asarray(block_ids, dtype=np.int64)):
        if 0 <= b < n_blocks:
            v[:, b, :] = st[i]
    return pool
