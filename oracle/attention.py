"""Oracle sparse MLA decode attention in FP64.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the
product path may import this module.

What the pages fix (Prime Inference write-up, section "A native NVFP4
sparse-MLA decode kernel"; wireai.ir article, 4-bit-caches section): each
query token attends only to the cache positions its sparse indexer
selected, the selected compressed rows are unpacked on chip, and attention
runs on FP16 operands with FP32 accumulation.  The 2048-position selection
list has its empty slots padded (wireai.ir, 4-bit-caches section, third
decision).

Readings taken where the pages are silent:

* A1  Absorbed-MLA decode: the key of a row is its 576 values [latent(512);
      rope(64)] and its value is the latent alone, so scores contract over
      576 and the output has 512 values per head.
* A2  A slot whose index is negative is masked (the pad).  Index 0 is an
      ordinary row, so a zero pad without a length could not be told apart
      from it; the padded list therefore uses -1.
* A3  Every slot counts on its own: a row listed twice contributes twice.
* A4  With a block table, logical position p of sequence b lives at
      physical row block_table[b, p // block_size] * block_size
      + p % block_size.
* A8  A slot that names no cache row is masked like a pad: without a
      block table, an index at or past the pool's last row; with one, a
      token whose sequence id is not a row of the table, a position whose
      block number is past the table's width, a block entry that is
      negative (unassigned), or a physical row at or past the pool's end.
* A5  lse is the natural-log log-sum-exp of the *scaled* scores.
* A6  A token with no valid slot has output 0 and lse = -inf.
* A7  q arrives as fp16 or bf16 and is taken at its exact value; sm_scale is
      the float32 value the caller passes, taken exactly.

The definition computed for token t and head h, over valid slots j with
key k_j and value v_j:

    s_j   = sm_scale * (q[t,h] . k_j)
    m     = max_j s_j
    out   = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m)
    lse   = m + ln(sum_j exp(s_j - m))

This is written out directly per token: no tiling, no splitting, no
online rescaling.  numpy's FP64 matrix product is the only library step.
"""

from __future__ import annotations

import numpy as np

from .codec import LATENT_DIM, ROPE_DIM


def physical_rows(positions, seq, block_table, block_size, cache_rows):
    """Physical cache rows of one token's non-negative slot indices (A4, A8).

    positions:   the token's indices that are >= 0, in list order.
    seq:         the token's sequence id (a row of block_table), or None.
    block_table: [B, W] integer table or None (indices are physical rows).
    cache_rows:  number of rows in the pool.

    Returns an int64 array of the same length: the physical row of each
    slot, or -1 where the slot names no row (A8), so that the caller masks it.
    """
    p = np.asarray(positions, dtype=np.int64)
    rows = np.full(p.shape, -1, dtype=np.int64)
    if block_table is None:
        ok = p < cache_rows
        rows[ok] = p[ok]
        return rows
    bt = np.asarray(block_table, dtype=np.int64)
    if seq is None or not 0 <= int(seq) < bt.shape[0]:
        return rows
    block = p // block_size
    entry = np.full(p.shape, -1, dtype=np.int64)
    inside = block < bt.shape[1]
    entry[inside] = bt[int(seq), block[inside]]
    phys = entry * block_size + p % block_size
    ok = (entry >= 0) & (phys < cache_rows)
    rows[ok] = phys[ok]
    return rows


def sparse_mla_token(q_t, lat_rows, rope_rows, sm_scale):
    """Attention for one token over its already gathered valid rows.

    q_t: [H, 576] FP64; lat_rows: [v, 512]; rope_rows: [v, 64] (FP64, decoded).
    Returns (out [H, 512], lse [H]).
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    h = q_t.shape[0]
    v = lat_rows.shape[0]
    if v == 0:                                                     # A6
        return np.zeros((h, LATENT_DIM)), np.full(h, -np.inf)
    keys = np.concatenate([lat_rows, rope_rows], axis=1)           # A1: [v, 576]
    s = float(sm_scale) * (q_t @ keys.T)                           # [H, v]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ lat_rows) / l                                       # A1: values = latent
    lse = (m + np.log(l))[:, 0]                                    # A5
    return out, lse


def sparse_mla(q, lat, rope, indices, sm_scale, block_table=None,
               token_seq=None, block_size=64):
    """Sparse MLA decode over a decoded cache.

    q:        [T, H, 576] query values (fp16/bf16 inputs; taken exactly, A7)
    lat:      [R, 512] FP64 decoded latent of every cache row
    rope:     [R, 64]  FP64 decoded rope
    indices:  [T, K] int, negative = masked (A2)
    sm_scale: python float holding the caller's float32 value (A7)
    block_table / token_seq / block_size: optional logical -> physical map (A4);
    slots that name no row are masked (A8)

    Returns (out [T, H, 512] FP64, lse [T, H] FP64).
    """
    q = np.asarray(q, dtype=np.float64)
    idx = np.asarray(indices, dtype=np.int64)
    t_count, h = q.shape[0], q.shape[1]
    assert q.shape[2] == LATENT_DIM + ROPE_DIM
    out = np.zeros((t_count, h, LATENT_DIM))
    lse = np.zeros((t_count, h))
    for t in range(t_count):
        valid = idx[t][idx[t] >= 0]                                 # A2, A3
        seq = None if token_seq is None else int(token_seq[t])
        rows = physical_rows(valid, seq, block_table, block_size, lat.shape[0])
        rows = rows[rows >= 0]                                      # A8
        out[t], lse[t] = sparse_mla_token(q[t], lat[rows], rope[rows], sm_scale)
    return out, lse


def dense_mla(q, lat, rope, sm_scale):
    """Dense MLA decode of every token over every cache row (no selection).

    Same formula as ``sparse_mla`` with the selection replaced by all rows;
    the tests use it to check that an index list naming every row in any
    order gives the dense answer.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.concatenate([lat, rope], axis=1)                      # [R, 576]
    s = float(sm_scale) * np.einsum("thd,rd->thr", q, keys)
    m = s.max(axis=2, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=2, keepdims=True)
    out = np.einsum("thr,rd->thd", e, lat) / l
    return out, (m + np.log(l))[..., 0]
