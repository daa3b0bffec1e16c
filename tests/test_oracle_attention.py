"""Pins for the oracle attention (CPU only).

The oracle is checked against: explicit-loop brute force with math.fsum on
tiny inputs; torch's scaled_dot_product_attention and logsumexp in FP64
(library routines) when the list names every row; closed forms (q = 0, a
single valid slot, a dominant row, a duplicated slot); invariants
(permutation, inserted pads, block-table relayout); and the empty-list case.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, codec

SM = float(np.float32(1.0 / 24.0))


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((n, 512)) * np.exp(0.5 * rng.standard_normal((n, 1)))
    rope = rng.standard_normal((n, 64))
    cache = codec.nvfp4_encode_rows(lat.astype(np.float16).astype(np.float64),
                                    rope.astype(np.float16).astype(np.float64))
    return codec.nvfp4_decode_rows(cache)


def _q(t, h, seed):
    return np.random.default_rng(seed + 100).standard_normal((t, h, 576)).astype(np.float16).astype(np.float64)


def _brute(q, lat, rope, idx, sm):
    """Attention by explicit loops and math.fsum (no numpy reductions)."""
    T, H = q.shape[0], q.shape[1]
    out = np.zeros((T, H, 512))
    lse = np.zeros((T, H))
    for t in range(T):
        sel = [int(i) for i in idx[t] if i >= 0]
        for h in range(H):
            if not sel:
                lse[t, h] = -math.inf
                continue
            s = []
            for r in sel:
                terms = [q[t, h, d] * lat[r, d] for d in range(512)]
                terms += [q[t, h, 512 + d] * rope[r, d] for d in range(64)]
                s.append(sm * math.fsum(terms))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = math.fsum(w)
            for d in range(512):
                out[t, h, d] = math.fsum(wi * lat[r, d] for wi, r in zip(w, sel)) / l
            lse[t, h] = m + math.log(l)
    return out, lse


def test_brute_force_tiny():
    lat, rope = _rows(4, 1)
    q = _q(2, 2, 1)
    idx = np.array([[0, 2, -1, 3], [1, -1, -1, -1]])
    out, lse = attention.sparse_mla(q, lat, rope, idx, SM)
    bo, bl = _brute(q, lat, rope, idx, SM)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def test_brute_force_tiny_larger_scores():
    lat, rope = _rows(4, 2)
    q = _q(1, 2, 2) * 8.0                                  # sharper softmax
    idx = np.array([[3, 1, 0, 2]])
    out, lse = attention.sparse_mla(q, lat, rope, idx, SM)
    bo, bl = _brute(q, lat, rope, idx, SM)
    np.testing.assert_allclose(out, bo, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(lse, bl, rtol=1e-12)


def test_all_positions_equal_dense_sdpa():
    n, T, H = 96, 3, 4
    lat, rope = _rows(n, 3)
    q = _q(T, H, 3)
    rng = np.random.default_rng(4)
    idx = np.stack([rng.permutation(n) for _ in range(T)])
    out, lse = attention.sparse_mla(q, lat, rope, idx, SM)
    qt = torch.from_numpy(q)                                       # [T, H, 576]
    k = torch.from_numpy(np.concatenate([lat, rope], 1))           # [n, 576]
    v = torch.from_numpy(lat)                                      # [n, 512]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[:, :, None, :], k[None, None].expand(T, H, n, 576),
        v[None, None].expand(T, H, n, 512), scale=SM)[:, :, 0, :]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    ref_lse = torch.logsumexp(SM * torch.einsum("thd,nd->thn", qt, k), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)
    d_out, d_lse = attention.dense_mla(q, lat, rope, SM)
    np.testing.assert_allclose(out, d_out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, d_lse, rtol=1e-12)


def test_zero_query_is_mean_of_valid_rows():
    lat, rope = _rows(50, 5)
    q = np.zeros((1, 3, 576))
    idx = np.array([[4, 9, -1, 17, 33, -1]])
    out, lse = attention.sparse_mla(q, lat, rope, idx, SM)
    np.testing.assert_allclose(out[0], np.broadcast_to(lat[[4, 9, 17, 33]].mean(0), (3, 512)), atol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(4), rtol=1e-14)


def test_single_slot_returns_its_row():
    lat, rope = _rows(20, 6)
    q = _q(1, 2, 6)
    idx = np.array([[-1, -1, 11, -1]])
    out, lse = attention.sparse_mla(q, lat, rope, idx, SM)
    np.testing.assert_array_equal(out[0], np.broadcast_to(lat[11], (2, 512)))
    k = np.concatenate([lat[11], rope[11]])
    np.testing.assert_allclose(lse[0], SM * (q[0] @ k), rtol=1e-13)


def test_dominant_row_takes_the_output():
    lat, rope = _rows(10, 7)
    q = np.zeros((1, 1, 576))
    q[0, 0, 512:] = rope[6] * 1e4                          # row 6 scores far above the rest
    idx = np.array([[1, 6, 2, 8]])
    out, _ = attention.sparse_mla(q, lat, rope, idx, SM)
    np.testing.assert_allclose(out[0, 0], lat[6], rtol=1e-12, atol=1e-12)


def test_duplicate_slot_equals_doubled_weight():
    """Listing a row twice is the same as adding ln 2 to its score."""
    lat, rope = _rows(12, 8)
    q = _q(1, 1, 8)
    out, lse = attention.sparse_mla(q, lat, rope, np.array([[2, 5, 5, 9]]), SM)
    keys = np.concatenate([lat[[2, 5, 9]], rope[[2, 5, 9]]], 1)
    s = SM * (q[0, 0] @ keys.T)
    s[1] += math.log(2)
    w = np.exp(s - s.max())
    np.testing.assert_allclose(out[0, 0], (w @ lat[[2, 5, 9]]) / w.sum(), rtol=1e-12)
    np.testing.assert_allclose(lse[0, 0], s.max() + math.log(w.sum()), rtol=1e-13)


def test_permutation_and_pad_insertion_invariance():
    lat, rope = _rows(64, 9)
    q = _q(1, 4, 9)
    rng = np.random.default_rng(10)
    base = rng.choice(64, 20, replace=False)
    o1, l1 = attention.sparse_mla(q, lat, rope, base[None], SM)
    perm = rng.permutation(base)
    padded = np.full(40, -1)
    padded[np.sort(rng.choice(40, 20, replace=False))] = perm
    o2, l2 = attention.sparse_mla(q, lat, rope, padded[None], SM)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_empty_list_gives_zero_and_minus_inf():
    lat, rope = _rows(8, 11)
    q = _q(2, 2, 11)
    out, lse = attention.sparse_mla(q, lat, rope, np.array([[-1, -1, -1], [0, -1, 3]]), SM)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def _paged_case(bs, seed):
    """Sequences held as contiguous decoded arrays, and the same rows copied
    block by block into a shared pool through a block table.

    Returns (pool_lat, pool_rope, bt, seqs, q, idx, token_seq, expected) where
    expected[t] lists token t's logical positions that exist in its sequence.
    Index lists mix positions inside the sequence, positions in unassigned
    blocks (entry -1), positions past the table's width and, for one token, a
    sequence id outside the table: all of those name no row (A8).
    """
    rng = np.random.default_rng(seed)
    ctx = [3 * bs + 1, 5 * bs, 2 * bs + bs // 2]
    width = 7                                        # table columns
    n_blocks = 24
    seqs = [_rows(c, seed + 10 * b) for b, c in enumerate(ctx)]
    # the pool starts out holding unrelated rows: a wrong address reads them
    pool_lat, pool_rope = _rows(n_blocks * bs, seed + 99)
    pool_lat, pool_rope = pool_lat.copy(), pool_rope.copy()
    bt = np.full((len(ctx), width), -1, dtype=np.int64)
    free = list(rng.permutation(n_blocks))
    for b, c in enumerate(ctx):
        nb = -(-c // bs)
        for k in range(nb):
            blk = free.pop()
            bt[b, k] = blk
            n = min(bs, c - k * bs)
            pool_lat[blk * bs:blk * bs + n] = seqs[b][0][k * bs:k * bs + n]
            pool_rope[blk * bs:blk * bs + n] = seqs[b][1][k * bs:k * bs + n]
    token_seq = np.array([0, 1, 2, 1, 5])            # token 4: no such sequence
    T, K = len(token_seq), 24
    q = _q(T, 2, seed)
    idx = np.full((T, K), -1, dtype=np.int64)
    expected = []
    for t, b in enumerate(token_seq):
        c = ctx[b] if b < len(ctx) else 0
        inside = list(rng.choice(c, min(c, 12), replace=False)) if c else []
        nb = -(-c // bs) if c else 0
        unassigned = [nb * bs + int(x) for x in rng.integers(0, (width - nb) * bs, 3)] if c else [1, 2]
        past_width = [width * bs + int(x) for x in rng.integers(0, 50, 2)]
        lst = inside + unassigned + past_width
        pos = np.sort(rng.choice(K, len(lst), replace=False))
        idx[t, pos] = rng.permutation(np.array(lst, dtype=np.int64))
        expected.append([int(p) for p in idx[t] if 0 <= p < c and b < len(ctx)])
    return pool_lat, pool_rope, bt, seqs, q, idx, token_seq, expected


def _paged_matches_contiguous(bs, seed):
    """Attention through the block table equals attention over each
    sequence's contiguous rows addressed directly by logical position."""
    pool_lat, pool_rope, bt, seqs, q, idx, token_seq, expected = _paged_case(bs, seed)
    out, lse = attention.sparse_mla(q, pool_lat, pool_rope, idx, SM, block_table=bt,
                                    token_seq=token_seq, block_size=bs)
    for t, b in enumerate(token_seq):
        if b >= len(seqs) or not expected[t]:
            if not (np.all(out[t] == 0.0) and np.all(np.isneginf(lse[t]))):
                return False
            continue
        lat, rope = seqs[b]
        o2, l2 = attention.sparse_mla_token(q[t], lat[expected[t]], rope[expected[t]], SM)
        if not (np.array_equal(out[t], o2) and np.array_equal(lse[t], l2)):
            return False
    return True


@pytest.mark.parametrize("bs", [4, 5, 64])
def test_block_table_relayout_against_contiguous_sequences(bs):
    assert _paged_matches_contiguous(bs, 40 + bs)


def test_relayout_pin_catches_a_swapped_block_and_offset(monkeypatch):
    """The pin above fails when the mapping swaps p // bs and p % bs, or
    wraps an unassigned entry instead of masking it (mistakes planted in the
    oracle)."""
    good = attention.physical_rows

    def swapped(positions, seq, block_table, block_size, cache_rows):
        p = np.asarray(positions, dtype=np.int64)
        q = (p % block_size) * block_size + p // block_size
        return good(q, seq, block_table, block_size, cache_rows)

    def wraps(positions, seq, block_table, block_size, cache_rows):
        p = np.asarray(positions, dtype=np.int64)
        bt = np.asarray(block_table)
        blk = np.minimum(p // block_size, bt.shape[1] - 1)
        r = bt[min(int(seq), bt.shape[0] - 1), blk] * block_size + p % block_size
        return np.where(r < 0, r % cache_rows, r)

    for bad in (swapped, wraps):
        monkeypatch.setattr(attention, "physical_rows", bad)
        assert not _paged_matches_contiguous(5, 45)
    monkeypatch.setattr(attention, "physical_rows", good)
    assert _paged_matches_contiguous(5, 45)


def test_index_past_the_pool_is_masked():
    """Without a block table an index at or past the last row names no row
    (A8): the result equals the list without it."""
    lat, rope = _rows(16, 13)
    q = _q(1, 3, 13)
    o1, l1 = attention.sparse_mla(q, lat, rope, np.array([[3, 16, 7, 1000]]), SM)
    o2, l2 = attention.sparse_mla_token(q[0], lat[[3, 7]], rope[[3, 7]], SM)
    np.testing.assert_array_equal(o1[0], o2)
    np.testing.assert_array_equal(l1[0], l2)


def test_staged_path_equals_native_on_fp8_exact_rows():
    """When every decoded value is an E4M3 value, staging changes nothing."""
    rng = np.random.default_rng(14)
    n = 32
    # codes with |c| in {0, .5, 1, 1.5, 2, 3, 4, 6} and power-of-two scales: products need
    # at most 2 significant bits, so E4M3 holds them exactly
    codes = rng.integers(0, 16, size=(n, 512))
    codes[:, ::16] = 7
    lat = codec.e2m1_decode(codes).reshape(n, 32, 16) * (2.0 ** rng.integers(-3, 3, (n, 32, 1)))
    lat = lat.reshape(n, 512)
    rope = codec.e4m3_decode(rng.integers(0, 0x7E, (n, 64)))
    cache = codec.nvfp4_encode_rows(lat, rope)
    q = _q(2, 3, 14)
    idx = np.array([[0, 5, -1, 9, 31], [2, -1, -1, 3, 4]])
    l_n, r_n = codec.nvfp4_decode_rows(cache)
    o1, s1 = attention.sparse_mla(q, l_n, r_n, idx, SM)
    rows, sidx = codec.staged_fp8_rows(cache, idx)
    l_s, r_s = codec.fp8_decode_rows(rows)
    o2, s2 = attention.sparse_mla(q, l_s, r_s, sidx, SM)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
