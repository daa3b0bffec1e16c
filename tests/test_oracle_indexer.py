"""Pins for the oracle sparse indexer (CPU only).

Checked against: brute force in exact rational arithmetic (fractions) over
values decoded by torch's float8_e4m3fn (a library routine) with an
explicit sort by (-score, position); closed cases (fewer positions than k,
all scores equal, an empty context, ties planted at the cut); a block-table
relayout against contiguous keys; and planted mistakes that these pins
must catch.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import indexer


def _codes(rng, shape, spread=1.0):
    """Random finite E4M3 bytes of values ~ N(0, spread^2)."""
    v = torch.from_numpy((rng.standard_normal(shape) * spread).astype(np.float32))
    c = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return c


def _brute(q_code, key_codes, ctx, k):
    """Exact scores as Fractions, list by sorted((-score, p))."""
    qv = torch.from_numpy(q_code.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    kv = torch.from_numpy(key_codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = [sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv, kv[p])), Fraction(0))
         for p in range(ctx)]
    chosen = sorted(range(ctx), key=lambda p: (-s[p], p))[:k]
    return sorted(chosen)


def test_brute_force_small():
    rng = np.random.default_rng(1)
    keys = _codes(rng, (300, 128))
    q = _codes(rng, (4, 128))
    ctx = [300, 37, 16, 5]
    got = indexer.indexer_topk(q, keys, ctx, 16, base=np.zeros(4, np.int64))
    for t in range(4):
        want = _brute(q[t], keys, ctx[t], 16)
        assert got[t, :len(want)].tolist() == want
        assert np.all(got[t, len(want):] == -1)


def test_scores_are_exact_at_the_extremes():
    """FP64 holds the score exactly even for 128 products of +-448 and of the
    smallest subnormals (X2)."""
    q = np.full(128, 0x7E, np.uint8)                         # 448
    keys = np.stack([np.full(128, 0x7E, np.uint8),           # 448: 128 * 448^2
                     np.where(np.arange(128) % 2 == 0, 0x7E, 0xFE).astype(np.uint8),
                     np.full(128, 0x01, np.uint8)])           # 2^-9
    s = indexer.scores(q, keys)
    assert s[0] == 128 * 448.0 ** 2
    assert s[1] == 0.0
    assert s[2] == 128 * 448.0 * 2.0 ** -9
    qs = np.full(128, 0x01, np.uint8)
    assert indexer.scores(qs, keys[2:])[0] == 128 * 2.0 ** -18
    # random operands against exact rationals
    rng = np.random.default_rng(2)
    q = _codes(rng, (128,), 40.0)
    keys = _codes(rng, (50, 128), 40.0)
    qv = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    kv = torch.from_numpy(keys.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = indexer.scores(q, keys)
    for p in range(50):
        exact = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv, kv[p])), Fraction(0))
        assert Fraction(float(s[p])) == exact


def test_fewer_positions_than_k_and_empty_context():
    rng = np.random.default_rng(3)
    keys = _codes(rng, (100, 128))
    q = _codes(rng, (3, 128))
    got = indexer.indexer_topk(q, keys, [10, 0, 64], 64, base=np.array([90, 0, 5]))
    assert got[0, :10].tolist() == list(range(90, 100)) and np.all(got[0, 10:] == -1)
    assert np.all(got[1] == -1)
    assert got[2].tolist() == list(range(5, 69))


def test_equal_scores_go_to_the_smaller_position():
    keys = np.zeros((40, 128), np.uint8)
    q = np.full((1, 128), 0x38, np.uint8)                     # 1.0
    got = indexer.indexer_topk(q, keys, [40], 8, base=np.zeros(1, np.int64))
    assert got[0].tolist() == list(range(8))                   # all scores 0
    # two equal high scores straddling the cut: the smaller position wins
    keys[[7, 30, 33], 0] = 0x40                                # 2.0
    keys[[12, 25], 0] = 0x48                                   # 4.0
    got = indexer.indexer_topk(q, keys, [40], 4, base=np.zeros(1, np.int64))
    assert got[0].tolist() == [7, 12, 25, 30]


def _paged(bs, seed):
    rng = np.random.default_rng(seed)
    ctx = [3 * bs + 2, 5 * bs]
    seq_keys = [_codes(rng, (c, 128)) for c in ctx]
    n_blocks = 16
    pool = _codes(rng, (n_blocks * bs, 128))                   # unrelated rows
    bt = np.full((2, 6), -1, np.int64)
    free = list(rng.permutation(n_blocks))
    for b, c in enumerate(ctx):
        for j in range(-(-c // bs)):
            blk = free.pop()
            bt[b, j] = blk
            n = min(bs, c - j * bs)
            pool[blk * bs:blk * bs + n] = seq_keys[b][j * bs:j * bs + n]
    q = _codes(rng, (3, 128))
    token_seq = np.array([0, 1, 1])
    tctx = np.array([ctx[0], ctx[1], ctx[1] - 7])
    return pool, bt, seq_keys, q, token_seq, tctx


def _paged_matches(bs, seed):
    pool, bt, seq_keys, q, token_seq, tctx = _paged(bs, seed)
    got = indexer.indexer_topk(q, pool, tctx, 8, block_table=bt, token_seq=token_seq, block_size=bs)
    for t in range(3):
        want = indexer.indexer_topk(q[t:t + 1], seq_keys[token_seq[t]], tctx[t:t + 1], 8,
                                    base=np.zeros(1, np.int64))
        if not np.array_equal(got[t], want[0]):
            return False
    return True


@pytest.mark.parametrize("bs", [4, 64])
def test_block_table_relayout_against_contiguous_keys(bs):
    assert _paged_matches(bs, 10 + bs)


def test_pins_catch_planted_mistakes(monkeypatch):
    """A tie rule that favours the larger position, a list in score order, or
    a swapped block and offset each fail a pin above."""
    good_topk, good_rows = indexer.topk_positions, indexer.key_rows

    def larger_first(s, k):
        s = np.asarray(s)
        if s.shape[0] <= k:
            return np.arange(s.shape[0])
        order = np.lexsort((-np.arange(s.shape[0]), -s))
        return np.sort(order[:k])

    def score_order(s, k):
        return np.argsort(-np.asarray(s), kind="stable")[:k]

    keys = np.zeros((40, 128), np.uint8)
    keys[[7, 30, 33], 0] = 0x40
    keys[[12, 25], 0] = 0x48
    q = np.full((1, 128), 0x38, np.uint8)
    for bad in (larger_first, score_order):
        monkeypatch.setattr(indexer, "topk_positions", bad)
        got = indexer.indexer_topk(q, keys, [40], 4, base=np.zeros(1, np.int64))
        assert got[0].tolist() != [7, 12, 25, 30]
    monkeypatch.setattr(indexer, "topk_positions", good_topk)

    def swapped(positions, seq, base, block_table, block_size, n_rows):
        p = np.asarray(positions, dtype=np.int64)
        if block_table is not None:                      # the paged path only
            p = (p % block_size) * block_size + p // block_size
        return good_rows(p, seq, base, block_table, block_size, n_rows)

    monkeypatch.setattr(indexer, "key_rows", swapped)
    assert not _paged_matches(4, 14)
    monkeypatch.setattr(indexer, "key_rows", good_rows)
    assert _paged_matches(4, 14)


def test_positions_without_a_key_row_are_not_candidates():
    """X6: past the pool, unassigned blocks, blocks past the table and an
    unknown sequence contribute no candidate; the rest is the top-k of the
    positions that do name a row."""
    rng = np.random.default_rng(30)
    keys = _codes(rng, (64, 128))
    q = _codes(rng, (4, 128))
    # contiguous: positions 0..39 from base 40 -> rows 40..79, rows >= 64 do not exist
    got = indexer.indexer_topk(q[:1], keys, [40], 30, base=np.array([40]))
    want = indexer.indexer_topk(q[:1], keys[40:], [24], 30, base=np.zeros(1, np.int64))
    assert np.array_equal(got[0], np.where(want[0] >= 0, want[0] + 40, -1))
    # paged, block size 8: sequence 0 has blocks 2, -1, 5 (width 3)
    bt = np.array([[2, -1, 5]])
    got = indexer.indexer_topk(q[1:4], keys, [40, 20, 20], 12, block_table=bt,
                               token_seq=np.array([0, 0, 3]), block_size=8)
    pos = np.array(list(range(8)) + list(range(16, 24)))        # positions with a row
    rows = np.concatenate([np.arange(16, 24), np.arange(40, 48)])
    s = indexer.scores(q[1], keys[rows])
    want = np.sort(pos[np.lexsort((pos, -s))[:12]])
    assert got[0].tolist() == want.tolist()
    assert got[1, :12].tolist() == sorted(got[1, :12].tolist()) and got[1].max() < 20
    assert np.all(got[2] == -1)                                  # sequence 3 is not in the table
