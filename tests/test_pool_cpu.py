"""The library's host-side pool manager (C++) against the pool oracle:
capacity arithmetic, block tables under random traffic (bit for bit), slot
mappings, copy descriptors and error handling.  No GPU involved."""

import numpy as np
import pytest

import nvfp4_compressed_sparse_mla_amd as mla
from oracle import pool as opool


def test_capacity_matches_the_oracle_and_the_pages():
    rng = np.random.default_rng(0)
    for _ in range(300):
        args = (int(rng.integers(0, 10**12)), int(rng.integers(1, 128)), int(rng.integers(1, 600)),
                int(rng.integers(0, 300)), int(rng.integers(1, 256)))
        assert mla.pool_capacity_blocks(*args) == opool.capacity_blocks(*args)
    layers, other = 80, 100
    budget = 1_090_000 * layers * (576 + other)
    fp8 = mla.Pool(budget, layers, 576, other, max_seqs=1, max_blocks_per_seq=1).num_blocks * 64
    nv = mla.Pool(budget, layers, 352, other, max_seqs=1, max_blocks_per_seq=1).num_blocks * 64
    assert abs(fp8 - 1_090_000) < 64 and round(nv / 1e6, 2) == 1.63


def test_block_tables_match_the_oracle_under_random_traffic():
    rng = np.random.default_rng(1)
    n_seqs, width = 24, 50
    p = mla.Pool(400 * 16 * 10 * 352, 10, 352, 0, block_rows=16, max_seqs=n_seqs, max_blocks_per_seq=width)
    o = opool.Pool(p.num_blocks, 16, n_seqs, width)
    assert p.num_blocks == 400
    for step in range(1500):
        s = int(rng.integers(n_seqs))
        if rng.random() < 0.3:
            p.release(s)
            o.release(s)
        else:
            tok = int(rng.integers(0, 900))
            assert p.reserve(s, tok) == o.reserve(s, tok), step
        if step % 50 == 0:
            want = np.array([o.table(x) for x in range(n_seqs)])
            assert np.array_equal(p.block_table().numpy(), want)
            assert p.free_blocks == sum(o.free)
    for s in range(n_seqs):
        n = len(o.tables[s]) * 16
        if n:
            first = int(rng.integers(0, n))
            cnt = int(rng.integers(0, n - first + 1))
            assert p.slots(s, first, cnt).tolist() == [o.slot(s, first + i) for i in range(cnt)]
        for layout in ("layer", "block"):
            assert p.descriptors(s, layout) == opool.descriptors(o.tables[s], 10, 400, 16 * 352, layout)


def test_a_200k_token_request_on_a_fragmented_pool():
    """Descriptor counts of a 200,000-token request that lands on a pool
    fragmented by earlier requests: one run per layer per contiguous stretch
    of blocks under the layer-major layout, one per stretch under the
    block-major layout."""
    layers = 100
    p = mla.Pool(6000 * 64 * layers * 352, layers, 352, 0, max_seqs=40, max_blocks_per_seq=4000)
    rng = np.random.default_rng(2)
    for s in range(1, 40):                              # other requests, then some leave
        p.reserve(s, int(rng.integers(64, 64 * 120)))
    for s in range(1, 40, 3):
        p.release(s)
    assert p.reserve(0, 200_000)
    table = [b for b in p.block_table()[0].tolist() if b >= 0]
    assert len(table) == 3125
    runs = 1 + sum(1 for a, b in zip(table, table[1:]) if b != a + 1)
    d_layer, bytes_layer = p.descriptors(0, "layer")
    d_block, bytes_block = p.descriptors(0, "block")
    assert bytes_layer == bytes_block == 3125 * layers * 64 * 352
    assert d_block == runs and d_layer == layers * runs
    assert (d_layer, d_block) == (opool.descriptors(table, layers, p.num_blocks, 64 * 352, "layer")[0],
                                  opool.descriptors(table, layers, p.num_blocks, 64 * 352, "block")[0])


def test_pool_errors():
    p = mla.Pool(10 * 64 * 352, 1, 352, 0, max_seqs=2, max_blocks_per_seq=4)
    assert p.num_blocks == 10
    assert not p.reserve(0, 64 * 5)                     # wider than the table
    assert p.reserve(0, 64 * 4) and p.reserve(1, 64 * 4)
    assert p.free_blocks == 2
    p.release(0)
    assert p.free_blocks == 6
    with pytest.raises(mla.MlaError):
        p.reserve(2, 1)                                 # no such sequence
    with pytest.raises(mla.MlaError):
        p.slots(1, 250, 10)                             # past the reserved positions
    with pytest.raises(mla.MlaError):
        mla.Pool(-1, 1, 352, 0)
