"""Pins for the pool oracle (CPU only): the pages' capacity figures, closed
forms and invariants of the allocator, and copy descriptors against a
byte-by-byte brute force."""

import numpy as np
import pytest

from oracle import pool


def test_capacity_reproduces_the_pages_figures():
    """576 -> 352-byte rows with other per-token state unchanged: about 1.09 M
    -> 1.63 M tokens at one budget.  With ~100 B of other state per token and
    layer (the value the two figures imply), a budget sized for 1.09 M tokens
    of 576-byte rows holds 1.63 M tokens of 352-byte rows, to the figures'
    rounding."""
    layers, other, bs = 80, 100, 64
    budget = 1_090_000 * layers * (576 + other)
    fp8 = pool.capacity_blocks(budget, layers, 576, other, bs) * bs
    nv = pool.capacity_blocks(budget, layers, 352, other, bs) * bs
    assert abs(fp8 - 1_090_000) < bs
    assert round(nv / 1e6, 2) == 1.63
    # the band of other-state sizes the rounded figures allow, 90..110 B: the
    # ratio stays within 1.625/1.095 .. 1.635/1.085
    for x in (90, 100, 110):
        r = (576 + x) / (352 + x)
        assert 1.625 / 1.095 <= r <= 1.635 / 1.085
    # and a 128-byte indexer key alone (no other state) would give +46.7%
    assert round((576 + 128) / (352 + 128), 3) == 1.467


def test_capacity_is_the_largest_whole_block_count():
    rng = np.random.default_rng(0)
    for _ in range(200):
        budget = int(rng.integers(0, 10**9))
        L, row, other, bs = int(rng.integers(1, 100)), int(rng.integers(1, 600)), int(rng.integers(0, 200)), int(
            rng.integers(1, 128))
        n = pool.capacity_blocks(budget, L, row, other, bs)
        per = L * bs * (row + other)
        assert n * per <= budget < (n + 1) * per


def test_allocator_lowest_free_first_and_all_or_nothing():
    p = pool.Pool(10, 64, 4, 6)
    assert p.reserve(0, 130)                      # 3 blocks
    assert p.reserve(1, 64)                       # 1 block
    assert p.tables[0] == [0, 1, 2] and p.tables[1] == [3]
    p.release(0)
    assert p.reserve(2, 200)                      # 4 blocks: 0, 1, 2, then 4
    assert p.tables[2] == [0, 1, 2, 4]
    assert not p.reserve(3, 64 * 6)               # 6 blocks wanted, 5 free: nothing taken
    assert p.tables[3] == [] and sum(p.free) == 5
    assert not p.reserve(1, 64 * 7)               # past the table's width
    assert p.reserve(1, 64 * 2) and p.tables[1] == [3, 5]
    assert p.reserve(1, 100) and p.tables[1] == [3, 5]       # already covered
    assert p.table(1) == [3, 5, -1, -1, -1, -1]
    assert p.slot(2, 64 * 3 + 5) == 4 * 64 + 5


def test_allocator_invariants_on_random_traffic():
    rng = np.random.default_rng(1)
    p = pool.Pool(300, 16, 20, 40)
    for _ in range(2000):
        s = int(rng.integers(20))
        if rng.random() < 0.3:
            p.release(s)
        else:
            p.reserve(s, int(rng.integers(0, 700)))
        owned = [b for t in p.tables for b in t]
        assert len(owned) == len(set(owned))                   # no block in two tables
        assert len(owned) + sum(p.free) == 300
        assert all(not p.free[b] for b in owned)
        assert all(len(t) <= 40 for t in p.tables)


def _brute_descriptors(blocks, layers, n_blocks, region, layout):
    addr = []
    for outer in range(layers if layout == "layer" else len(blocks)):
        for inner in range(len(blocks) if layout == "layer" else layers):
            l, b = (outer, blocks[inner]) if layout == "layer" else (inner, blocks[outer])
            base = (l * n_blocks + b) * region if layout == "layer" else (b * layers + l) * region
            addr.extend(range(base, base + region))
    runs = 1 + sum(1 for a, b in zip(addr, addr[1:]) if b != a + 1)
    return runs, len(addr)


@pytest.mark.parametrize("layout", ["layer", "block"])
def test_descriptors_against_brute_force(layout):
    rng = np.random.default_rng(2)
    for _ in range(30):
        n_blocks, layers, region = int(rng.integers(4, 20)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        k = int(rng.integers(1, n_blocks + 1))
        blocks = [int(b) for b in rng.permutation(n_blocks)[:k]]
        if rng.random() < 0.5:
            blocks.sort()
        assert pool.descriptors(blocks, layers, n_blocks, region, layout) == \
            _brute_descriptors(blocks, layers, n_blocks, region, layout)


def test_descriptor_closed_forms():
    L, n, R = 80, 5000, 64 * 352
    run = list(range(100, 3225))                                  # a 200K-token request, consecutive blocks
    assert pool.descriptors(run, L, n, R, "layer") == (L, L * len(run) * R)
    assert pool.descriptors(run, L, n, R, "block") == (1, L * len(run) * R)
    spread = list(range(0, 6250, 2))                              # every other block
    assert pool.descriptors(spread, L, 7000, R, "layer")[0] == L * len(spread)
    assert pool.descriptors(spread, L, 7000, R, "block")[0] == len(spread)


@pytest.mark.parametrize("layout", ["layer", "block"])
def test_pack_reads_the_regions_the_layout_places(layout):
    """Byte values that spell out (layer, block, offset) come back from pack
    in staging order [i][layer][offset]; unpack of a pack into other blocks
    moves exactly those regions."""
    n_blocks, layers, region = 7, 3, 8
    pool_b = np.zeros(n_blocks * layers * region, np.uint8)
    for l in range(layers):
        for b in range(n_blocks):
            start = (l * n_blocks + b) * region if layout == "layer" else (b * layers + l) * region
            pool_b[start:start + region] = 16 * l + b
    ids = [5, 0, 3]
    st = pool.pack(pool_b, layout, n_blocks, layers, region, ids).reshape(3, layers, region)
    for i, b in enumerate(ids):
        for l in range(layers):
            assert np.all(st[i, l] == 16 * l + b)
    moved = pool.unpack(st.reshape(-1), [1, 2, 6], np.zeros_like(pool_b), layout, n_blocks, layers, region)
    back = pool.pack(moved, layout, n_blocks, layers, region, [1, 2, 6])
    assert np.array_equal(back, st.reshape(-1))
    assert not pool.pack(moved, layout, n_blocks, layers, region, [0, 3, 4, 5]).any()
