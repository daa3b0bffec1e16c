"""GPU sparse indexer vs the oracle: the position lists must be identical
(integer work, bit-exact), at small sizes with ties, pads, empty contexts and
block tables, and at the decode workloads' full sizes; the lists then drive
the decode, whose output is checked against the oracle's attention."""

import numpy as np
import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla
from oracle import indexer as oidx
from synth import fp8_values, indexer_inputs, make_custom, make_workload
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle(q, keys, ctx, topk, base=None, bt=None, seq=None, bs=64, tokens=None):
    qn = q.cpu().numpy()
    kn = keys.cpu().numpy()
    cn = ctx.cpu().numpy()
    bn = None if base is None else base.cpu().numpy()
    btn = None if bt is None else bt.cpu().numpy()
    sn = None if seq is None else seq.cpu().numpy()
    tokens = range(qn.shape[0]) if tokens is None else tokens
    rows = []
    for t in tokens:
        rows.append(oidx.indexer_topk(qn[t:t + 1], kn, cn[t:t + 1], topk,
                                      base=None if bn is None else bn[t:t + 1],
                                      block_table=btn, token_seq=None if sn is None else sn[t:t + 1],
                                      block_size=bs)[0])
    return np.stack(rows)


def test_small_contiguous_every_context_size():
    keys = fp8_values((6000, 128), 1, 0, DEV)
    q = fp8_values((7, 128), 1, 1, DEV)
    ctx = torch.tensor([0, 1, 100, 2047, 2048, 2049, 5000], dtype=torch.int32, device=DEV)
    base = torch.tensor([0, 5, 17, 900, 1000, 3000, 1000], dtype=torch.int64, device=DEV)
    out = mla.indexer_topk(q, keys, ctx, 2048, 5000, key_base=base)
    torch.cuda.synchronize()
    want = _oracle(q, keys, ctx, 2048, base=base)
    assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("topk", [1, 7, 100, 1000])
def test_small_topk_widths(topk):
    keys = fp8_values((3000, 128), topk, 0, DEV)
    q = fp8_values((3, 128), topk, 1, DEV)
    ctx = torch.tensor([3000, 1500, topk], dtype=torch.int32, device=DEV)
    base = torch.zeros(3, dtype=torch.int64, device=DEV)
    out = mla.indexer_topk(q, keys, ctx, topk, 3000, key_base=base)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), _oracle(q, keys, ctx, topk, base=base))


def test_ties_down_to_the_last_bit():
    """Keys repeat a few rows, so whole runs of positions share one exact
    score and the selection is decided by position alone (the radix select
    refines through all 64 key bits); all-zero keys tie everywhere."""
    rng = np.random.default_rng(3)
    distinct = fp8_values((5, 128), 3, 0, DEV)
    pick = torch.from_numpy(rng.integers(0, 5, 4000)).to(DEV)
    keys = distinct[pick].contiguous()
    keys[3000:] = 0
    q = fp8_values((4, 128), 3, 1, DEV)
    ctx = torch.tensor([3000, 3000, 4000, 1000], dtype=torch.int32, device=DEV)
    base = torch.tensor([0, 0, 0, 3000], dtype=torch.int64, device=DEV)
    for topk in (1, 333, 2048):
        out = mla.indexer_topk(q, keys, ctx, topk, 4000, key_base=base)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), _oracle(q, keys, ctx, topk, base=base)), topk


@pytest.mark.parametrize("bs", [64, 48])
def test_block_table_with_missing_rows(bs):
    keys = fp8_values((bs * 50, 128), bs, 0, DEV)
    q = fp8_values((5, 128), bs, 1, DEV)
    rng = np.random.default_rng(bs)
    bt = np.stack([rng.permutation(50)[:40] for _ in range(3)]).astype(np.int32)
    bt[1, 10:20] = -1                                   # unassigned blocks
    seq = torch.tensor([0, 1, 2, 1, 9], dtype=torch.int32, device=DEV)   # sequence 9: not in the table
    ctx = torch.tensor([40 * bs, 40 * bs, 41 * bs, 7, 100], dtype=torch.int32, device=DEV)  # 41 blocks: past the width
    btt = torch.from_numpy(bt).to(DEV)
    out = mla.indexer_topk(q, keys, ctx, 512, 41 * bs, block_table=btt, token_seq=seq, block_size=bs)
    torch.cuda.synchronize()
    want = _oracle(q, keys, ctx, 512, bt=btt, seq=seq, bs=bs)
    assert np.array_equal(out.cpu().numpy(), want)
    assert np.all(want[4] == -1)


def test_workspace_reuse_and_determinism():
    keys = fp8_values((5000, 128), 9, 0, DEV)
    q = fp8_values((6, 128), 9, 1, DEV)
    ctx = torch.full((6,), 5000, dtype=torch.int32, device=DEV)
    base = torch.zeros(6, dtype=torch.int64, device=DEV)
    ws = mla.indexer_workspace(6, 5000, DEV)
    first = mla.indexer_topk(q, keys, ctx, 2048, 5000, key_base=base, workspace=ws).clone()
    for _ in range(3):
        again = mla.indexer_topk(q, keys, ctx, 2048, 5000, key_base=base, workspace=ws)
        assert torch.equal(first, again)
    hist_bytes = 6 * 4096 * 4
    torch.cuda.synchronize()
    assert torch.all(ws[:hist_bytes] == 0)              # the histograms are left at zero
    assert torch.all(ws[hist_bytes:hist_bytes + 6 * 4] == 0)   # and so are the candidate counts


def test_long_contexts_of_equal_scores():
    """100K positions whose keys are all one row: every score ties, so the
    list is the first topk positions; several bitmap words per thread of the
    ordered emit, tie ranks running across threads.  A second token mixes
    two distinct keys, so its threshold falls inside a run of ties."""
    one = fp8_values((2, 128), 11, 0, DEV)
    n = 100_000
    keys = one[torch.zeros(n, dtype=torch.long, device=DEV)].contiguous()
    keys[::3] = one[1]
    q = fp8_values((3, 128), 11, 1, DEV)
    ctx = torch.tensor([n, n, 70_001], dtype=torch.int32, device=DEV)
    base = torch.zeros(3, dtype=torch.int64, device=DEV)
    same = keys.clone()
    same[:] = one[0]
    for kk in (same, keys):
        for topk in (2048, 777):
            out = mla.indexer_topk(q, kk, ctx, topk, n, key_base=base)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), _oracle(q, kk, ctx, topk, base=base)), topk


def test_contexts_past_the_emit_registers():
    """Contexts longer than 8 x 32 x 1024 positions take the ordered emit's
    chunked path (more than 8 bitmap words per thread).  With random keys
    ~8% of 300K positions share the threshold bucket, more than the finish
    kernel's LDS candidate cache holds; a long run of one key puts the
    threshold inside ties spread over many words."""
    n = 300_000
    keys = fp8_values((n, 128), 12, 0, DEV)
    q = fp8_values((3, 128), 12, 1, DEV)
    runs = keys.clone()
    runs[100_000:280_000] = keys[5]
    ctx = torch.tensor([n, 270_001, n - 31], dtype=torch.int32, device=DEV)
    base = torch.zeros(3, dtype=torch.int64, device=DEV)
    for kk in (keys, runs):
        for topk in (2048, 513):
            out = mla.indexer_topk(q, kk, ctx, topk, n, key_base=base)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), _oracle(q, kk, ctx, topk, base=base)), topk


def test_decode15_full_size_every_token():
    w = make_workload("decode15", DEV)
    ix = indexer_inputs(w)
    out = mla.indexer_topk(ix.q, ix.keys, ix.ctx, 2048, ix.max_ctx, key_base=ix.base)
    torch.cuda.synchronize()
    want = _oracle(ix.q, ix.keys, ix.ctx, 2048, base=ix.base)
    assert np.array_equal(out.cpu().numpy(), want)


def test_batch128_full_size_sampled_tokens():
    w = make_workload("batch128", DEV)
    ix = indexer_inputs(w)
    out = mla.indexer_topk(ix.q, ix.keys, ix.ctx, 2048, ix.max_ctx, block_table=w.block_table,
                           token_seq=w.token_seq, block_size=w.block_size)
    torch.cuda.synchronize()
    toks = [8 * k + x for x in range(8) for k in (0, 9)]
    want = _oracle(ix.q, ix.keys, ix.ctx, 2048, bt=w.block_table, seq=w.token_seq, bs=w.block_size,
                   tokens=toks)
    assert np.array_equal(out.cpu().numpy()[toks], want)


def test_indexer_lists_drive_the_decode():
    """padded35: the indexer's lists (many shorter than 2048, one empty)
    feed the decode, which matches the oracle's attention over the oracle's
    own lists."""
    w = make_workload("padded35", DEV)
    ix = indexer_inputs(w)
    lists = mla.indexer_topk(ix.q, ix.keys, ix.ctx, 2048, ix.max_ctx, key_base=ix.base)
    want = _oracle(ix.q, ix.keys, ix.ctx, 2048, base=ix.base)
    torch.cuda.synchronize()
    assert np.array_equal(lists.cpu().numpy(), want)
    cache = torch.empty((w.pool_rows, 352), dtype=torch.uint8, device=DEV)
    mla.quantize_append(w.latent, w.rope, torch.arange(w.pool_rows, device=DEV), cache)
    out, lse = mla.sparse_decode(w.q, cache, lists, w.sm_scale)
    torch.cuda.synchronize()
    ref_o, ref_l = parity.oracle_reference(w.latent, w.rope, w.q, torch.from_numpy(want.astype(np.int32)),
                                           w.sm_scale, gpu_cache=cache)
    parity.assert_close(out, lse, ref_o, ref_l, what="indexer->decode")
