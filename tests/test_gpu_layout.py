"""GPU pack / unpack of a request's blocks against the pool oracle (bytes
bit for bit, both pool layouts), and an end-to-end move of a request from
one pool to another: the pool manager places it, quantize-append writes its
rows, pack + unpack move its blocks, and the decode through the new block
table gives what it gave through the old one."""

import numpy as np
import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla
from oracle import pool as opool
from synth import make_custom

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("layout", ["layer", "block"])
def test_pack_unpack_bit_exact(layout):
    n_blocks, layers, rows, rb = 50, 3, 64, 352
    region = rows * rb
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    pool_t = torch.randint(0, 256, (n_blocks * layers * region,), generator=g, dtype=torch.uint8, device=DEV)
    ids = torch.tensor([7, 0, 49, 13, 50, -1, 21], dtype=torch.int32, device=DEV)   # 50, -1: no such block
    staging = torch.zeros(ids.numel() * layers * region, dtype=torch.uint8, device=DEV)
    mla.kv_pack_blocks(pool_t, layout, n_blocks, layers, ids, staging)
    torch.cuda.synchronize()
    pool_np = pool_t.cpu().numpy()
    want = opool.pack(pool_np, layout, n_blocks, layers, region, ids.cpu().numpy())
    assert np.array_equal(staging.cpu().numpy(), want)
    dst = torch.zeros_like(pool_t)
    new_ids = torch.tensor([3, 4, 5, 6, 8, 9, 40], dtype=torch.int32, device=DEV)
    mla.kv_unpack_blocks(staging, new_ids, dst, layout, n_blocks, layers)
    torch.cuda.synchronize()
    want_pool = opool.unpack(want, new_ids.cpu().numpy(), np.zeros_like(pool_np), layout, n_blocks, layers, region)
    assert np.array_equal(dst.cpu().numpy(), want_pool)


def test_request_moves_between_pools_and_decodes_the_same():
    layers, row = 2, 352
    # prefill side: a pool fragmented by another request; decode side: a fresh pool
    src_mgr = mla.Pool(60 * 64 * layers * row, layers, row, 0, max_seqs=3, max_blocks_per_seq=40)
    dst_mgr = mla.Pool(80 * 64 * layers * row, layers, row, 0, max_seqs=3, max_blocks_per_seq=40)
    assert src_mgr.reserve(1, 64 * 7) and src_mgr.reserve(2, 64 * 5)
    src_mgr.release(1)
    ctx = 1500
    assert src_mgr.reserve(0, ctx)
    assert dst_mgr.reserve(2, 64 * 11) and dst_mgr.reserve(0, ctx)
    region = 64 * row
    src_pool = torch.zeros(src_mgr.num_blocks * layers * region, dtype=torch.uint8, device=DEV)
    dst_pool = torch.zeros(dst_mgr.num_blocks * layers * region, dtype=torch.uint8, device=DEV)
    w = make_custom(ctx, 3, 32, 256, seed=44, device=DEV)        # values of the request's positions
    slots = src_mgr.slots(0, 0, ctx).to(DEV)
    layer_rows = src_mgr.num_blocks * 64
    for l in range(layers):                                       # layer-major: layer l's rows are one cache
        cache_l = src_pool[l * layer_rows * row:(l + 1) * layer_rows * row].view(layer_rows, row)
        mla.quantize_append(w.latent * (l + 1), w.rope, slots, cache_l)
    src_ids = torch.tensor([b for b in src_mgr.block_table()[0].tolist() if b >= 0], dtype=torch.int32, device=DEV)
    dst_ids = torch.tensor([b for b in dst_mgr.block_table()[0].tolist() if b >= 0], dtype=torch.int32, device=DEV)
    assert src_ids.numel() == dst_ids.numel() == -(-ctx // 64)
    staging = torch.empty(src_ids.numel() * layers * region, dtype=torch.uint8, device=DEV)
    mla.kv_pack_blocks(src_pool, "layer", src_mgr.num_blocks, layers, src_ids, staging)
    mla.kv_unpack_blocks(staging, dst_ids, dst_pool, "layer", dst_mgr.num_blocks, layers)
    seq = torch.zeros(3, dtype=torch.int32, device=DEV)           # every token reads sequence 0
    for l in range(layers):
        outs = []
        for mgr, pool_t in ((src_mgr, src_pool), (dst_mgr, dst_pool)):
            rows_l = mgr.num_blocks * 64
            cache_l = pool_t[l * rows_l * row:(l + 1) * rows_l * row].view(rows_l, row)
            bt = mgr.block_table()[:1].to(DEV)
            outs.append(mla.sparse_decode(w.q, cache_l, w.indices, w.sm_scale, block_table=bt,
                                          token_seq=seq, block_size=64))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # and the staging buffer is one block-major run of the request's bytes
    d, nbytes = src_mgr.descriptors(0, "block")
    assert nbytes == staging.numel()
