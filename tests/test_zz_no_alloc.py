"""The allocation-free decode entry point (mla_sparse_decode_noalloc) gives
what mla_sparse_decode gives with a workspace of its own, call after call.

Two calls in a row share the library's scratch array: the first with many
units and split partials, the second smaller and with another layout (more
head groups, another split count, a block table).  Each is compared with the
entry point that takes a workspace, on the same inputs and split count
(bit for bit: the kernels are the same), and the first also with the oracle.
"""

import numpy as np
import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla
from synth import make_custom
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cache(w):
    cache = torch.empty((w.latent.shape[0], 352), dtype=torch.uint8, device=DEV)
    mla.quantize_append(w.latent, w.rope, torch.arange(w.latent.shape[0], device=DEV), cache)
    return cache


def _both(w, cache, splits, **kw):
    T, H = w.tokens, w.heads
    out_a = torch.empty((T, H, 512), dtype=w.q.dtype, device=DEV)
    lse_a = torch.empty((T, H), dtype=torch.float32, device=DEV)
    mla.sparse_decode_noalloc(w.q, cache, w.indices, w.sm_scale, out_a, lse_a, num_splits=splits, **kw)
    out_b, lse_b = mla.sparse_decode(w.q, cache, w.indices, w.sm_scale, num_splits=splits, **kw)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b


def test_noalloc_matches_workspace_entry_on_two_calls():
    # call 1: 24 tokens x 32 heads, 4 splits (partials in the scratch array)
    w1 = make_custom(6000, 24, 32, 2048, seed=21, device=DEV,
                     valid_per_token=[2048, 1999, 0, 17] + [1024] * 20)
    c1 = _cache(w1)
    a, la, b, lb = _both(w1, c1, 4)
    assert torch.equal(a, b) and torch.equal(la, lb)
    ref_o, ref_l = parity.oracle_reference(w1.latent, w1.rope, w1.q, w1.indices, w1.sm_scale,
                                           tokens=[0, 2, 3, 23], gpu_cache=c1)
    parity.assert_close(a, la, ref_o, ref_l, tokens=[0, 2, 3, 23], what="noalloc-1")

    # call 2, smaller: 5 tokens x 64 heads (two head groups), 7 splits, block table
    w2 = make_custom(64 * 40, 5, 64, 300, seed=22, device=DEV)
    rng = np.random.default_rng(22)
    bt = np.stack([rng.permutation(40)[:30] for _ in range(3)]).astype(np.int32)
    bt[2, 20:] = -1
    w2.block_table = torch.from_numpy(bt).to(DEV)
    w2.token_seq = torch.tensor([0, 1, 2, 1, 7], dtype=torch.int32, device=DEV)
    w2.indices = torch.from_numpy(np.stack([rng.choice(30 * 64, 300, replace=False)
                                            for _ in range(5)]).astype(np.int32)).to(DEV)
    c2 = _cache(w2)
    kw = dict(block_table=w2.block_table, token_seq=w2.token_seq, block_size=64)
    a, la, b, lb = _both(w2, c2, 7, **kw)
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert torch.all(a[4] == 0) and torch.all(torch.isneginf(la[4]))     # sequence 7 is not in the table

    # the first shape again after the smaller call: the counters were left at zero
    a, la, b, lb = _both(w1, c1, 4)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_noalloc_rejects_calls_beyond_its_scratch():
    w = make_custom(3000, 300, 32, 2048, seed=23, device=DEV)
    cache = _cache(w)
    out = torch.empty((300, 32, 512), dtype=torch.float16, device=DEV)
    lse = torch.empty((300, 32), dtype=torch.float32, device=DEV)
    with pytest.raises(mla.MlaError):
        mla.sparse_decode_noalloc(w.q, cache, w.indices, w.sm_scale, out, lse, num_splits=8)
    # the same tokens with one split need no partials and fit
    mla.sparse_decode_noalloc(w.q, cache, w.indices, w.sm_scale, out, lse, num_splits=1)
    ref, ref_l = mla.sparse_decode(w.q, cache, w.indices, w.sm_scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_l)
