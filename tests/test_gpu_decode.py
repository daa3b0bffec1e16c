"""GPU sparse MLA decode vs the oracle.

Small cases run the oracle on every token; the full-size workloads (the
15-token decode point over a 2.2M-row pool, the 128-token block-table batch,
the 4096-token prefill chunk) run in the launch configuration the benchmark
times and are checked on sampled tokens.
"""

import numpy as np
import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla
from oracle import codec
from synth import make_custom, make_workload
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fill(w, fmt="nvfp4", kv_scale=1.0):
    rows = w.latent.shape[0]
    slots = torch.arange(rows, dtype=torch.int64, device=DEV)
    if fmt == "nvfp4":
        cache = torch.empty((rows, 352), dtype=torch.uint8, device=DEV)
        mla.quantize_append(w.latent, w.rope, slots, cache)
    else:
        cache = torch.empty((rows, 576), dtype=torch.uint8, device=DEV)
        mla.fp8_quantize_append(w.latent, w.rope, slots, cache, kv_scale)
    return cache


def _run(w, cache, fmt="nvfp4", kv_scale=1.0, num_splits=0, workspace=None):
    out, lse = mla.sparse_decode(w.q, cache, w.indices, w.sm_scale, fmt=fmt, kv_scale=kv_scale,
                                 block_table=w.block_table, token_seq=w.token_seq,
                                 block_size=w.block_size, num_splits=num_splits, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def _check(w, cache, out, lse, tokens=None, fmt="nvfp4", kv_scale=1.0, what=""):
    ref_o, ref_l = parity.oracle_reference(w.latent, w.rope, w.q, w.indices, w.sm_scale, tokens=tokens,
                                           block_table=w.block_table, token_seq=w.token_seq,
                                           block_size=w.block_size, gpu_cache=cache, fmt=fmt,
                                           kv_scale=kv_scale)
    eo, el = parity.assert_close(out, lse, ref_o, ref_l, tokens=tokens, what=what or w.name)
    print(f"[{what or w.name}] worst out err / max|ref| = {eo:.2e}, worst lse err = {el:.2e}", flush=True)
    return eo, el


def test_tiny_full_parity():
    w = make_workload("tiny", DEV)
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse)


@pytest.mark.parametrize("pad_random", [False, True])
def test_padded35_full_parity(pad_random):
    w = make_workload("padded35", DEV, pad_random=pad_random)
    cache = _fill(w)
    out, lse = _run(w, cache)
    eo, el = _check(w, cache, out, lse)
    empty = [t for t in range(w.tokens) if (w.indices[t] >= 0).sum() == 0]
    assert len(empty) == 1
    assert torch.all(out[empty[0]] == 0) and torch.all(torch.isneginf(lse[empty[0]]))


@pytest.mark.parametrize("topk,valid", [(1, [1, 0, 1]), (7, [7, 3, 0]), (33, [33, 32, 1]),
                                        (100, [64, 65, 100]), (2048, [2048, 1, 777])])
def test_ragged_tiles_and_tails(topk, valid):
    w = make_custom(3000, 3, 32, topk, seed=topk, device=DEV, valid_per_token=valid)
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse, what=f"topk{topk}")


@pytest.mark.parametrize("scale", [-1.0 / 24.0, 0.0, 0.2])
def test_softmax_scale_sign_and_zero(scale):
    # a negative scale is handled by flipping q's signs; zero gives uniform
    # weights over the valid rows (also in a ragged last tile)
    w = make_custom(3000, 3, 32, 300, seed=5, device=DEV, valid_per_token=[300, 77, 1])
    w.sm_scale = scale
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse, what=f"scale{scale:+.3f}")


def _column_max(w, cache_rows_np):
    """V[t, e] = max over token t's valid rows of |decoded latent[e]|."""
    lat, _ = codec.nvfp4_decode_rows(cache_rows_np)
    idx = w.indices.cpu().numpy()
    v = np.zeros((w.tokens, 512))
    for t in range(w.tokens):
        sel = idx[t][idx[t] >= 0]
        if sel.size:
            v[t] = np.abs(lat[sel]).max(axis=0)
    return v


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64])
def test_split_count_invariance(splits):
    w = make_custom(5000, 4, 32, 2048, seed=11, device=DEV, valid_per_token=[2048, 1500, 90, 0])
    cache = _fill(w)
    ref_out, ref_lse = _run(w, cache, num_splits=1)
    out, lse = _run(w, cache, num_splits=splits)
    _check(w, cache, out, lse, what=f"splits{splits}")
    # Element-wise bound between a split and an unsplit run (derived from the
    # arithmetic: every output is a convex combination of the token's rows,
    # so each rounding below moves element e by at most that many units of
    # 2^-11 times V[t, e], the largest |row value| in column e):
    #   FP16 rounding of each split's normalised partial          1
    #   FP16 rounding of P against each run's own reference       2 (one per run)
    #   FP32 sums in a different order (n <= 2048 terms, 2^-24)   2048 * 2^-24 * 2 = 2^-2 units
    # plus the FP16 rounding of each run's output, 2^-11 * |out| per run.
    v = _column_max(w, cache.cpu().numpy())
    a = out.float().cpu().numpy()
    b = ref_out.float().cpu().numpy()
    bound = (3.25 * v[:, None, :] + np.abs(a) + np.abs(b)) * 2.0 ** -11
    assert np.all(np.abs(a - b) <= bound), float((np.abs(a - b) / np.maximum(bound, 1e-30)).max())
    fin = torch.isfinite(ref_lse)
    assert torch.equal(fin, torch.isfinite(lse))
    assert torch.allclose(lse[fin], ref_lse[fin], atol=1e-4)


def test_workspace_reuse_across_calls():
    w = make_custom(4000, 5, 32, 512, seed=12, device=DEV)
    cache = _fill(w)
    ws = mla.make_workspace(5, 32, 512, DEV, splits=6)
    first = _run(w, cache, num_splits=6, workspace=ws)
    for _ in range(3):
        again = _run(w, cache, num_splits=6, workspace=ws)
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
    # per (token, head group), 64 bytes: the arrival word (epoch << 32 |
    # arrivals), then the taken and left masks of each epoch parity.  After
    # every call the arrivals are back at zero and the epoch has moved once
    # per call; the last call (epoch 3, odd) has every slice but the last
    # arrival's own taken or left, and the next call's masks are clear.
    state = ws[:5 * 64].view(torch.int64).view(5, 8).cpu()
    assert torch.all(state[:, 0] == (4 << 32)), state
    for row in state.tolist():
        marked = row[2] | row[4]
        assert 0 <= marked < (1 << 6) and bin(marked).count("1") == 5, state
        assert row[1] == 0 and row[3] == 0, state


@pytest.mark.parametrize("tokens,splits", [(32, 16), (8, 64), (100, 5)])
def test_split_merge_when_the_grid_cannot_all_be_resident(tokens, splits):
    # More workgroups than CUs (one per CU): no split waits, and the last
    # arrival merges every unit, eight splits per batch with the running
    # maximum carried across batches.  Short and empty token lists give
    # splits with no rows (log2-sum-exp -inf) inside and across batches.
    valid = [2048 if t % 4 == 0 else (37 * t) % 2049 for t in range(tokens)]
    valid[1] = 0
    w = make_custom(20000, tokens, 32, 2048, seed=40 + splits, device=DEV, valid_per_token=valid)
    cache = _fill(w)
    out, lse = _run(w, cache, num_splits=splits)
    _check(w, cache, out, lse, tokens=sorted({0, 1, 2, 3, 5, tokens - 1}), what=f"T={tokens} S={splits}")


@pytest.mark.parametrize("tokens,splits", [(15, 8), (35, 7), (128, 2), (1, 64), (3, 3)])
def test_merge_split_between_splits_or_by_the_last_arrival(tokens, splits):
    # The slices of the split merge are combined by their own splits (they
    # wait for the others' arrival) or, with no waiting, all by the last
    # arrival: the same arithmetic in the same order, so the results are
    # bit-identical.  Polls of 1 leave most slices to the last arrival's
    # claim, which mixes both.
    w = make_custom(50000, tokens, 32, 2048, seed=30 + tokens, device=DEV)
    cache = _fill(w)
    ws = mla.make_workspace(tokens, 32, 2048, DEV, splits=splits)
    prev = mla.set_merge_polls(256)
    try:
        ref = _run(w, cache, num_splits=splits, workspace=ws)
        _check(w, cache, *ref, tokens=[0, tokens - 1], what=f"S={splits}")
        for polls in (0, 1, 256):
            mla.set_merge_polls(polls)
            got = _run(w, cache, num_splits=splits, workspace=ws)
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), polls
    finally:
        mla.set_merge_polls(prev)
    with pytest.raises(ValueError):
        mla.set_merge_polls(-1)


@pytest.mark.parametrize("heads", [16, 64, 128])
def test_head_counts(heads):
    w = make_custom(2000, 2, heads, 300, seed=heads, device=DEV, valid_per_token=[300, 150])
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse, what=f"H{heads}")


def test_bf16_queries():
    w = make_custom(3000, 3, 32, 700, seed=13, device=DEV, q_dtype=torch.bfloat16)
    cache = _fill(w)
    out, lse = _run(w, cache)
    assert out.dtype == torch.bfloat16
    _check(w, cache, out, lse, what="bf16")


def test_duplicates_and_out_of_range_indices():
    w = make_custom(1000, 2, 32, 64, seed=14, device=DEV)
    idx = w.indices.clone()
    idx[0, 10:20] = idx[0, 0]                       # a row listed 11 times counts 11 times
    idx[1, 5] = 1000                                # past the pool: masked by the guard
    idx[1, 6] = 2**31 - 1
    cache = _fill(w)
    w.indices = idx
    out, lse = _run(w, cache)
    ref_idx = idx.clone()
    ref_idx[1, 5] = -1
    ref_idx[1, 6] = -1
    w.indices = ref_idx
    _check(w, cache, out, lse, what="dups")


@pytest.mark.parametrize("splits", [1, 2, 5, 8])
@pytest.mark.parametrize("kind", ["negative", "past_pool", "unmapped_block"])
def test_masked_middle_slots_after_speculated_first_tiles(kind, splits):
    # Every list ends in a valid slot and its first tiles' rows are valid, so
    # the score waves issue their first tiles' DMA from the slot list before
    # the compaction; the masked slots further in then shift the compacted
    # rows and the split boundaries, and the waves must replace that DMA.
    bs, nblk, topk = 64, 48, 2048
    w = make_custom(bs * nblk, 3, 32, topk, seed=31, device=DEV)
    rng = np.random.default_rng(31)
    bt = np.stack([rng.permutation(nblk) for _ in range(3)]).astype(np.int32)
    idx = np.stack([rng.choice(bs * nblk, topk, replace=False) for _ in range(3)]).astype(np.int64)
    ref = idx.copy()
    # masked slots: a few in the middle and one just past the first tiles
    for t, cols in enumerate([[700], [300, 301, 1500], [64 * 4 + 1, 1024, 2000]]):
        for c in cols:
            if kind == "negative":
                idx[t, c] = -1
            elif kind == "past_pool":
                idx[t, c] = 2**31 - 1
            else:
                # a position in a block whose table entry is unmapped
                blk = int(idx[t, c]) // bs
                bt[t, blk] = -1
                ref[t, idx[t] // bs == blk] = -1          # every slot in that block is masked
            ref[t, c] = -1
    assert (idx[:, -1] >= 0).all() and (ref[:, -1] >= 0).all() or kind == "unmapped_block"
    w.indices = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    w.block_table = torch.from_numpy(bt).to(DEV)
    w.token_seq = torch.arange(3, dtype=torch.int32, device=DEV)
    w.block_size = bs
    cache = _fill(w)
    out, lse = _run(w, cache, num_splits=splits)
    w.indices = torch.from_numpy(np.where(ref < 0, -1, ref).astype(np.int32)).to(DEV)
    _check(w, cache, out, lse, what=f"masked-{kind}-S{splits}")


@pytest.mark.parametrize("bs", [64, 48, 16])
def test_block_table_small(bs):
    # power-of-two block sizes take the shift path, others the division
    w = make_custom(bs * 40, 3, 32, 200, seed=15, device=DEV)
    rng = np.random.default_rng(15)
    bt = np.stack([rng.permutation(40)[:30] for _ in range(2)]).astype(np.int32)
    bt[1, 25:] = -1                                 # unassigned blocks
    seq = np.array([0, 1, 0], dtype=np.int32)
    idx = np.stack([rng.choice(30 * bs, 200, replace=False) for _ in range(3)]).astype(np.int32)
    idx[1] = rng.choice(25 * bs, 200, replace=False)
    idx[2, 150:] = -1
    w.indices = torch.from_numpy(idx).to(DEV)
    w.block_table = torch.from_numpy(bt).to(DEV)
    w.token_seq = torch.from_numpy(seq).to(DEV)
    w.block_size = bs
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse, what=f"blocktable-bs{bs}")


@pytest.mark.parametrize("splits", [1, 3])
def test_block_table_guards_past_width_and_bad_sequences(splits):
    # Slots the block table cannot map are masked (the oracle's reading of
    # an index list through a block table): positions past the table's width
    # (token 0, mixed with valid ones), and every slot of a token whose
    # sequence is outside the table (token 1: past the last row, token 2:
    # negative), which then has out = 0 and lse = -inf.
    bs, width, seqs = 64, 20, 2
    w = make_custom(bs * 48, 4, 32, 512, seed=61, device=DEV)
    rng = np.random.default_rng(61)
    bt = np.stack([rng.permutation(48)[:width] for _ in range(seqs)]).astype(np.int32)
    idx = np.stack([rng.choice(width * bs, 512, replace=False) for _ in range(4)]).astype(np.int64)
    idx[0, 100:140] = width * bs + rng.integers(0, 5 * bs, 40)      # past the table's width
    idx[0, 500] = width * bs                                          # (first position past it)
    w.indices = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    w.block_table = torch.from_numpy(bt).to(DEV)
    w.token_seq = torch.tensor([0, seqs, -1, 1], dtype=torch.int32, device=DEV)
    w.block_size = bs
    cache = _fill(w)
    out, lse = _run(w, cache, num_splits=splits)
    _check(w, cache, out, lse, what=f"bt-guards-S{splits}")
    assert torch.all(out[1:3] == 0) and torch.all(torch.isneginf(lse[1:3]))
    # the staged gather maps (and masks) the same slots: the oracle's staged
    # rows over each slot's physical row (-1 where the table maps none)
    from oracle import attention, codec
    rows, sidx = mla.gather_dequant_fp8(cache, w.indices, 1.0, block_table=w.block_table,
                                        token_seq=w.token_seq, block_size=bs)
    torch.cuda.synchronize()
    seq = w.token_seq.cpu().numpy()
    pidx = np.full(idx.shape, -1, dtype=np.int64)
    for t in range(4):
        pidx[t] = attention.physical_rows(idx[t], int(seq[t]), bt, bs, w.pool_rows)
    pool = parity.encode_rows(parity.host(w.latent), parity.host(w.rope))
    ref_rows, ref_sidx = codec.staged_fp8_rows(pool, pidx)
    assert np.array_equal(sidx.cpu().numpy(), ref_sidx)
    assert np.array_equal(rows.cpu().numpy(), ref_rows)


def test_fp8_rows_path():
    w = make_custom(3000, 3, 32, 512, seed=16, device=DEV, valid_per_token=[512, 200, 1])
    for kv in (1.0, 0.5):
        cache = _fill(w, "fp8", kv)
        out, lse = _run(w, cache, fmt="fp8", kv_scale=kv)
        _check(w, cache, out, lse, fmt="fp8", kv_scale=kv, what=f"fp8 kv={kv}")


def test_staged_path_matches_oracle_on_staged_rows():
    from oracle import attention, codec
    w = make_custom(3000, 3, 32, 256, seed=17, device=DEV, valid_per_token=[256, 100, 0])
    cache = _fill(w)
    rows, sidx = mla.gather_dequant_fp8(cache, w.indices, 1.0)
    out, lse = mla.sparse_decode(w.q, rows, sidx, w.sm_scale, fmt="fp8", kv_scale=1.0)
    torch.cuda.synchronize()
    pool = parity.encode_rows(parity.host(w.latent), parity.host(w.rope))
    ref_rows, ref_idx = codec.staged_fp8_rows(pool, w.indices.cpu().numpy())
    assert np.array_equal(rows.cpu().numpy(), ref_rows)
    lat, rp = codec.fp8_decode_rows(ref_rows)
    ro, rl = attention.sparse_mla(parity.host(w.q), lat, rp, ref_idx, w.sm_scale)
    parity.assert_close(out, lse, ro, rl, what="staged")


# ------------------------------------------------------------ full-size workloads

def test_decode15_full_size_every_token():
    w = make_workload("decode15", DEV)
    cache = _fill(w)
    out, lse = _run(w, cache)
    _check(w, cache, out, lse, tokens=range(w.tokens))


def _batch128_tokens():
    """32 tokens, four of each residue mod 8: the launch deals a unit's
    workgroups to the XCD given by that residue."""
    return [8 * k + x for x in range(8) for k in (0, 5, 9, 15)]


def test_batch128_full_size_every_xcd_residue():
    w = make_workload("batch128", DEV)
    cache = _fill(w)
    out, lse = _run(w, cache)
    assert mla.num_splits(w.tokens, w.heads, w.topk) >= 2
    _check(w, cache, out, lse, tokens=_batch128_tokens())
    # FP8-576 comparison pool of the same shapes, one token per residue
    del cache
    c8 = _fill(w, "fp8")
    o8, l8 = _run(w, c8, fmt="fp8")
    _check(w, c8, o8, l8, tokens=[8 * 3 + x for x in range(8)], fmt="fp8", what="batch128-fp8")


@pytest.mark.parametrize("qdt", [torch.float16, torch.bfloat16])
def test_prefill4k_full_size_every_sequence(qdt):
    w = make_workload("prefill4k", DEV, q_dtype=qdt)
    cache = torch.zeros((w.pool_rows, 352), dtype=torch.uint8, device=DEV)
    # cached rows first, then the chunk's 4096 new rows through quantize-append
    new = torch.zeros(w.pool_rows, dtype=torch.bool, device=DEV)
    new[w.append_slots] = True
    old_slots = torch.nonzero(~new)[:, 0]
    mla.quantize_append(w.latent[old_slots], w.rope[old_slots], old_slots, cache)
    mla.quantize_append(w.latent[w.append_slots], w.rope[w.append_slots], w.append_slots, cache)
    out, lse = _run(w, cache)
    # the first, a middle and the last token of each of the 4 sequences
    toks = [b * 1024 + j for b in range(4) for j in (0, 517, 1023)]
    _check(w, cache, out, lse, tokens=toks, what=f"prefill4k-{qdt}")


def _finite_e4m3_codes():
    """All 256 byte values with the two NaN codes replaced by zeros: every
    finite E4M3 code appears."""
    c = np.arange(256, dtype=np.uint8)
    c[0x7F], c[0xFF] = 0x00, 0x80
    return c


@pytest.mark.parametrize("fmt,kv", [("nvfp4", 1.0), ("fp8", 1.0), ("fp8", 0.5)])
def test_every_rope_code_through_the_score_path(fmt, kv):
    """A single valid slot's lse is its score.  With q one-hot on rope
    dimension d and sm_scale 1, lse equals the decoded rope value, so every
    E4M3 code passes through the kernel's own rope decode and score MFMA."""
    rng = np.random.default_rng(77)
    codes = _finite_e4m3_codes().reshape(4, 64)
    width = 352 if fmt == "nvfp4" else 576
    rows = rng.integers(0, 256, size=(4, width), dtype=np.uint8)
    if fmt == "nvfp4":
        rows[:, 256:288] = rng.integers(0, 0x7F, size=(4, 32), dtype=np.uint8)   # finite scales
        rows[:, 288:] = codes
    else:
        lat = rows[:, :512]
        lat[(lat & 0x7F) == 0x7F] = 0
        rows[:, 512:] = codes
    cache = torch.from_numpy(rows).to(DEV)
    T, H = 16, 16
    q = torch.zeros((T, H, 576), dtype=torch.float16, device=DEV)
    idx = torch.full((T, 8), -1, dtype=torch.int32, device=DEV)
    for t in range(T):
        idx[t, 5] = t // 4
        for h in range(H):
            q[t, h, 512 + 16 * (t % 4) + h] = 1.0
    out, lse = mla.sparse_decode(q, cache, idx, 1.0, fmt=fmt, kv_scale=kv)
    torch.cuda.synchronize()
    vals = codec.e4m3_decode(codes) * (kv if fmt == "fp8" else 1.0)      # [4, 64]
    want = np.array([[vals[t // 4, 16 * (t % 4) + h] for h in range(H)] for t in range(T)])
    got = lse.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("kv", [1.0, 0.5, 2.0])
def test_every_fp8_latent_code_decodes_exactly_through_attention(kv):
    """FP8-576 rows: a single valid slot with q = 0 returns the row's latent
    exactly (byte value * kv_scale), for every finite E4M3 code."""
    codes = _finite_e4m3_codes()
    rows = np.zeros((3, 576), dtype=np.uint8)
    rows[0, :256], rows[0, 256:512] = codes, codes[::-1]
    rows[1, :512] = np.roll(np.concatenate([codes, codes]), 77)
    rows[2, :512] = codes[np.random.default_rng(5).integers(0, 256, 512)]
    rows[:, 512:] = codes[:64]
    cache = torch.from_numpy(rows).to(DEV)
    T = 3
    q = torch.zeros((T, 32, 576), dtype=torch.float16, device=DEV)
    idx = torch.full((T, 16), -1, dtype=torch.int32, device=DEV)
    idx[:, 9] = torch.arange(T, dtype=torch.int32, device=DEV)
    out, lse = mla.sparse_decode(q, cache, idx, 0.1, fmt="fp8", kv_scale=kv)
    torch.cuda.synchronize()
    want, _ = codec.fp8_decode_rows(rows, kv)
    got = out.float().cpu().numpy()
    for t in range(T):
        for h in (0, 17, 31):
            assert np.array_equal(got[t, h], want[t]), (t, h)
    assert np.all(lse.cpu().numpy() == 0.0)


def test_kernel_timing_hook():
    """The benchmark timing hook records the kernel's own duration and leaves results unchanged."""
    w = make_custom(3000, 2, 32, 512, seed=31, device=DEV)
    cache = _fill(w)
    plain = _run(w, cache)
    mla.kernel_timing(True)
    try:
        timed = _run(w, cache)
        ms = mla.last_kernel_ms()
    finally:
        mla.kernel_timing(False)
    assert 0.0 < ms < 100.0
    assert torch.equal(plain[0], timed[0]) and torch.equal(plain[1], timed[1])
