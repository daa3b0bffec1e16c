"""GPU quantize-append (and the staged step's re-encode) vs the oracle, bit for bit."""

import numpy as np
import pytest
import torch

import nvfp4_compressed_sparse_mla_amd as mla
from oracle import codec
from synth import pool_values
import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quantize(lat, rope, slots=None, rows=None):
    n = lat.shape[0]
    rows = n if rows is None else rows
    cache = torch.zeros((rows, 352), dtype=torch.uint8, device=DEV)
    if slots is None:
        slots = torch.arange(n, dtype=torch.int64, device=DEV)
    mla.quantize_append(lat, rope, slots, cache)
    torch.cuda.synchronize()
    return cache


def test_pool_rows_bit_exact():
    lat, rope = pool_values(4096, 0, DEV)
    cache = _quantize(lat, rope)
    ref = parity.encode_rows(parity.host(lat), parity.host(rope))
    got = cache.cpu().numpy()
    assert np.array_equal(got, ref), f"{(got != ref).any(1).sum()} rows differ"


def _adversarial_rows():
    """Blocks built to hit every rounding decision: ties, scale midpoints, zeros, signs, saturation."""
    rng = np.random.default_rng(21)
    rows = []
    e4 = codec.E4M3_POS
    # scale ties: amax = 6 * midpoint between E4M3 neighbours, all fp16-exact ones
    mids = [(a + b) / 2 for a, b in zip(e4[:-1], e4[1:])]
    amaxes = [6 * m for m in mids] + [6 * v for v in e4] + [6 * 2.0 ** -10, 3000.0, 60000.0, 0.0]
    amaxes = [a for a in amaxes if np.isfinite(np.float16(a)) and np.float16(a) == a]
    for a in amaxes:
        row = np.zeros(576)
        for g in range(32):
            s = a / 6
            blk = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.1, 6.0, 7.0], size=16) * s
            blk *= rng.choice([-1.0, 1.0], size=16)
            blk = np.clip(blk, -65504.0, 65504.0)        # inputs stay finite fp16 values
            blk[0] = a
            row[16 * g: 16 * g + 16] = blk
        row[512:] = rng.choice(list(e4[:-1] + np.diff(e4) / 2) + list(e4), size=64) * rng.choice([-1, 1], 64)
        rows.append(row)
    r = np.array(rows).astype(np.float16)
    r[0, 3] = np.float16(-0.0)
    r[1, 512] = np.float16(-0.0)
    r[2, 16:32] = np.float16(-(2.0 ** -20))            # scale rounds to zero, sign kept
    r[3, 512:520] = np.float16(500.0)                  # rope saturates
    return r


def test_adversarial_rows_bit_exact():
    r = _adversarial_rows()
    lat = torch.from_numpy(r[:, :512].copy()).to(DEV)
    rope = torch.from_numpy(r[:, 512:].copy()).to(DEV)
    cache = _quantize(lat, rope)
    ref = codec.nvfp4_encode_rows(r[:, :512].astype(np.float64), r[:, 512:].astype(np.float64))
    got = cache.cpu().numpy()
    bad = np.nonzero((got != ref).any(1))[0]
    assert bad.size == 0, f"rows {bad[:5]} differ: got {got[bad[0]][:16]} want {ref[bad[0]][:16]}"


def test_bf16_inputs_bit_exact():
    lat, rope = pool_values(1024, 5, DEV)
    latb = (lat.float() * 3.7).to(torch.bfloat16)
    ropeb = rope.to(torch.bfloat16)
    cache = _quantize(latb, ropeb)
    ref = parity.encode_rows(parity.host(latb), parity.host(ropeb))
    assert np.array_equal(cache.cpu().numpy(), ref)


def test_slots_strides_and_skips():
    lat, rope = pool_values(300, 6, DEV)
    big = torch.zeros((300, 640), dtype=torch.float16, device=DEV)
    big[:, :512] = lat
    big_r = torch.zeros((300, 72), dtype=torch.float16, device=DEV)
    big_r[:, :64] = rope
    slots = torch.randperm(1000, device=DEV)[:300].to(torch.int64)
    slots[::7] = -1                                   # skipped
    slots[5] = 5000                                   # out of range: skipped
    cache = torch.full((1000, 352), 0xAB, dtype=torch.uint8, device=DEV)
    mla.quantize_append(big[:, :512], big_r[:, :64], slots, cache)
    torch.cuda.synchronize()
    ref = parity.encode_rows(parity.host(lat), parity.host(rope))
    got = cache.cpu().numpy()
    s = slots.cpu().numpy()
    written = np.zeros(1000, bool)
    for i, sl in enumerate(s):
        if 0 <= sl < 1000:
            assert np.array_equal(got[sl], ref[i]), i
            written[sl] = True
    assert np.all(got[~written] == 0xAB)


def test_fp8_rows_bit_exact():
    lat, rope = pool_values(2048, 7, DEV)
    cache = torch.zeros((2048, 576), dtype=torch.uint8, device=DEV)
    mla.fp8_quantize_append(lat, rope, torch.arange(2048, device=DEV), cache, kv_scale=1.0)
    cache2 = torch.zeros((2048, 576), dtype=torch.uint8, device=DEV)
    mla.fp8_quantize_append(lat, rope, torch.arange(2048, device=DEV), cache2, kv_scale=0.25)
    torch.cuda.synchronize()
    ref = parity.encode_rows(parity.host(lat), parity.host(rope), fmt="fp8", kv_scale=1.0)
    ref2 = parity.encode_rows(parity.host(lat), parity.host(rope), fmt="fp8", kv_scale=0.25)
    assert np.array_equal(cache.cpu().numpy(), ref)
    assert np.array_equal(cache2.cpu().numpy(), ref2)


def test_quantize_is_deterministic():
    lat, rope = pool_values(8192, 8, DEV)
    a = _quantize(lat, rope)
    b = _quantize(lat, rope)
    assert torch.equal(a, b)


def _exhaustive_cache():
    """NVFP4 rows (built by the oracle from codes) holding every (code, scale) pair
    and every rope byte: 254 finite scale bytes x 16 codes, 256 rope bytes."""
    scales = [c for c in range(256) if c & 0x7F != 0x7F]
    n_rows = (len(scales) + 31) // 32
    rows = np.zeros((n_rows, 352), dtype=np.uint8)
    codes = np.arange(16, dtype=np.uint8)
    nib = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)        # the 16 codes in one group
    for i, sc in enumerate(scales):
        r, g = divmod(i, 32)
        rows[r, 8 * g: 8 * g + 8] = nib
        rows[r, 256 + g] = sc
    for r in range(n_rows):
        rows[r, 288:] = (np.arange(64) + 64 * r) % 256
    rows[:, 288:][(rows[:, 288:] & 0x7F) == 0x7F] = 0x00             # no NaN rope bytes
    return rows


def test_every_code_scale_pair_decodes_exactly_through_attention():
    """A single valid slot returns that row's latent exactly, so the output shows
    the on-chip decode of every (E2M1 code, E4M3 scale) pair."""
    rows = _exhaustive_cache()
    n = rows.shape[0]
    cache = torch.from_numpy(rows).to(DEV)
    q = torch.zeros((n, 32, 576), dtype=torch.float16, device=DEV)
    idx = torch.full((n, 8), -1, dtype=torch.int32, device=DEV)
    idx[:, 3] = torch.arange(n, dtype=torch.int32, device=DEV)
    out, lse = mla.sparse_decode(q, cache, idx, 0.1, num_splits=1)
    torch.cuda.synchronize()
    want, _ = codec.nvfp4_decode_rows(rows)
    got = out.float().cpu().numpy()
    for t in range(n):
        assert np.array_equal(got[t, 0], want[t]), t
        assert np.array_equal(got[t, 31], want[t]), t
    assert np.all(lse.cpu().numpy() == 0.0)             # q = 0: lse = ln 1


def test_staged_rows_bit_exact_and_rope_decode():
    """The staged step decodes on chip and re-encodes: its bytes match the
    oracle's, and rope bytes (E4M3 -> FP16 -> E4M3) come back unchanged."""
    rows = _exhaustive_cache()
    lat, rope = pool_values(512, 9, DEV)
    pool = np.concatenate([rows, parity.encode_rows(parity.host(lat), parity.host(rope))])
    cache = torch.from_numpy(pool).to(DEV)
    rng = np.random.default_rng(3)
    idx = rng.integers(0, pool.shape[0], size=(5, 200)).astype(np.int32)
    idx[:, ::9] = -1
    idx[0, :rows.shape[0]] = np.arange(rows.shape[0])
    t_idx = torch.from_numpy(idx).to(DEV)
    st_rows, st_idx = mla.gather_dequant_fp8(cache, t_idx, 1.0)
    torch.cuda.synchronize()
    ref_rows, ref_idx = codec.staged_fp8_rows(pool, idx, 1.0)
    assert np.array_equal(st_idx.cpu().numpy(), ref_idx)
    assert np.array_equal(st_rows.cpu().numpy(), ref_rows)
    assert np.array_equal(st_rows.cpu().numpy()[: rows.shape[0], 512:], rows[:, 288:])
