"""Pins for the oracle codec (CPU only).

Each test checks the oracle against something other than itself: the
hand-written format tables in tests/golden, torch's float8_e4m3fn cast (a
library routine), exact rational brute force (fractions.Fraction nearest
search written here from the rounding rule), closed-form round trips, and
the row sizes the Prime Inference write-up gives ("Making room for
low-latency decode": 576 bytes -> 352 bytes).
"""

import os
from fractions import Fraction as Fr

import numpy as np
import pytest
import torch

from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- brute force


def _fr_e4m3(code):
    """Exact value of a non-NaN E4M3 byte from its bit fields (written here, not imported)."""
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    mag = Fr(m, 8) * Fr(1, 64) if e == 0 else Fr(2) ** (e - 7) * (1 + Fr(m, 8))
    return sign * mag


E4M3_FR = [_fr_e4m3(c) for c in range(127)]                 # non-negative finite values
E2M1_FR = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def _bf_nearest_even(a, grid):
    """Index of grid point nearest to a (exact), ties to the even index."""
    best, best_d = None, None
    for k, g in enumerate(grid):
        d = abs(a - g)
        if best_d is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return best


def _is_neg(x: float) -> bool:
    return bool(np.signbit(x))


def bf_e4m3(x: float) -> int:
    return (0x80 if _is_neg(x) else 0) | _bf_nearest_even(abs(Fr(x)), E4M3_FR)


def bf_scale(amax: float) -> int:
    return _bf_nearest_even(Fr(amax) / 6, E4M3_FR)


def bf_e2m1(x: float, s: Fr) -> int:
    sign = 0x8 if _is_neg(x) else 0
    if s == 0:
        return sign
    return sign | _bf_nearest_even(abs(Fr(x)), [g * s for g in E2M1_FR])


def _fp16(vals):
    return np.asarray(vals, dtype=np.float16).astype(np.float64)


# ---------------------------------------------------------------- tables


def _golden_values():
    e2, e4 = {}, {}
    with open(os.path.join(GOLDEN, "e2m1_e4m3_values.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            kind, code, val = line.split()
            (e2 if kind == "e2m1" else e4)[int(code, 16)] = float(val)
    return e2, e4


def test_e2m1_table_matches_format_definition():
    e2, _ = _golden_values()
    assert len(e2) == 16
    for code, val in e2.items():
        got = codec.e2m1_decode(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e4m3_landmarks_match_format_definition():
    _, e4 = _golden_values()
    for code, val in e4.items():
        got = codec.e4m3_decode(code)
        assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)
    assert np.isnan(codec.e4m3_decode(0x7F)) and np.isnan(codec.e4m3_decode(0xFF))


def test_e4m3_table_matches_torch_for_every_code():
    raw = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codec.e4m3_decode(np.arange(256))
    finite = ~np.isnan(raw)
    assert finite.sum() == 254
    assert np.array_equal(np.isnan(ours), ~finite)
    assert np.array_equal(ours[finite], raw[finite])
    assert np.array_equal(np.signbit(ours[finite]), np.signbit(raw[finite]))


def test_e4m3_table_matches_bit_fields():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert Fr(float(codec.e4m3_decode(c))) == _fr_e4m3(c)


# ---------------------------------------------------------------- E4M3 encode


def _e4m3_adversarial():
    vals = [0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 448.0, 449.0,
            464.0, 465.0, 480.0, 1e4, -1e4, 65504.0]
    pos = sorted(set(E4M3_FR))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        for v in (a, b, mid):
            vals.append(float(v))
            vals.append(-float(v))
        # just either side of the midpoint, still exact in FP64
        eps = (b - a) / 1024
        vals += [float(mid - eps), float(mid + eps)]
    return vals


def test_e4m3_encode_brute_force_adversarial():
    vals = _e4m3_adversarial()
    got = codec.e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert int(g) == bf_e4m3(v), (v, hex(int(g)), hex(bf_e4m3(v)))


def test_e4m3_encode_brute_force_random_fp16():
    rng = np.random.default_rng(123)
    vals = np.concatenate([
        rng.standard_normal(1500) * np.exp(rng.uniform(-12, 7, 1500)),
        rng.uniform(-500, 500, 300),
    ])
    vals = _fp16(vals)
    got = codec.e4m3_encode(vals)
    for v, g in zip(vals, got):
        assert int(g) == bf_e4m3(float(v)), (v, hex(int(g)))


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    vals = _fp16(rng.standard_normal(200_000) * np.exp(rng.uniform(-10, 5, 200_000)))
    vals = vals[np.abs(vals) <= 448.0]
    ref = torch.from_numpy(vals).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codec.e4m3_encode(vals), ref)


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    assert np.array_equal(codec.e4m3_encode(codec.e4m3_decode(codes)), codes.astype(np.uint8))


# ---------------------------------------------------------------- group scale


def test_group_scale_brute_force_adversarial():
    amax = [0.0, 2.0 ** -24, 6 * 2.0 ** -10, 6 * 2.0 ** -10 * 1.0001, 2688.0, 2700.0, 60000.0]
    pos = sorted(set(E4M3_FR))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        for v in (6 * a, 6 * mid, 6 * b):
            f16 = np.float16(float(v))
            if np.isfinite(f16):
                amax.append(float(f16))
                amax.append(float(np.nextafter(f16, np.float16(np.inf))))
                amax.append(float(np.nextafter(f16, np.float16(0))))
    amax = np.array(amax)
    lat = np.zeros((len(amax), 512))
    lat[:, 0] = amax                                       # group 0 carries the amax
    lat[:, 17] = -amax                                     # group 1 carries it with a minus sign
    sc = codec.nvfp4_group_scales(lat)
    for i, a in enumerate(amax):
        assert int(sc[i, 0]) == bf_scale(a), (a, hex(int(sc[i, 0])), hex(bf_scale(a)))
        assert int(sc[i, 1]) == bf_scale(a)
        assert int(sc[i, 2]) == 0


def test_group_scale_float32_division_equivalence():
    """fp32 amax/6 rounded then RNE'd to E4M3 equals the exact-quotient rule."""
    rng = np.random.default_rng(11)
    a16 = _fp16(np.abs(rng.standard_normal(100_000)) * np.exp(rng.uniform(-12, 9, 100_000)))
    a16 = a16[np.isfinite(a16)]
    q32 = (a16.astype(np.float32) / np.float32(6.0)).astype(np.float64)
    via_fp32 = codec.e4m3_encode(q32)
    exact = codec.e4m3_encode_quotient(a16, 6.0)
    assert np.array_equal(via_fp32, exact)


# ---------------------------------------------------------------- E2M1 encode


def test_e2m1_tie_cases_go_to_even_code():
    # midpoint t between grid neighbours -> expected magnitude code (even one)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for s_code in (0x01, 0x07, 0x08, 0x30, 0x38, 0x3B, 0x55, 0x7E):
        s = float(codec.e4m3_decode(s_code))
        for t, want in ties.items():
            for sign in (1.0, -1.0):
                x = sign * t * s
                got = int(codec.e2m1_encode(np.array([x]), np.array([s]))[0])
                assert got == (want | (0x8 if sign < 0 else 0)), (s, t, sign, got)
        # past the largest point saturates to 6
        assert int(codec.e2m1_encode(np.array([7.5 * s]), np.array([s]))[0]) == 7
        assert int(codec.e2m1_encode(np.array([-100 * s]), np.array([s]))[0]) == 0xF


def test_e2m1_encode_brute_force_random_blocks():
    rng = np.random.default_rng(5)
    n_blocks = 120
    z = rng.standard_normal((n_blocks, 16)) * np.exp(rng.uniform(-9, 6, (n_blocks, 1)))
    x = _fp16(z)
    sc = codec.nvfp4_group_scales(np.pad(x, ((0, 0), (0, 496))))[:, 0]
    s = codec.e4m3_decode(sc)
    got = codec.e2m1_encode(x, s[:, None])
    for b in range(n_blocks):
        assert int(sc[b]) == bf_scale(float(np.abs(x[b]).max()))
        sf = _fr_e4m3(int(sc[b]))
        for j in range(16):
            assert int(got[b, j]) == bf_e2m1(float(x[b, j]), sf), (b, j, x[b, j])


def test_signed_zero_and_zero_scale():
    lat = np.zeros((1, 512))
    lat[0, 0] = -0.0
    lat[0, 16:32] = -(2.0 ** -14)                          # amax/6 < 2**-10 -> scale 0
    lat[0, 33] = -2.0 ** -24
    lat[0, 32] = 1.0                                        # group 2: tiny negative rounds to 0
    rope = np.zeros((1, 64))
    rope[0, 0] = -0.0
    rope[0, 1] = -(2.0 ** -12)                              # rounds to zero, keeps sign
    row = codec.nvfp4_encode_rows(lat, rope)[0]
    assert row[0] & 0xF == 0x8                              # -0.0 keeps its sign
    assert row[256] == 0 and row[257] == 0                  # scales 0
    assert all(b == 0x88 for b in row[8:16])                # sign-only codes
    assert row[16] >> 4 == 0x8                              # element 33: tiny negative
    assert row[288] == 0x80 and row[289] == 0x80
    lat_d, rope_d = codec.nvfp4_decode_rows(row[None])
    assert np.all(lat_d[0, 16:32] == 0.0)


# ---------------------------------------------------------------- the 352-byte row


def test_row_sizes_match_the_pages():
    assert codec.NIBBLE_BYTES + codec.N_GROUPS + codec.ROPE_DIM == 352 == codec.ROW_BYTES
    assert codec.LATENT_DIM + codec.ROPE_DIM == 576 == codec.FP8_ROW_BYTES
    assert codec.GROUP == 16


def _read_handbuilt():
    out = {}
    with open(os.path.join(GOLDEN, "nvfp4_row_handbuilt.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = [int(v, 16) for v in vals]
    return out


def test_handbuilt_row_golden():
    g = _read_handbuilt()
    C = [6, 0.5, -1, 1.5, 2, -3, 4, 0, -6, 0.5, 1, -1.5, -2, 3, -4, 6]
    lat = np.array([[C[j] * 2.0 ** (gi % 4 - 1) for gi in range(32) for j in range(16)]])
    rope_codes = [(0x80 if r % 2 else 0) | (0x20 + r) for r in range(64)]
    rope = np.array([[float(_fr_e4m3(c)) for c in rope_codes]])
    row = codec.nvfp4_encode_rows(_fp16(lat), _fp16(rope))[0]
    for gi in range(32):
        assert list(row[8 * gi: 8 * gi + 8]) == g["group_bytes"], gi
    assert list(row[256:288]) == g["scale_bytes"] * 8
    assert list(row[288:296]) == g["rope_first8"]
    assert list(row[350:352]) == g["rope_last2"]
    assert list(row[288:]) == rope_codes
    lat_d, rope_d = codec.nvfp4_decode_rows(row[None])
    assert np.array_equal(lat_d[0], lat[0]) and np.array_equal(rope_d[0], rope[0])


def test_row_round_trip_on_exact_grid_values():
    """x = c * s with max|c| = 6 and s an E4M3 value comes back exactly."""
    rng = np.random.default_rng(3)
    n = 64
    codes = rng.integers(0, 16, size=(n, 32, 16))
    codes[:, :, rng.integers(16)] = rng.choice([0x7, 0xF], size=(n, 32))   # one |c| = 6 per group
    s_codes = rng.integers(1, 0x7F, size=(n, 32))
    vals = np.array([[[float(Fr(E2M1_FR[c & 7]) * (-1 if c & 8 else 1)) for c in grp] for grp in row]
                     for row in codes])
    s = np.array([[float(_fr_e4m3(int(c))) for c in row] for row in s_codes])
    lat = (vals * s[:, :, None]).reshape(n, 512)
    assert np.array_equal(_fp16(lat), lat)                 # all exact in fp16
    rope = _fp16(rng.standard_normal((n, 64)))
    rows = codec.nvfp4_encode_rows(lat, rope)
    assert np.array_equal(rows[:, 256:288], s_codes.astype(np.uint8))
    lat_d, _ = codec.nvfp4_decode_rows(rows)
    assert np.array_equal(lat_d, lat)


def test_decode_products_exact_in_fp16():
    """Every (E2M1 code, E4M3 scale) product is an fp16 value."""
    prod = codec.E2M1_TABLE[:, None] * codec.e4m3_decode(np.arange(256))[None, :]
    fin = np.isfinite(prod)
    assert np.array_equal(prod[fin].astype(np.float16).astype(np.float64), prod[fin])


# ---------------------------------------------------------------- FP8 rows and staging


def test_fp8_rows_match_torch_cast():
    rng = np.random.default_rng(9)
    lat = _fp16(rng.standard_normal((50, 512)) * 3)
    rope = _fp16(rng.standard_normal((50, 64)))
    rows = codec.fp8_encode_rows(lat, rope)
    ref = torch.from_numpy(np.concatenate([lat, rope], 1)).to(torch.float8_e4m3fn)
    assert np.array_equal(rows, ref.view(torch.uint8).numpy())
    l2, r2 = codec.fp8_decode_rows(rows)
    assert np.array_equal(l2, ref.to(torch.float64).numpy()[:, :512])


def _fp8_scaled_case(kv, seed):
    """fp16 rows whose quotients v / kv stay below 464 (torch's cast turns
    larger values into NaN instead of saturating), with E4M3 rounding
    midpoints times kv planted among them."""
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((40, 512)) * np.exp(rng.standard_normal((40, 1)))
    grid = codec.E4M3_POS
    mids = (grid[1:] + grid[:-1]) / 2                  # exact in FP64
    lat[:, :len(mids)] = mids * kv * np.where(rng.random(len(mids)) < 0.5, -1, 1)
    lat = np.clip(lat, -440 * kv, 440 * kv)
    rope = rng.standard_normal((40, 64)) * 4 * kv
    return _fp16(lat), _fp16(rope)


def _fp8_scaled_matches_torch(kv, seed):
    lat, rope = _fp8_scaled_case(kv, seed)
    rows = codec.fp8_encode_rows(lat, rope, kv)
    v = np.concatenate([lat, rope], 1)
    # v / kv is exact in float32 (kv is a power of two, v an fp16 value)
    ref = torch.from_numpy((v / kv).astype(np.float32)).to(torch.float8_e4m3fn)
    if not np.array_equal(rows, ref.view(torch.uint8).numpy()):
        return False
    l2, r2 = codec.fp8_decode_rows(rows, kv)
    dec = ref.to(torch.float64).numpy() * kv
    return np.array_equal(l2, dec[:, :512]) and np.array_equal(r2, dec[:, 512:])


@pytest.mark.parametrize("kv", [0.25, 0.5, 2.0])
def test_fp8_rows_with_kv_scale_match_torch_cast(kv):
    """Bytes are E4M3(v / kv_scale) and decode to byte value * kv_scale, as
    torch's float8_e4m3fn cast of the quotient gives them (ties included)."""
    assert _fp8_scaled_matches_torch(kv, 20 + int(4 * kv))


@pytest.mark.parametrize("kv", [0.25, 2.0])
def test_fp8_rows_with_kv_scale_saturate(kv):
    lat = np.zeros((1, 512))
    lat[0, :4] = [464 * kv, -1e4 * kv, 448 * kv, -449 * kv]
    rows = codec.fp8_encode_rows(_fp16(lat), np.zeros((1, 64)), kv)
    assert rows[0, :4].tolist() == [0x7E, 0xFE, 0x7E, 0xFE]


def test_fp8_kv_scale_pin_catches_a_flipped_scale(monkeypatch):
    """The pin fails when the encoder multiplies by kv_scale instead of
    dividing, or the decoder divides (mistakes planted in the oracle)."""
    enc, dec = codec.fp8_encode_rows, codec.fp8_decode_rows
    monkeypatch.setattr(codec, "fp8_encode_rows", lambda l, r, kv=1.0: enc(l, r, 1.0 / kv))
    assert not _fp8_scaled_matches_torch(0.5, 7)
    monkeypatch.setattr(codec, "fp8_encode_rows", enc)
    monkeypatch.setattr(codec, "fp8_decode_rows", lambda rows, kv=1.0: dec(rows, 1.0 / kv))
    assert not _fp8_scaled_matches_torch(0.5, 7)
    monkeypatch.setattr(codec, "fp8_decode_rows", dec)
    assert _fp8_scaled_matches_torch(0.5, 7)


def test_staged_rows_definition():
    rng = np.random.default_rng(13)
    lat = _fp16(rng.standard_normal((40, 512)))
    rope = _fp16(rng.standard_normal((40, 64)))
    cache = codec.nvfp4_encode_rows(lat, rope)
    idx = np.array([[3, -1, 7, 39], [-1, -1, 0, 5]])
    rows, sidx = codec.staged_fp8_rows(cache, idx)
    assert sidx.tolist() == [[0, -1, 2, 3], [-1, -1, 6, 7]]
    assert not rows[1].any() and not rows[4].any()
    ld, rd = codec.nvfp4_decode_rows(cache[[3, 7, 39, 0, 5]])
    ref = torch.from_numpy(np.concatenate([ld, rd], 1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rows[[0, 2, 3, 6, 7]], ref)
    # rope values are already E4M3, so staging keeps them exactly
    assert np.array_equal(rows[[0, 2, 3, 6, 7], 512:], cache[[3, 7, 39, 0, 5], 288:])


# ---------------------------------------------------------------- two-level variant (R10)


def _wide_rows(rng, n, spread):
    lat = rng.standard_normal((n, 512)) * np.exp(spread * rng.standard_normal((n, 1)))
    return _fp16(lat), _fp16(rng.standard_normal((n, 64)))


def test_two_level_with_unit_scale_is_the_one_level_encoding():
    rng = np.random.default_rng(40)
    lat, rope = _wide_rows(rng, 64, 1.0)
    lat[0, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2)     # ties at scale 1
    assert np.array_equal(codec.nvfp4_encode_rows_2level(lat, rope, 1.0), codec.nvfp4_encode_rows(lat, rope))


@pytest.mark.parametrize("k", [-20, -7, -1, 3, 12])
def test_two_level_with_power_of_two_scale_encodes_the_scaled_values(k):
    """For g = 2^k every FP32 step is exact, so the bytes equal the one-level
    encoding of latent / g (an identity of the definitions)."""
    rng = np.random.default_rng(41 + k)
    lat, rope = _wide_rows(rng, 64, 1.5)
    g = 2.0 ** k
    assert np.array_equal(codec.nvfp4_encode_rows_2level(lat, rope, g), codec.nvfp4_encode_rows(lat / g, rope))


def test_two_level_codes_are_the_nearest_grid_points_in_exact_arithmetic():
    """Away from the few values within an FP32 rounding of a decision boundary,
    scale and codes are the exact round-to-nearest-even choices for an
    arbitrary g, checked with rationals."""
    rng = np.random.default_rng(42)
    lat, rope = _wide_rows(rng, 12, 1.0)
    g = float(np.float32(0.0371))
    rows = codec.nvfp4_encode_rows_2level(lat, rope, g)
    lv, _ = codec.nvfp4_decode_rows(rows)
    gf = Fr(g)
    grid = [Fr(v) for v in codec.E2M1_GRID]
    e4 = [Fr(float(v)) for v in codec.E4M3_POS]
    checked = 0
    for r in range(lat.shape[0]):
        for gi in range(32):
            x = [Fr(float(v)) for v in lat[r, 16 * gi:16 * gi + 16]]
            q = max(abs(v) for v in x) / (6 * gf)
            # nearest E4M3 to the exact quotient; skip groups near a midpoint
            dist = sorted((abs(q - v), i) for i, v in enumerate(e4))
            if dist[1][0] - dist[0][0] <= q * Fr(2, 2 ** 23):
                continue
            s = e4[dist[0][1]]
            assert Fr(float(codec.e4m3_decode(rows[r, 256 + gi]))) == s
            for j, v in enumerate(x):
                cand = sorted((abs(abs(v) - c * s * gf), k) for k, c in enumerate(grid))
                if s == 0 or cand[1][0] - cand[0][0] <= abs(v) * Fr(2, 2 ** 23):
                    continue
                assert Fr(abs(float(lv[r, 16 * gi + j]))) == grid[cand[0][1]] * s
                checked += 1
    assert checked > 5000


def test_two_level_scale_extends_the_range():
    """Latents far past the one-level range (largest code x largest scale =
    2688) or far below it keep their E2M1 precision with g = amax / 2688,
    while the one-level encoding saturates or flushes them."""
    rng = np.random.default_rng(43)
    for factor in (1e4, 1e-6):
        lat = rng.standard_normal((8, 512)) * factor
        lat = lat.astype(np.float32).astype(np.float64)      # beyond fp16's range: float32 inputs
        rope = np.zeros((8, 64))
        g = float(np.float32(np.abs(lat).max() / 2688.0))
        two, _ = codec.nvfp4_decode_rows_2level(codec.nvfp4_encode_rows_2level(lat, rope, g), g)
        one, _ = codec.nvfp4_decode_rows(codec.nvfp4_encode_rows(lat, rope))
        gmax = np.abs(lat.reshape(8, 32, 16)).max(axis=2, keepdims=True)
        err2 = (np.abs(two - lat).reshape(8, 32, 16) / gmax).max()
        err1 = (np.abs(one - lat).reshape(8, 32, 16) / gmax).max()
        assert err2 <= 0.25 and err1 >= 0.9, (factor, err1, err2)
