"""Oracle codec: E2M1, E4M3, the 352-byte NVFP4 MLA row, the 576-byte FP8 row.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the
product path may import this module.

What the pages fix (Prime Inference write-up, section "Making room for
low-latency decode"; the mo.ai.kr article, KV-cache section; the
wireai.ir article, 4-bit-caches section):

* the MLA latent has 512 values, stored at four bits each, with one FP8
  scale for every group of 16 values;
* the 64 positional (rope) values stay FP8;
* with the scales included a row shrinks from 576 bytes to 352 bytes
  (256 B of nibbles + 32 B of scales + 64 B of rope).

Readings taken where the pages are silent:

* R1  The four-bit element is E2M1 (sign, 2 exponent bits with bias 1,
      1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; no Inf/NaN),
      which is what "NVFP4" denotes.
* R2  The FP8 type is OCP E4M3FN (bias 7, max 448, 0x7F/0xFF NaN, no Inf).
* R3  Encoders round to nearest, ties to the even code, and saturate to
      the largest finite value; the sign bit always copies the input's
      sign bit (so -0.0 and small negatives that round to zero keep it).
* R4  Group scale s = E4M3(amax / 6) computed on the exact real quotient;
      there is no second-level per-tensor scale.
* R5  Elements are coded against the *rounded* scale: code = E2M1(x / s).
      When s rounds to zero every magnitude is 0.
* R6  Row layout: bytes [0,256) hold the latent nibbles, element 2i in the
      low nibble of byte i and element 2i+1 in the high nibble; bytes
      [256,288) hold the 32 group scales in group order; bytes [288,352)
      hold the 64 rope values in order.
* R7  The rope part is cast to E4M3 directly, with no scale.
* R8  The FP8 comparison row stores E4M3(v / kv_scale) for all 512 + 64
      values (latent first), decoded as code * kv_scale.
* R10 Two-level variant (the NVFP4 format's second, per-tensor scale; the
      pages name only the per-16 FP8 scale): a positive FP32 global scale g
      multiplies every decoded latent value, code * s * g; the rope is not
      scaled.  With g arbitrary the exact quotient amax / (6 g) and the
      code thresholds t * s * g are no longer all FP32 values, so the
      encoding is defined by the FP32 steps that make its decisions:
        d   = fl32(6 * g)
        s   = E4M3 of fl32(amax / d), round to nearest even, saturating
        thr = fl32(t * s * g) for t in .25, .75, 1.25, 1.75, 2.5, 3.5, 5
              (t * s is exact; one rounding)
        magnitude = number of thresholds passed, |x| > thr for t in
              .25, 1.25, 2.5, 5 and |x| >= thr for t in .75, 1.75, 3.5
              (ties to the even code, as in R5), 0 when s = 0.
      With g = 1 every step is exact and this is R4 and R5 exactly.

All arithmetic is FP64 on values that FP64 holds exactly: every fp16 /
bf16 input, every grid point g * s (at most 7 significant bits) and every
difference between them (well under 53 bits apart), so each rounding
decision below is exact.
"""

from __future__ import annotations

import numpy as np

LATENT_DIM = 512
ROPE_DIM = 64
GROUP = 16
N_GROUPS = LATENT_DIM // GROUP          # 32
NIBBLE_BYTES = LATENT_DIM // 2          # 256
SCALE_OFF = NIBBLE_BYTES                # 256
ROPE_OFF = SCALE_OFF + N_GROUPS         # 288
ROW_BYTES = ROPE_OFF + ROPE_DIM         # 352
FP8_ROW_BYTES = LATENT_DIM + ROPE_DIM   # 576

# --------------------------------------------------------------------------
# E2M1 (R1)
# --------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its bit fields (R1).

    bit 3 = sign, bits 2..1 = exponent e (bias 1), bit 0 = mantissa m.
    e == 0 is subnormal: m * 0.5.  Otherwise 2**(e-1) * (1 + m/2).
    """
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
# non-negative grid, indexed by the 3-bit magnitude code
E2M1_GRID = E2M1_TABLE[:8].copy()


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64) & 0xF]


# --------------------------------------------------------------------------
# E4M3 (R2)
# --------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3FN byte from its bit fields (R2).

    bit 7 = sign, bits 6..3 = exponent e (bias 7), bits 2..0 = mantissa m.
    e == 0 is subnormal: (m/8) * 2**-6.  e == 15 with m == 7 is NaN.
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
# the 127 non-negative finite values, ascending, indexed by their code 0..126
E4M3_POS = E4M3_TABLE[:127].copy()


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def _nearest_even(a: np.ndarray, grid: np.ndarray, weight: float = 1.0) -> np.ndarray:
    """Index k of the grid point nearest to a/weight, ties to even k, saturating.

    ``grid`` is ascending and non-negative; ``a`` is non-negative.  The
    comparison is done as |a - weight*grid[k]|, which is exact in FP64 for
    every input this module sees, so ties are detected exactly.  Values
    beyond the last grid point pick the last point (saturation).
    """
    a = np.asarray(a, dtype=np.float64)
    g = grid * weight                              # exact: <= 7 significant bits
    hi = np.searchsorted(g, a, side="left")        # first g[hi] >= a
    hi = np.clip(hi, 0, len(g) - 1)
    lo = np.clip(hi - 1, 0, len(g) - 1)
    d_lo = np.abs(a - g[lo])
    d_hi = np.abs(g[hi] - a)
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    return np.where(pick_hi, hi, lo).astype(np.int64)


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN byte for each finite FP64 value: RNE, satfinite, sign kept (R2, R3)."""
    x = np.asarray(x, dtype=np.float64)
    k = _nearest_even(np.abs(x), E4M3_POS)
    sign = np.signbit(x).astype(np.int64) << 7
    return (sign | k).astype(np.uint8)


def e4m3_encode_quotient(a, divisor: float) -> np.ndarray:
    """E4M3 byte of the exact real quotient a/divisor for a >= 0 (R4).

    Compares a against divisor * v_k, which FP64 holds exactly for the
    divisor 6 used by the group scale, so no rounding of a/divisor ever
    enters the decision.
    """
    a = np.asarray(a, dtype=np.float64)
    return _nearest_even(a, E4M3_POS, weight=float(divisor)).astype(np.uint8)


# --------------------------------------------------------------------------
# NVFP4 group quantisation (R4, R5) and the 352-byte row (R6, R7)
# --------------------------------------------------------------------------


def nvfp4_group_scales(latent: np.ndarray) -> np.ndarray:
    """E4M3 scale byte per group of 16: E4M3(amax/6) on the exact quotient (R4).

    latent: [N, 512] values exactly representable in FP64 (fp16 / bf16 inputs).
    returns uint8 [N, 32].
    """
    lat = np.asarray(latent, dtype=np.float64).reshape(-1, N_GROUPS, GROUP)
    amax = np.abs(lat).max(axis=2)
    return e4m3_encode_quotient(amax, 6.0).reshape(-1, N_GROUPS)


def e2m1_encode(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """4-bit code of x against the decoded scale s: RNE of x/s on the E2M1 grid (R3, R5).

    x and s broadcast against each other; s >= 0.  The nearest grid point is
    found by comparing |x| with g_k * s exactly; ties take the even code,
    values past 6*s saturate to 6, and s == 0 gives magnitude 0.  The sign
    bit copies the sign bit of x.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    ax = np.abs(x)
    d = np.abs(ax[..., None] - E2M1_GRID * s[..., None])       # exact differences
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    # among the nearest points prefer an even magnitude code
    even = cand & ((np.arange(8) % 2) == 0)
    mag = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    mag = np.where(s == 0.0, 0, mag)
    sign = np.signbit(x).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def nvfp4_encode_rows(latent, rope) -> np.ndarray:
    """Encode rows into 352-byte NVFP4 MLA cache rows (R1-R7).

    latent: [N, 512], rope: [N, 64]; both hold fp16/bf16 values (any float
    array whose values FP64 represents exactly).  Returns uint8 [N, 352].
    """
    lat = np.asarray(latent, dtype=np.float64).reshape(-1, LATENT_DIM)
    rp = np.asarray(rope, dtype=np.float64).reshape(-1, ROPE_DIM)
    n = lat.shape[0]
    scale_codes = nvfp4_group_scales(lat)                         # [N, 32]
    s = e4m3_decode(scale_codes)                                  # decoded scales
    codes = e2m1_encode(lat.reshape(n, N_GROUPS, GROUP), s[:, :, None]).reshape(n, LATENT_DIM)
    codes = codes.astype(np.uint16)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)   # [N, 256]
    out = np.empty((n, ROW_BYTES), dtype=np.uint8)
    out[:, :SCALE_OFF] = packed
    out[:, SCALE_OFF:ROPE_OFF] = scale_codes
    out[:, ROPE_OFF:] = e4m3_encode(rp)
    return out


# E2M1 thresholds between magnitude codes k and k+1, and whether reaching
# the threshold itself moves up (ties go to the even code k+1)
E2M1_THRESHOLDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
E2M1_TIE_UP = (False, True, False, True, False, True, False)


def nvfp4_encode_rows_2level(latent, rope, global_scale: float) -> np.ndarray:
    """352-byte rows of the two-level variant (R10): the group scales and codes
    of latent / g, decided by the FP32 steps R10 lists; rope as in R7.

    latent: [N, 512], rope: [N, 64] fp16/bf16 values; global_scale: g > 0,
    taken as the float32 value the caller passes.
    """
    lat = np.asarray(latent, dtype=np.float64).reshape(-1, LATENT_DIM)
    rp = np.asarray(rope, dtype=np.float64).reshape(-1, ROPE_DIM)
    n = lat.shape[0]
    g32 = np.float32(global_scale)
    d = np.float32(6.0) * g32                                     # fl32(6 g)
    grp = lat.reshape(n, N_GROUPS, GROUP)
    amax = np.abs(grp).max(axis=2).astype(np.float32)             # exact (fp16/bf16 inputs)
    q = (amax / d).astype(np.float64)                             # fl32(amax / d), held exactly
    scale_codes = e4m3_encode(q)                                  # RNE, saturating (R3)
    sv = e4m3_decode(scale_codes)[:, :, None]                     # [N, 32, 1]
    ax = np.abs(grp)
    mag = np.zeros(grp.shape, dtype=np.int64)
    for t, up in zip(E2M1_THRESHOLDS, E2M1_TIE_UP):
        thr = (t * sv * np.float64(g32)).astype(np.float32).astype(np.float64)   # exact product, one rounding
        mag += (ax >= thr) if up else (ax > thr)
    mag = np.where(sv == 0.0, 0, mag)
    codes = (mag | (np.signbit(grp).astype(np.int64) << 3)).reshape(n, LATENT_DIM).astype(np.uint16)
    out = np.empty((n, ROW_BYTES), dtype=np.uint8)
    out[:, :SCALE_OFF] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    out[:, SCALE_OFF:ROPE_OFF] = scale_codes
    out[:, ROPE_OFF:] = e4m3_encode(rp)
    return out


def nvfp4_decode_rows_2level(rows, global_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Decoded (latent * g, rope) of two-level rows (R10)."""
    lat, rope = nvfp4_decode_rows(rows)
    return lat * float(np.float32(global_scale)), rope


def nvfp4_decode_rows(rows) -> tuple[np.ndarray, np.ndarray]:
    """Decode 352-byte rows to (latent [N,512], rope [N,64]) in FP64 (R6).

    latent element j of group g is E2M1(code_j) * E4M3(scale_g).
    """
    r = np.asarray(rows, dtype=np.uint8).reshape(-1, ROW_BYTES)
    n = r.shape[0]
    nib = r[:, :SCALE_OFF].astype(np.int64)
    codes = np.empty((n, LATENT_DIM), dtype=np.int64)
    codes[:, 0::2] = nib & 0xF
    codes[:, 1::2] = nib >> 4
    scales = e4m3_decode(r[:, SCALE_OFF:ROPE_OFF])                # [N, 32]
    lat = e2m1_decode(codes).reshape(n, N_GROUPS, GROUP) * scales[:, :, None]
    rope = e4m3_decode(r[:, ROPE_OFF:])
    return lat.reshape(n, LATENT_DIM), rope


# --------------------------------------------------------------------------
# FP8-576 comparison row (R8) and the staged FP8 re-encoding
# --------------------------------------------------------------------------


def fp8_encode_rows(latent, rope, kv_scale: float = 1.0) -> np.ndarray:
    """576-byte FP8 rows: E4M3(v / kv_scale) for latent then rope (R8)."""
    lat = np.asarray(latent, dtype=np.float64).reshape(-1, LATENT_DIM)
    rp = np.asarray(rope, dtype=np.float64).reshape(-1, ROPE_DIM)
    v = np.concatenate([lat, rp], axis=1)
    if kv_scale == 1.0:
        return e4m3_encode(v)
    # an exact quotient decision for a general scale: compare v with kv_scale * grid
    k = _nearest_even(np.abs(v), E4M3_POS, weight=float(kv_scale))
    sign = np.signbit(v).astype(np.int64) << 7
    return (sign | k).astype(np.uint8)


def fp8_decode_rows(rows, kv_scale: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    r = np.asarray(rows, dtype=np.uint8).reshape(-1, FP8_ROW_BYTES)
    v = e4m3_decode(r) * float(kv_scale)
    return v[:, :LATENT_DIM], v[:, LATENT_DIM:]


def staged_fp8_rows(cache_rows, indices, fp8_scale: float = 1.0):
    """The staged comparator's first step: selected NVFP4 rows re-encoded as FP8 rows.

    For token t and slot j with indices[t, j] >= 0 the NVFP4 row is decoded
    exactly and re-encoded as a 576-byte FP8 row with scale ``fp8_scale``;
    masked slots become zero rows.  Returns (rows [T*K, 576] uint8,
    staged_indices [T, K] int32) where staged_indices[t, j] = t*K + j for a
    valid slot and -1 for a masked one.  (The pages describe this path as an
    unpack into an FP8 temporary buffer ahead of the older FP8 attention
    kernel; reading R9: only the selected rows are converted, per step.)
    """
    idx = np.asarray(indices, dtype=np.int64)
    t_count, k = idx.shape
    out = np.zeros((t_count * k, FP8_ROW_BYTES), dtype=np.uint8)
    sidx = np.full((t_count, k), -1, dtype=np.int32)
    flat = idx.reshape(-1)
    valid = flat >= 0
    if valid.any():
        lat, rope = nvfp4_decode_rows(np.asarray(cache_rows)[flat[valid]])
        out[valid] = fp8_encode_rows(lat, rope, fp8_scale)
        pos = np.nonzero(valid)[0]
        sidx.reshape(-1)[pos] = pos.astype(np.int32)
    return out, sidx
