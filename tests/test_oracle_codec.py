"""Pins of the oracle's MXFP8 codec against things other than itself:
torch's independent float8 casts, hand-derived closed forms, a brute-force
nearest-value search, and the scale invariant of the OCP MX rule."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_finite_bf16_as_f64():
    bits = np.arange(1 << 16, dtype=np.uint32)
    f32 = (bits << 16).view(np.float32)
    f32 = f32[np.isfinite(f32)]
    return f32.astype(np.float64)


def torch_e4m3_codes(v64):
    """torch's RNE cast to float8_e4m3fn, after clamping to +-448 (the cast
    maps values past 464 to NaN instead of saturating)."""
    v32 = np.clip(v64, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(v32).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


@pytest.mark.parametrize("X", [-127, -20, -1, 0, 1, 20, 119])
def test_e4m3_encode_matches_torch_exhaustive_bf16(X):
    v = np.ldexp(all_finite_bf16_as_f64(), -X)
    # values below 2^-126 are not exact in float32, but they are far below
    # half the smallest E4M3 subnormal, so both sides give a signed zero
    ours = O.e4m3_encode(v)
    ref = torch_e4m3_codes(v)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    assert np.nanmax(ours) == 448.0


def _parse_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, code = line.split()[:2]
            rows.append((float(v), int(code, 16)))
    return rows


def test_e4m3_closed_forms_golden():
    rows = _parse_golden("e4m3_closed_forms.txt")
    assert len(rows) >= 15
    for v, code in rows:
        assert int(O.e4m3_encode(np.array([v]))[0]) == code, (v, hex(code))


def _positive_e4m3_table():
    """(code, value) of the 127 finite non-negative E4M3 codes, built from
    the bit fields directly (1.m * 2^(e-7), or m/8 * 2^-6 when e == 0)."""
    out = []
    for c in range(127):                      # 0x7F is NaN
        e, m = c >> 3, c & 7
        out.append((c, math.ldexp(m / 8.0, -6) if e == 0
                    else math.ldexp(1.0 + m / 8.0, e - 7)))
    return out


_E4M3_TABLE = _positive_e4m3_table()


def brute_force_e4m3(v):
    """Nearest finite E4M3 value to clamp(v, +-448), ties to the code with an
    even mantissa, sign kept: a search over all finite codes."""
    a = min(abs(v), 448.0)
    best = None
    for c, x in _E4M3_TABLE:
        d = abs(x - a)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_encode_brute_force_random():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(400) * 50,
                        rng.standard_normal(200) * 0.01,
                        rng.uniform(440, 520, 50), -rng.uniform(0, 2e-3, 50)])
    ours = O.e4m3_encode(v)
    for x, c in zip(v, ours):
        assert int(c) == brute_force_e4m3(float(x)), x


def test_scale_rule_invariant_and_e8m0():
    vals = np.abs(all_finite_bf16_as_f64())
    vals = vals[vals > 0]
    X = O.block_scale_exponent(vals)
    unclamped = (X > -127) & (X < 127)
    lo = 256.0 * np.ldexp(1.0, X)
    hi = 512.0 * np.ldexp(1.0, X)
    assert np.all(lo[unclamped] <= vals[unclamped])
    assert np.all(vals[unclamped] < hi[unclamped])
    # clamped only at the bottom for finite bf16; max exponent is 127-8=119
    assert X.max() == 119 and np.all(X[~unclamped] == -127)
    assert O.block_scale_exponent(np.array([0.0]))[0] == -127
    # E8M0 decode vs torch on every code
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(
        torch.float64).numpy()
    assert np.array_equal(O.e8m0_decode(codes), ref)
    assert np.isnan(O.e8m0_decode(np.array([255]))[0])


def test_scaled_values_fit_e4m3_range():
    """After scaling by 2^-X the block max sits in [256, 512): only the top
    of that range saturates."""
    rng = np.random.default_rng(2)
    blk = rng.standard_normal((1000, 32)) * np.exp(rng.uniform(-30, 30, (1000, 1)))
    codes, scales = O.quantize_lastdim(blk)
    X = scales[:, 0].astype(np.int64) - 127
    m = np.abs(blk).max(axis=1) * np.ldexp(1.0, -X)
    assert np.all((m >= 256) & (m < 512))


def brute_force_quantize_rows(v):
    """Pure-Python block quantization of a small 2-D array along rows."""
    R, C = v.shape
    codes = np.zeros((R, C), np.uint8)
    scales = np.zeros((R, C // 32), np.uint8)
    for i in range(R):
        for b in range(C // 32):
            blk = [float(x) for x in v[i, 32 * b:32 * b + 32]]
            amax = max(abs(x) for x in blk)
            if amax == 0:
                X = -127
            else:
                m, e = math.frexp(amax)
                X = max(-127, min(127, e - 1 - 8))
            scales[i, b] = X + 127
            for j, x in enumerate(blk):
                codes[i, 32 * b + j] = brute_force_e4m3(math.ldexp(x, -X))
    return codes, scales


def test_quantize_lastdim_brute_force():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 96))
    v[1] *= 1e-3
    v[2, 32:64] = 0.0                       # all-zero block
    v[3, 5] = 1e4                           # outlier block
    v[4, 70] = -0.0
    c, s = O.quantize_lastdim(v)
    cb, sb = brute_force_quantize_rows(v)
    assert np.array_equal(c, cb) and np.array_equal(s, sb)
    assert s[2, 1] == 0 and not c[2, 32:64].any()


def exact_block_values(rng, shape, glo=-20, ghi=20):
    """Values of the form m * 2^g with |m| in {1, 1.25, 1.5, 1.75, 0.5} and
    one exponent g per block of 32 along the last axis: every such block is
    MXFP8-representable.  The first value of each block is 1.75 * 2^g."""
    m = rng.choice([1.0, 1.25, 1.5, 1.75, 0.5, -1.0, -1.25, -1.75], shape)
    m[..., ::32] = 1.75
    nb = shape[-1] // 32
    g = rng.integers(glo, ghi, shape[:-1] + (nb,))
    g = np.repeat(g, 32, axis=-1)
    return m * np.ldexp(1.0, g)


def test_round_trip_exact_for_representable_blocks():
    rng = np.random.default_rng(4)
    v = exact_block_values(rng, (64, 128))
    assert np.array_equal(O.qdq_lastdim(v), v)


def test_round_trip_saturation_closed_form():
    # block max with significand 1.875 is not representable at scale 2^(e-8):
    # 240 -> X = floor(log2 240) - 8 = -1 -> 480 saturates to 448 -> 224
    blk = np.zeros((1, 32))
    blk[0, 0] = 240.0
    assert O.qdq_lastdim(blk)[0, 0] == 224.0
    blk[0, 0] = 511.9                       # X = 0, 511.9 -> 448
    assert O.qdq_lastdim(blk)[0, 0] == 448.0


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(5)
    v32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal
        np.array([3.3e38, -3.39e38, 1e-45], np.float32)])
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    ours = O.round_bf16(v32.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_table_dequantization_of_the_full_size_tests():
    """The full-size GPU tests dequantize with a 256-entry table of the
    oracle's decode; it equals the oracle's dequantization."""
    from tests.test_gpu_full_size import deq
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (7, 96)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0                  # no NaN codes
    scales = rng.integers(0, 255, (7, 3)).astype(np.uint8)
    assert np.array_equal(deq(codes, scales), O.dequantize_lastdim(codes, scales))
