"""Pins of oracle/fp8_tensor.py (per-tensor scaled FP8) against what does not
share its code: a brute-force nearest-value search over every E4M3 value with
fp32 rounding done by ``struct`` (the exact product or quotient rounded once,
which double rounding from float64 does not disturb for these operand
widths), exact power-of-two invariances, exact round trips of representable
tensors, the E4M3 half-spacing error bound, and loops for the grouped GEMM."""
import struct

import numpy as np
import pytest

from oracle import fp8_tensor as P
from oracle import mx_oracle as O


def f32(v):
    """Round a Python float (float64) to the nearest float32, ties to even."""
    return struct.unpack("f", struct.pack("f", v))[0]


def e4m3_table():
    """Value of every finite non-negative E4M3 code 0x00..0x7E."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m / 512.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


TABLE = e4m3_table()


def brute_code(v):
    """Nearest E4M3 value (ties to the even code), magnitude saturated at
    448, sign kept."""
    a = min(abs(v), 448.0)
    d = np.abs(TABLE - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if np.signbit(v) else 0)


def brute_quantize(x):
    flat = [float(v) for v in np.asarray(x, dtype=np.float64).reshape(-1)]
    amax = max([abs(v) for v in flat], default=0.0)
    if amax == 0.0:
        s = 1.0
    else:
        s = f32(448.0 / amax)
        if s == float("inf"):
            s = float(np.finfo(np.float32).max)
    codes = [brute_code(f32(v * s)) for v in flat]
    return np.array(codes, dtype=np.uint8).reshape(np.shape(x)), amax, f32(1.0 / s)


def bf16_values(rng, shape, scale=1.0):
    """float64 values that are exactly bfloat16 (top 16 bits of a float32)."""
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (v.view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("scale", [1.0, 3e-3, 250.0, 1e-30])
def test_codes_match_brute_force(scale):
    rng = np.random.default_rng(int(np.log2(scale) + 200))
    x = bf16_values(rng, (9, 40), scale)
    x[0, 0] = -0.0
    x[1, :4] = x[2, :4]                              # repeated values
    codes, amax, s_inv = P.quantize_tensor(x)
    bc, bamax, bsinv = brute_quantize(x)
    assert np.array_equal(codes, bc)
    assert float(amax) == bamax and float(s_inv) == bsinv


def test_largest_element_encodes_to_448():
    rng = np.random.default_rng(2)
    for _ in range(20):
        x = bf16_values(rng, (16, 16), rng.uniform(1e-3, 1e3))
        codes, amax, _ = P.quantize_tensor(x)
        top = np.abs(x) == float(amax)
        assert np.all((codes[top] & 0x7F) == 0x7E)  # 448, the largest finite code
        assert np.all((codes & 0x7F) <= 0x7E)       # never NaN


@pytest.mark.parametrize("k", [-20, -3, 1, 7])
def test_power_of_two_rescale_keeps_codes(k):
    rng = np.random.default_rng(5)
    x = bf16_values(rng, (12, 33))
    c0, a0, s0 = P.quantize_tensor(x)
    c1, a1, s1 = P.quantize_tensor(x * 2.0 ** k)
    assert np.array_equal(c0, c1)
    assert float(a1) == float(a0) * 2.0 ** k and float(s1) == float(s0) * 2.0 ** k


def test_zero_empty_and_tiny_tensors():
    c, a, s = P.quantize_tensor(np.zeros((4, 8)))
    assert np.all(c == 0) and a == 0 and s == 1
    x = np.zeros((6, 32))
    x[3:] = 1.5
    codes, amax, s_inv = P.quantize_groups(x, [0, 3, 3, 6])   # middle group empty
    assert amax.tolist() == [0.0, 0.0, 1.5] and s_inv[1] == 1 and s_inv[0] == 1
    assert np.all(codes[3:] == 0x7E)
    # amax so small that 448 / amax overflows fp32: the largest finite scale
    tiny = np.full((2, 2), 2.0 ** -130)
    c, a, s = P.quantize_tensor(tiny)
    assert float(s) == f32(1.0 / float(np.finfo(np.float32).max))
    assert np.all(c == brute_quantize(tiny)[0])


@pytest.mark.parametrize("k", [0, -5, 9])
def test_exact_round_trip_of_representable_tensors(k):
    """E4M3 values times 2^k whose largest magnitude is 448 * 2^k: the scale
    is 2^-k exactly and quantize-dequantize returns the tensor."""
    rng = np.random.default_rng(11 + k)
    codes = rng.integers(0, 0x7F, size=(20, 32)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[0, 0] = 0x7E
    x = O.e4m3_decode(codes) * 2.0 ** k
    c, _, s_inv = P.quantize_tensor(x)
    assert np.array_equal(P.dequantize(c, s_inv), x)


def test_error_within_half_spacing():
    """|deq - x| <= 2^-4 |x| where x * scale is an E4M3 normal (three
    mantissa bits: half a unit is 2^-4 of the value), and <= 2^-10 / scale in
    the subnormal range; the fp32 product adds at most 2^-24 relative."""
    rng = np.random.default_rng(13)
    v = (rng.standard_normal((64, 64)) * np.exp(rng.uniform(-6, 6, size=(64, 64))))
    x = (v.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
    c, amax, s_inv = P.quantize_tensor(x)
    deq = P.dequantize(c, s_inv)
    s = 1.0 / float(s_inv)
    normal = np.abs(x) * s >= 2.0 ** -6
    assert np.all(np.abs(deq - x)[normal] <= (2.0 ** -4 + 2.0 ** -22) * np.abs(x[normal]))
    assert np.all(np.abs(deq - x)[~normal] <= 2.0 ** -10 * float(s_inv) * 1.0001)


def test_grouped_gemm_matches_loops():
    rng = np.random.default_rng(17)
    offs = [0, 5, 5, 12, 20]                       # an empty expert
    M, K, N, E = 20, 8, 6, 4
    x = bf16_values(rng, (M, K))
    w = bf16_values(rng, (E, N, K), 0.02)
    r = rng.random(M)
    xc, _, xs = P.quantize_groups(x, offs)
    wc, _, ws = P.quantize_groups(w)
    got = P.grouped_linear_fp8(xc, xs, wc, ws, offs, r)
    ref = np.zeros((M, N))
    for e in range(E):
        for m in range(offs[e], offs[e + 1]):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += (O.e4m3_decode(xc[m, k]) * float(xs[e])) * (
                        O.e4m3_decode(wc[e, n, k]) * float(ws[e]))
                ref[m, n] = acc * r[m]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_grouped_gemm_equals_plain_gemm_on_representable_operands():
    """Operands that round-trip exactly: the FP8 grouped GEMM is the plain
    grouped GEMM of the original values."""
    rng = np.random.default_rng(19)
    offs = [0, 7, 16, 16, 30]
    K, N, E = 32, 16, 4
    xcodes = rng.integers(0, 0x7F, size=(30, K)).astype(np.uint8)
    xcodes[[0, 7, 16], 0] = 0x7E                   # amax 448 * 2^k in every group
    x = O.e4m3_decode(xcodes) * 2.0 ** -3
    wcodes = rng.integers(0, 0x7F, size=(E, N, K)).astype(np.uint8) | 0x80
    wcodes[:, 0, 0] = 0xFE
    w = O.e4m3_decode(wcodes) * 2.0 ** -12
    xc, _, xs = P.quantize_groups(x, offs)
    wc, _, ws = P.quantize_groups(w)
    assert np.allclose(P.grouped_linear_fp8(xc, xs, wc, ws, offs),
                       O.grouped_linear(x, w, offs), rtol=1e-13, atol=0)
