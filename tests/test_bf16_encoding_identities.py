"""Host checks of the bf16 facts the 128-column tile quantizer relies on when
it works on the loaded bf16 pairs instead of fp32 values (exhaustive over the
finite bf16 patterns and the scale codes a finite block can have):

* finite bf16 magnitudes (the pattern with the sign bit cleared) order like
  16-bit unsigned integers, so a packed 16-bit max finds the block amax;
* the exponent field of the amax pattern gives the same E8M0 code as the
  fp32 rule X = floor(log2 amax) - 8, floored at -127;
* ((c + 8) << 7) | 0x60 is the bf16 pattern of 448 * 2^X (X = c - 127), so a
  packed 16-bit min of magnitudes against it clamps |v| to 448 * 2^X exactly.

The device side (the conversion instruction itself) is pinned by the GPU
quantizer tests, which compare every finite bf16 pattern with the oracle.
"""
import numpy as np


def _bf16_to_f64(patterns):
    return (patterns.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


MAGS = np.arange(0, 0x7F80, dtype=np.uint32)           # every finite magnitude pattern


def test_finite_magnitudes_order_like_integers():
    v = _bf16_to_f64(MAGS)
    assert np.all(np.diff(v) > 0)


def test_scale_code_from_the_exponent_field():
    v = _bf16_to_f64(MAGS)
    code = np.maximum((MAGS >> 7).astype(np.int64) - 8, 0)
    nz = v > 0
    _, e = np.frexp(v[nz])                              # v = f * 2^e, f in [0.5, 1)
    x = np.maximum(e - 1 - 8, -127)                     # floor(log2 v) - 8, floored
    assert np.array_equal(code[nz], x + 127)
    assert code[0] == 0                                 # an all-zero block: X = -127


def test_limit_pattern_is_448_times_the_scale():
    c = np.arange(0, 247, dtype=np.uint32)              # finite blocks: c <= 254 - 8
    lim = ((c + 8) << 7) | 0x60
    assert np.array_equal(_bf16_to_f64(lim), np.ldexp(448.0, c.astype(np.int64) - 127))


def test_integer_clamp_equals_float_clamp():
    # every magnitude against every limit pattern: min on patterns is the
    # pattern of min on values (both are monotone in the same order)
    c = np.arange(0, 247, dtype=np.uint32)
    lim = ((c + 8) << 7) | 0x60
    mags = MAGS[::7]
    clamped = np.minimum(mags[None, :], lim[:, None])
    ref = np.minimum(_bf16_to_f64(mags)[None, :], _bf16_to_f64(lim)[:, None])
    assert np.array_equal(_bf16_to_f64(clamped), ref)
