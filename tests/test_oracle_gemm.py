"""Pins of the oracle's grouped GEMM and token-axis quantizer: brute-force
loops, the identity grouped GEMM = per-expert loop, reduction to a plain GEMM
at E=1, and zero-token experts."""
import math

import numpy as np
import torch

from oracle import mx_oracle as O
from tests.test_oracle_codec import brute_force_e4m3


def triple_loop_grouped(A, B, offsets):
    M, K = A.shape
    E, N, _ = B.shape
    Y = np.zeros((M, N))
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            for j in range(N):
                acc = 0.0
                for k in range(K):
                    acc += A[i, k] * B[e, j, k]
                Y[i, j] = acc
    return Y


def test_grouped_linear_brute_force():
    rng = np.random.default_rng(10)
    offsets = np.array([0, 3, 3, 11, 17])         # expert 1 is empty
    A = rng.standard_normal((17, 32))
    B = rng.standard_normal((4, 5, 32))
    assert np.allclose(O.grouped_linear(A, B, offsets),
                       triple_loop_grouped(A, B, offsets), rtol=1e-12,
                       atol=1e-12)


def test_grouped_linear_single_expert_is_plain_gemm():
    rng = np.random.default_rng(11)
    A = rng.standard_normal((40, 64))
    B = rng.standard_normal((1, 24, 64))
    ref = (torch.from_numpy(A) @ torch.from_numpy(B[0]).T).numpy()
    assert np.allclose(O.grouped_linear(A, B, np.array([0, 40])), ref,
                       rtol=1e-12, atol=1e-12)


def test_zero_token_experts_do_not_shift_neighbours():
    rng = np.random.default_rng(12)
    A = rng.standard_normal((20, 32))
    B = rng.standard_normal((2, 7, 32))
    ref = O.grouped_linear(A, B, np.array([0, 12, 20]))
    Bz = np.stack([B[0], rng.standard_normal((7, 32)), B[1],
                   rng.standard_normal((7, 32))])
    got = O.grouped_linear(A, Bz, np.array([0, 12, 12, 20, 20]))
    assert np.array_equal(got, ref)


def test_grouped_linear_row_scale():
    rng = np.random.default_rng(13)
    A = rng.standard_normal((9, 32))
    B = rng.standard_normal((2, 3, 32))
    r = rng.uniform(0, 1, 9)
    off = np.array([0, 4, 9])
    assert np.allclose(O.grouped_linear(A, B, off, r),
                       O.grouped_linear(A, B, off) * r[:, None])


def brute_force_token_quant(v, offsets, align):
    """Pure-Python per-expert, per-column block quantization of the token
    axis into the padded transposed layout."""
    M, C = v.shape
    poff = [0]
    for e in range(len(offsets) - 1):
        n = offsets[e + 1] - offsets[e]
        poff.append(poff[-1] + (n + align - 1) // align * align)
    Mp = poff[-1]
    codes = np.zeros((C, Mp), np.uint8)
    scales = np.zeros((C, Mp // 32), np.uint8)
    for e in range(len(offsets) - 1):
        n = offsets[e + 1] - offsets[e]
        for c in range(C):
            for b in range((n + align - 1) // align * align // 32):
                rows = range(offsets[e] + 32 * b,
                             min(offsets[e] + 32 * b + 32, offsets[e + 1]))
                vals = [float(v[i, c]) for i in rows]
                amax = max([abs(x) for x in vals], default=0.0)
                if amax == 0:
                    X = -127
                else:
                    X = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
                col0 = poff[e] + 32 * b
                scales[c, col0 // 32] = X + 127
                for j, x in enumerate(vals):
                    codes[c, col0 + j] = brute_force_e4m3(math.ldexp(x, -X))
    return codes, scales, np.array(poff)


def test_quantize_tokens_brute_force_ragged():
    rng = np.random.default_rng(14)
    counts = [0, 1, 31, 32, 33, 0, 5]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    v = rng.standard_normal((offsets[-1], 64)) * np.exp(
        rng.uniform(-3, 3, (offsets[-1], 1)))
    for align in (32, 128):
        c, s, p = O.quantize_tokens(v, offsets, align)
        cb, sb, pb = brute_force_token_quant(v, offsets, align)
        assert np.array_equal(p, pb)
        assert np.array_equal(c, cb) and np.array_equal(s, sb)


def test_token_quant_equals_row_quant_of_expert_transpose():
    """With counts that are multiples of 32, the token-axis blocks of an
    expert are the row blocks of that expert's transposed slice."""
    rng = np.random.default_rng(15)
    offsets = np.array([0, 64, 64, 160])
    v = rng.standard_normal((160, 32))
    got = O.qdq_tokens(v, offsets, 128)
    for e in range(3):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            assert np.array_equal(got[lo:hi], O.qdq_lastdim(v[lo:hi].T).T)


def test_padded_offsets():
    assert O.padded_offsets([0, 0, 1, 129, 257], 128).tolist() == [
        0, 0, 128, 256, 384]
    assert O.padded_offsets([0, 0, 1, 129, 257], 32).tolist() == [
        0, 0, 32, 160, 288]
