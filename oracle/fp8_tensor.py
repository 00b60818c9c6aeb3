"""FP64 CPU oracle for per-tensor scaled FP8 (E4M3) on the grouped GEMM.
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it imports nothing from the product path.

Source (cited by page title): "MoE-Training für biologische Grundmodelle
optimieren" (hyper.ai, German) -- the paragraph on activation memory names
plain FP8 beside MXFP8 as the 8-bit formats the recipe supports, without
saying how FP8 is scaled.  The E4M3 element codec is the one of
``oracle.mx_oracle`` (OCP E4M3 "FN": RNE, saturating at +-448).

Readings (the page gives no recipe; also listed in the design notes of the
repository):

* R-pt-tensor  "per tensor" on a grouped operand: every expert's slice is one
               tensor -- rows [o_e, o_{e+1}) of the token-sorted activations,
               matrix e of the stacked weights -- with its own scale.
* R-pt-scale   scale = 448 / amax, amax = max |x| over the tensor, the
               quotient computed in fp32 (one IEEE rounding); amax = 0 gives
               scale 1; a quotient past the largest finite fp32 gives that
               largest value.  scale_inv = 1 / scale in fp32.
* R-pt-code    code = E4M3 (RNE, saturating) of the fp32 product x * scale:
               the product is rounded to fp32 first, so the device, which
               multiplies in fp32, takes the same decision.
* R-pt-gemm    dequantized value = decode(code) * scale_inv; the grouped GEMM
               of two such operands is (decoded codes of X_e) (decoded codes of
               W_e)^T * scale_inv_x[e] * scale_inv_w[e] (* the row's routing
               weight), accumulated in float64 here.

Functions with no independent pin: none (see tests/test_oracle_fp8_tensor.py).
"""
from __future__ import annotations

import numpy as np

from oracle.mx_oracle import E4M3_MAX, e4m3_decode, e4m3_encode

F32 = np.float32
F32_MAX = float(np.finfo(np.float32).max)


def tensor_scale(amax):
    """(scale, scale_inv) of one tensor from its amax (R-pt-scale), as
    float32 numbers."""
    amax = F32(amax)
    if amax == 0:
        return F32(1.0), F32(1.0)
    with np.errstate(over="ignore"):
        s = F32(E4M3_MAX) / amax
    if not np.isfinite(s):
        s = F32(F32_MAX)
    return s, F32(1.0) / s


def encode(x, scale):
    """E4M3 codes of x * scale, the product rounded to fp32 first (R-pt-code).
    x: values representable in float32 (bf16 in practice); scale: float32."""
    prod = np.asarray(x, dtype=np.float32) * F32(scale)     # one fp32 rounding
    return e4m3_encode(prod.astype(np.float64))


def quantize_tensor(x):
    """Codes of one tensor plus its amax and scale_inv (R-pt-scale,
    R-pt-code)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = F32(np.max(np.abs(x32))) if x32.size else F32(0.0)
    s, s_inv = tensor_scale(amax)
    return encode(x32, s), amax, s_inv


def quantize_groups(x, offsets=None):
    """Per-tensor FP8 copy of a grouped operand (R-pt-tensor).

    x [M, C] with row groups ``offsets`` [G+1], or x [G, R, C] (one tensor
    per matrix) when ``offsets`` is None.  Returns codes uint8 (the shape of
    x), amax float32 [G] and scale_inv float32 [G].
    """
    x = np.asarray(x)
    if offsets is None:
        parts = [x[g] for g in range(x.shape[0])]
    else:
        parts = [x[offsets[g]:offsets[g + 1]] for g in range(len(offsets) - 1)]
    codes, amax, s_inv = [], [], []
    for p in parts:
        c, a, si = quantize_tensor(p)
        codes.append(c)
        amax.append(a)
        s_inv.append(si)
    out = np.stack(codes) if offsets is None else (
        np.concatenate(codes) if codes else np.zeros((0, x.shape[1]), np.uint8))
    return out, np.array(amax, dtype=np.float32), np.array(s_inv, dtype=np.float32)


def dequantize(codes, scale_inv):
    """decode(code) * scale_inv, float64."""
    return e4m3_decode(codes) * np.float64(scale_inv)


def grouped_linear_fp8(xc, x_sinv, wc, w_sinv, offsets, row_scale=None):
    """Y[o_e:o_{e+1}] = decode(xc_e) decode(wc[e])^T * x_sinv[e] * w_sinv[e]
    (* row_scale) for every expert e (R-pt-gemm), float64."""
    M = xc.shape[0]
    N = wc.shape[1]
    Y = np.zeros((M, N))
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            Y[lo:hi] = (e4m3_decode(xc[lo:hi]) @ e4m3_decode(wc[e]).T) * (
                np.float64(x_sinv[e]) * np.float64(w_sinv[e]))
    if row_scale is not None:
        Y *= np.asarray(row_scale, dtype=np.float64)[:, None]
    return Y
