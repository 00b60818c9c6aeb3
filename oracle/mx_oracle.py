"""FP64 CPU oracle for the MXFP8 MoE expert path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it imports nothing from
the product path.

What it models (sources: three news rewrites of one tutorial on MoE training of
biological foundation models, cited by page title):

* "MoE-Training für biologische Grundmodelle optimieren" (hyper.ai, German;
  the paragraphs on GroupedLinear, on MXFP8 and on the GroupedMLP fusion
  kernel);
* "NVIDIA apresenta técnicas para tornar mais eficiente o treinamento de
  modelos biológicos baseados em arquitetura MoE" (conexaotc, Portuguese;
  third paragraph: GroupedLinear, MXFP8, GroupedMLP = quantization + SwiGLU +
  routing-weight scaling);
* "NVIDIA optimise l'entraînement MoE des modèles biologiques" (hyper.ai,
  French; the three improvements).

The pages say: every expert's linear runs in one grouped call driven by
per-expert token counts; values are stored in 8 bits with one scale per block
of 32 values; the MLP fuses the gate-up projection, a SwiGLU activation scaled
by the routing weight, and the quantization, forward and backward.  They give
no formula.  The element/scale encoding fixed here is the OCP Microscaling
(MX) v1.0 MXFP8 format: E4M3 (OCP "FN" variant, max 448) elements and an E8M0
power-of-two scale per 32 values, scale exponent floor(log2(amax)) - 8
(8 = exponent of the largest E4M3 normal), round-to-nearest-even, saturating.

Every function works in float64 and is written for reading, not speed.  The
only library primitives used as steps are ``numpy.frexp`` / ``ldexp`` /
``rint`` (exact), ``numpy.exp`` and ``numpy.matmul``.

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):

* R-amax0   a block whose amax is 0 gets scale code 0x00 (2^-127), codes 0.
* R-sign    negative values that round to zero keep the sign (code 0x80).
* R-tokpad  token-axis (columnwise) blocks restart at each expert's first row;
            every expert's token range is padded with zeros to a multiple of
            ``align`` tokens (128 in the library) in the transposed copy.
* R-swiglu  W1 rows [0, F) are the gate, rows [F, 2F) the up projection;
            s = silu(gate) * up, z = r * s, then z is quantized and fed to the
            down projection.
* R-recomp  the backward uses the gate-up pre-activation h exactly as the
            forward computed it (float64 here): the fused kernel keeps h on
            chip and the backward recomputes it from the same quantized
            operands instead of reading a stored copy (the pages: the fused
            GroupedMLP does not hold intermediate results in memory).
* R-save    an alternative mode, ``h_bf16=True``: the forward stores h rounded
            once to bfloat16 (RNE) and the backward reads that copy, so the
            SwiGLU backward sees bf16(h); h is never requantized.
* R-ste     the backward is straight-through: each GEMM quantizes its own two
            operands along its own contraction axis.
* R-out     Y, dX, dW1, dW2 are the FP64 results; callers compare them with the
            device's bfloat16 outputs within tolerance.

Functions with no independent pin: none (see tests/test_oracle_*.py).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32            # values per shared scale (MXFP8)
E4M3_MAX = 448.0      # largest finite OCP E4M3 value, 1.75 * 2^8
E4M3_EMAX = 8         # exponent of E4M3_MAX
E8M0_BIAS = 127


# --------------------------------------------------------------------------
# Element codec: OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
# bits; no infinities; S.1111.111 is NaN; max normal 448; min normal 2^-6;
# min subnormal 2^-9).
# --------------------------------------------------------------------------

def floor_log2(a):
    """floor(log2(a)) for finite a > 0, exactly (frexp, never log2)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def e4m3_encode(v):
    """Round float64 values to OCP E4M3 codes, RNE, saturating at +-448.

    Saturation is applied to the magnitude before rounding; because 448 is
    the largest code and (448, 464] rounds to 448 under RNE while anything
    above would round past it, this equals round-then-saturate.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.zeros(v.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    # subnormal grid: integer multiples of 2^-9; k = 8 lands on 0x08 = 2^-6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    nrm = ~sub
    e = floor_log2(a[nrm])
    m = np.rint(np.ldexp(a[nrm], -(e - 3)))      # significand * 8, in [8, 16]
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m).astype(np.int64)
    code[nrm] = ((e + 7) << 3) | (m - 8)

    code |= np.signbit(v).astype(np.int64) << 7
    return code.astype(np.uint8)


def e4m3_decode(codes):
    """Exact float64 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    sgn = (c >> 7) & 1
    exp = (c >> 3) & 15
    man = c & 7
    val = np.where(exp == 0,
                   man * 2.0 ** -9,                       # subnormal
                   (8 + man) * np.ldexp(1.0, exp - 10))   # (1 + m/8) 2^(e-7)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return np.where(sgn == 1, -val, val)


# --------------------------------------------------------------------------
# Scale codec: E8M0, code c in [0, 254] means 2^(c - 127); 255 is NaN.
# --------------------------------------------------------------------------

def e8m0_decode(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - E8M0_BIAS))


def block_scale_exponent(amax):
    """Shared exponent X of a block: floor(log2 amax) - 8, clamped to
    [-127, 127]; X = -127 for an all-zero block (reading R-amax0)."""
    amax = np.asarray(amax, dtype=np.float64)
    X = np.full(amax.shape, -E8M0_BIAS, dtype=np.int64)
    nz = amax > 0
    X[nz] = np.clip(floor_log2(amax[nz]) - E4M3_EMAX, -127, 127)
    return X


# --------------------------------------------------------------------------
# Block quantization along the last axis.
# --------------------------------------------------------------------------

def quantize_lastdim(v):
    """MXFP8-quantize ``v[..., C]`` in blocks of 32 along the last axis.

    Returns (codes uint8 [..., C], scale codes uint8 [..., C/32]).
    For each block: amax = max |v|, X = block_scale_exponent(amax),
    codes = E4M3(v * 2^-X) (the product is exact in float64).
    """
    v = np.asarray(v, dtype=np.float64)
    C = v.shape[-1]
    if C % BLOCK:
        raise ValueError("last dimension must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (C // BLOCK, BLOCK))
    X = block_scale_exponent(np.abs(blk).max(axis=-1))
    codes = e4m3_encode(blk * np.ldexp(1.0, -X)[..., None])
    return codes.reshape(v.shape), (X + E8M0_BIAS).astype(np.uint8)


def dequantize_lastdim(codes, scales):
    """Inverse of quantize_lastdim: decode(code) * 2^(scale - 127)."""
    codes = np.asarray(codes)
    C = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (C // BLOCK, BLOCK))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def qdq_lastdim(v):
    """Quantize then dequantize along the last axis."""
    return dequantize_lastdim(*quantize_lastdim(v))


# --------------------------------------------------------------------------
# Token-axis (columnwise) quantization with expert groups (reading R-tokpad).
# --------------------------------------------------------------------------

def padded_offsets(offsets, align=128):
    """Start of each expert's token range in the padded, transposed copy."""
    offsets = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(offsets)
    padded = (counts + align - 1) // align * align
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)


def quantize_tokens(v, offsets, align=128):
    """Quantize ``v[M, C]`` in blocks of 32 consecutive rows of one expert.

    Returns (codesT uint8 [C, Mpad], scalesT uint8 [C, Mpad/32], poff) where
    expert e's rows [o_e, o_e + n_e) sit at columns [poff_e, poff_e + n_e) of
    the transposed copy and columns up to poff_{e+1} hold zeros.
    """
    v = np.asarray(v, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    poff = padded_offsets(offsets, align)
    buf = np.zeros((v.shape[1], int(poff[-1])))
    for e in range(len(offsets) - 1):
        n = offsets[e + 1] - offsets[e]
        buf[:, poff[e]:poff[e] + n] = v[offsets[e]:offsets[e + 1]].T
    codes, scales = quantize_lastdim(buf)
    return codes, scales, poff


def qdq_tokens(v, offsets, align=128):
    """Token-axis quantize-dequantize, returned in the original [M, C] layout."""
    codes, scales, poff = quantize_tokens(v, offsets, align)
    deq = dequantize_lastdim(codes, scales)
    out = np.zeros(np.shape(v))
    for e in range(len(offsets) - 1):
        n = offsets[e + 1] - offsets[e]
        out[offsets[e]:offsets[e + 1]] = deq[:, poff[e]:poff[e] + n].T
    return out


# --------------------------------------------------------------------------
# bfloat16 rounding (used where a bf16 value is stored and read back by a
# later step: the inputs, and h in the R-save mode).
# --------------------------------------------------------------------------

def round_bf16(v):
    """Round float64 to the nearest bfloat16 value (RNE, one rounding)."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    e = np.maximum(floor_log2(a), -126)          # bf16 min normal exponent
    q = np.ldexp(np.rint(np.ldexp(a, -(e - 7))), e - 7)   # 8 significant bits
    q = np.where(q >= 2.0 ** 128, np.inf, q)      # overflow past bf16 max
    out[fin] = np.copysign(q, v[fin])
    return out


# --------------------------------------------------------------------------
# Grouped linear: one call over all experts, rows grouped by offsets.
# --------------------------------------------------------------------------

def grouped_linear(A, B, offsets, row_scale=None):
    """Y[o_e:o_{e+1}] = A[o_e:o_{e+1}] @ B[e].T for every expert e.

    A [M, K], B [E, N, K], offsets [E+1] with offsets[0] = 0, offsets[E] = M.
    With row_scale, row i of Y is multiplied by row_scale[i].
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    Y = np.zeros((A.shape[0], B.shape[1]))
    for e in range(B.shape[0]):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            Y[lo:hi] = A[lo:hi] @ B[e].T
    if row_scale is not None:
        Y *= np.asarray(row_scale, dtype=np.float64)[:, None]
    return Y


def grouped_linear_mxfp8(A, B, offsets, row_scale=None):
    """Grouped linear on MXFP8 operands: both quantized along K first."""
    return grouped_linear(qdq_lastdim(A), qdq_lastdim(B), offsets, row_scale)


# --------------------------------------------------------------------------
# GroupedMLP forward and backward.
# --------------------------------------------------------------------------

def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def grouped_mlp_fwd(X, W1, W2, r, offsets, quantize=True):
    """Forward of the fused GroupedMLP, in the order gate-up -> SwiGLU ->
    routing-weight scale -> down projection.

    X [M, H] token-sorted rows, W1 [E, 2F, H], W2 [E, H, F], r [M],
    offsets [E+1].  Returns (Y [M, H], saved dict for the backward).
    """
    F = W2.shape[2]
    q = qdq_lastdim if quantize else (lambda t: np.asarray(t, np.float64))
    h = grouped_linear(q(X), q(W1), offsets)            # [M, 2F], K = H
    a, b = h[:, :F], h[:, F:]
    s = a * sigmoid(a) * b                              # SwiGLU
    z = np.asarray(r, np.float64)[:, None] * s          # routing-weight scale
    Y = grouped_linear(q(z), q(W2), offsets)            # K = F
    return Y, {"h": h, "s": s, "z": z}


def grouped_mlp_bwd(dY, X, W1, W2, r, offsets, saved, quantize=True,
                    align=128, h_bf16=False):
    """Backward of grouped_mlp_fwd (straight-through quantizers, R-ste).

    Returns dict with dX [M, H], dW1 [E, 2F, H], dW2 [E, H, F], dr [M].
    With quantize=False this is the exact gradient of the unquantized
    forward (loss L = sum(Y * dY)).  The SwiGLU backward reads h as the
    forward computed it (reading R-recomp); with h_bf16=True (quantized mode
    only) it reads bf16(h) instead, the copy a forward that stores h keeps
    (reading R-save).
    """
    dY = np.asarray(dY, np.float64)
    X = np.asarray(X, np.float64)
    W1 = np.asarray(W1, np.float64)
    W2 = np.asarray(W2, np.float64)
    r = np.asarray(r, np.float64)
    E, H, F = W2.shape
    h = saved["h"]                                      # reading R-recomp
    if quantize:
        q_row = qdq_lastdim
        q_tok = lambda t: qdq_tokens(t, offsets, align)
        if h_bf16:
            h = round_bf16(h)                           # reading R-save
    else:
        if h_bf16:
            raise ValueError("h_bf16 applies to the quantized backward only")
        q_row = q_tok = lambda t: np.asarray(t, np.float64)
    z = saved["z"]

    # dgrad of the down projection: dz = dY W2 (K = H), W2 blocks along H.
    dz = grouped_linear(q_row(dY), q_row(W2.transpose(0, 2, 1)), offsets)

    # wgrad of the down projection: dW2_e = dY_e^T z_e (K = tokens of e).
    dYt, zt = q_tok(dY), q_tok(z)
    dW2 = np.zeros((E, H, F))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        dW2[e] = dYt[lo:hi].T @ zt[lo:hi]

    # SwiGLU and routing-weight backward.
    a, b = h[:, :F], h[:, F:]
    sg = sigmoid(a)
    silu = a * sg
    s = silu * b
    dr = (dz * s).sum(axis=1)
    ds = r[:, None] * dz
    da = ds * b * sg * (1.0 + a * (1.0 - sg))
    db = ds * silu
    dh = np.concatenate([da, db], axis=1)               # [M, 2F]

    # dgrad of the gate-up projection: dX = dh W1 (K = 2F).
    dX = grouped_linear(q_row(dh), q_row(W1.transpose(0, 2, 1)), offsets)

    # wgrad of the gate-up projection: dW1_e = dh_e^T X_e (K = tokens of e).
    dht, Xt = q_tok(dh), q_tok(X)
    dW1 = np.zeros((E, 2 * F, H))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        dW1[e] = dht[lo:hi].T @ Xt[lo:hi]

    return {"dX": dX, "dW1": dW1, "dW2": dW2, "dr": dr, "dz": dz, "dh": dh}


# --------------------------------------------------------------------------
# Parity metrics.
# --------------------------------------------------------------------------

def parity_metrics(got, ref, row_axis_len=None):
    """(relative Frobenius error, max |got-ref| / rms(ref row)).

    Rows are the leading axes flattened, the last axis is the row.  For a
    1-D vector the whole vector is one row.  A row whose reference RMS is
    zero must be exactly zero in ``got``: any nonzero entry there returns
    an infinite row error.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.ndim == 1:
        got2, ref2 = got[None, :], ref[None, :]
    else:
        got2 = got.reshape(-1, ref.shape[-1])
        ref2 = ref.reshape(-1, ref.shape[-1])
    diff = got2 - ref2
    nref = np.linalg.norm(ref2)
    rel = np.linalg.norm(diff) / nref if nref > 0 else (
        0.0 if not np.any(diff) else np.inf)
    rms = np.sqrt((ref2 ** 2).mean(axis=1))
    worst = 0.0
    zero = rms == 0
    if np.any(zero) and np.any(diff[zero] != 0):
        worst = np.inf
    nz = ~zero
    if np.any(nz):
        worst = max(worst, float((np.abs(diff[nz]) / rms[nz][:, None]).max()))
    return float(rel), float(worst)
