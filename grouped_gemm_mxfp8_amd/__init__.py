"""MXFP8 MoE expert path for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libmxmoe.so`` (C ABI in ``include/mxmoe.h``).  The
functions carry the C names; each one checks tensor dtypes/devices, allocates
the outputs with torch (device memory only) and passes raw pointers and the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels: there is no fallback.  If the library is missing, importing the
functions raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MXMOE_LIB names another build of the same library (e.g. a host-sanitizer
# build); by default the in-tree one
LIB_PATH = os.environ.get("MXMOE_LIB") or os.path.join(HERE, "libmxmoe.so")

MX_DTYPE_BF16 = 0
MX_DTYPE_MXFP8 = 1
TOKEN_ALIGN = 128
BLOCK = 32
MX_CTX_H, MX_CTX_XCOL, MX_CTX_ZCOL, MX_CTX_POFF, MX_CTX_W1COL, MX_CTX_W2COL = 0, 1, 2, 3, 4, 5
MX_CTX_XROW, MX_CTX_W1ROW, MX_CTX_W2ROW = 6, 7, 8
MX_WS_ZROW, MX_WS_DHROW, MX_WS_DHCOL, MX_WS_DYROW, MX_WS_DYCOL = 0, 1, 2, 3, 4
MX_FWD_REUSE_WEIGHTS = 1
MX_MLP_SAVE_H = 2

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGS = {
    "mx_last_error": (ctypes.c_char_p, []),
    "mx_version": (ctypes.c_char_p, []),
    "mx_padded_rows_bound": (_I64, [_I64, _I32, _I32]),
    "mx_validate_offsets": (_I32, [_P, _I32, _I64]),
    "mxfp8_quantize": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _I32, _P, _P, _I64, _P, _P]),
    "grouped_linear_fwd": (_I32, [_I32, _P, _P, _P, _I32, _I64, _P, _P, _I64, _I64, _P, _P, _P]),
    "fp8_tensor_quantize": (_I32, [_P, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P]),
    "grouped_linear_fwd_fp8": (_I32, [_P, _P, _P, _I32, _I64, _P, _P, _I64, _I64, _P, _P, _P]),
    "grouped_mlp_fwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P,
                               _SZ, _P]),
    "grouped_mlp_fwd_ex": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P,
                                  _SZ, ctypes.c_uint32, _P]),
    "grouped_mlp_bwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P, _P, _P,
                               _P, _P, _SZ, _P]),
    "grouped_mlp_bwd_ex": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P, _P,
                                  _P, _P, _P, _SZ, ctypes.c_uint32, _P]),
    "grouped_mlp_ctx_bytes": (_SZ, [_I64, _I64, _I64, _I32, ctypes.c_uint32]),
    "moe_router": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_route_ws_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_route_plan": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_plan_noalloc": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_permute_quantize": (_I32, [_P, _I64, _I64, _P, _I64, _P, _I32, _P, _P, _P, _P, _I64,
                                    _P, _P]),
    "moe_combine": (_I32, [_P, _I64, _I64, _P, _I64, _I32, _P, _P, _P]),
    "moe_combine_bwd": (_I32, [_P, _I64, _I64, _I32, _P, _P, _P, _I64, _P, _P, _P]),
    "grouped_mlp_fwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I32, ctypes.c_uint32]),
    "grouped_mlp_bwd_ws_bytes": (_SZ, [_I64, _I64, _I64, _I32, ctypes.c_uint32]),
    "grouped_mlp_ctx_offset": (_I64, [_I32, _I64, _I64, _I64, _I32, ctypes.c_uint32]),
    "grouped_mlp_ws_offset": (_I64, [_I32, _I64, _I64, _I64, _I32, ctypes.c_uint32]),
}


class MxError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m grouped_gemm_mxfp8_amd._build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mx_last_error().decode()


def _check(fn, status):
    if status != 0:
        raise MxError(fn, status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def padded_rows_bound(M: int, G: int, align: int = TOKEN_ALIGN) -> int:
    return int(lib().mx_padded_rows_bound(M, G, align))


@dataclasses.dataclass
class MxTensor:
    """MXFP8 operand: E4M3 codes (uint8) and E8M0 scales (uint8)."""
    codes: torch.Tensor
    scales: torch.Tensor


def mxfp8_quantize(x: torch.Tensor, rowwise: bool = True, colwise: bool = False,
                   offsets: Optional[torch.Tensor] = None):
    """Block-quantize bf16 ``x`` ([R, C] or [batch, R, C]) to MXFP8.

    Returns a dict with ``row`` (MxTensor [.., R, C] / [.., R, C/32]) and/or
    ``col`` (MxTensor [.., C, ld] / [.., C, ld/32], transposed, token groups
    padded to 128) and ``padded_offsets`` (int64 [G+1]) when ``offsets`` is
    given.
    """
    _need(x, torch.bfloat16, "x")
    dev = x.device
    if x.dim() == 2:
        batch, (R, C) = 1, x.shape
        lead = ()
    elif x.dim() == 3:
        batch, R, C = x.shape
        lead = (batch,)
    else:
        raise ValueError("x must be 2-D or 3-D")
    G = 1
    if offsets is not None:
        _need(offsets, torch.int64, "offsets", dev)
        G = offsets.numel() - 1
    out = {}
    rc = rs = cc = cs = poff = None
    ld = 0
    if rowwise:
        rc = torch.empty((*lead, R, C), dtype=torch.uint8, device=dev)
        rs = torch.empty((*lead, R, C // BLOCK), dtype=torch.uint8, device=dev)
        out["row"] = MxTensor(rc, rs)
    if colwise:
        ld = padded_rows_bound(R, G)
        ld = max(ld, TOKEN_ALIGN)
        cc = torch.empty((*lead, C, ld), dtype=torch.uint8, device=dev)
        cs = torch.empty((*lead, C, ld // BLOCK), dtype=torch.uint8, device=dev)
        out["col"] = MxTensor(cc, cs)
        if offsets is not None:
            poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
            out["padded_offsets"] = poff
    st = lib().mxfp8_quantize(_ptr(x), batch, R, C, _ptr(rc), _ptr(rs), _ptr(offsets), G,
                              _ptr(cc), _ptr(cs), ld, _ptr(poff), _stream(dev))
    _check("mxfp8_quantize", st)
    return out


def grouped_linear_fwd(x, offsets: torch.Tensor, w, row_scale: Optional[torch.Tensor] = None):
    """GroupedLinear: y[rows of e] = x[rows of e] @ w[e].T for every expert.

    ``x`` bf16 [M, K] and ``w`` bf16 [E, N, K], or both MxTensor (rowwise
    MXFP8 copies).  Returns bf16 [M, N].
    """
    if isinstance(x, MxTensor):
        if not isinstance(w, MxTensor):
            raise TypeError("x and w must both be MXFP8 or both bf16")
        dtype = MX_DTYPE_MXFP8
        xc, xs, wc, ws = x.codes, x.scales, w.codes, w.scales
        _need(xc, torch.uint8, "x.codes")
        dev = xc.device
        _need(xs, torch.uint8, "x.scales", dev)
        _need(wc, torch.uint8, "w.codes", dev)
        _need(ws, torch.uint8, "w.scales", dev)
        M, K = xc.shape
        E, N, K2 = wc.shape
    else:
        dtype = MX_DTYPE_BF16
        _need(x, torch.bfloat16, "x")
        dev = x.device
        _need(w, torch.bfloat16, "w", dev)
        xc, xs, wc, ws = x, None, w, None
        M, K = x.shape
        E, N, K2 = w.shape
    if K2 != K:
        raise ValueError(f"K mismatch: x has {K}, w has {K2}")
    _need(offsets, torch.int64, "offsets", dev)
    if offsets.numel() != E + 1:
        raise ValueError("offsets must have E+1 entries")
    if row_scale is not None:
        _need(row_scale, torch.float32, "row_scale", dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = lib().grouped_linear_fwd(dtype, _ptr(xc), _ptr(xs), _ptr(offsets), E, M, _ptr(wc),
                                  _ptr(ws), N, K, _ptr(row_scale), _ptr(y), _stream(dev))
    _check("grouped_linear_fwd", st)
    return y


@dataclasses.dataclass
class Fp8Tensor:
    """Per-tensor scaled FP8 operand: E4M3 codes (uint8), and per group the
    amax and scale_inv (fp32)."""
    codes: torch.Tensor
    amax: torch.Tensor
    scale_inv: torch.Tensor


def fp8_tensor_quantize(x: torch.Tensor, offsets: Optional[torch.Tensor] = None) -> Fp8Tensor:
    """Per-tensor FP8 copy of bf16 ``x``: [M, C] with row groups ``offsets``
    (one scale per group), or [G, R, C] with one scale per matrix."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    if offsets is not None:
        if x.dim() != 2:
            raise ValueError("row groups need a 2-D x")
        _need(offsets, torch.int64, "offsets", dev)
        batch, (R, C) = 1, x.shape
        G = offsets.numel() - 1
    else:
        if x.dim() != 3:
            raise ValueError("without offsets x must be [G, R, C]")
        batch, R, C = x.shape
        G = batch
    codes = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    amax = torch.empty(G, dtype=torch.float32, device=dev)
    sinv = torch.empty(G, dtype=torch.float32, device=dev)
    st = lib().fp8_tensor_quantize(_ptr(x), batch, R, C, _ptr(offsets), G, _ptr(codes),
                                   _ptr(amax), _ptr(sinv), _stream(dev))
    _check("fp8_tensor_quantize", st)
    return Fp8Tensor(codes, amax, sinv)


def grouped_linear_fwd_fp8(x: Fp8Tensor, offsets: torch.Tensor, w: Fp8Tensor,
                           row_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GroupedLinear on per-tensor FP8 operands: bf16 [M, N]."""
    _need(x.codes, torch.uint8, "x.codes")
    dev = x.codes.device
    _need(x.scale_inv, torch.float32, "x.scale_inv", dev)
    _need(w.codes, torch.uint8, "w.codes", dev)
    _need(w.scale_inv, torch.float32, "w.scale_inv", dev)
    _need(offsets, torch.int64, "offsets", dev)
    M, K = x.codes.shape
    E, N, K2 = w.codes.shape
    if K2 != K:
        raise ValueError(f"K mismatch: x has {K}, w has {K2}")
    if offsets.numel() != E + 1 or x.scale_inv.numel() != E or w.scale_inv.numel() != E:
        raise ValueError("offsets must have E+1 entries and each scale_inv E")
    if row_scale is not None:
        _need(row_scale, torch.float32, "row_scale", dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = lib().grouped_linear_fwd_fp8(_ptr(x.codes), _ptr(x.scale_inv), _ptr(offsets), E, M,
                                      _ptr(w.codes), _ptr(w.scale_inv), N, K, _ptr(row_scale),
                                      _ptr(y), _stream(dev))
    _check("grouped_linear_fwd_fp8", st)
    return y


def _flags(save_h: bool) -> int:
    return MX_MLP_SAVE_H if save_h else 0


@dataclasses.dataclass
class MlpCtx:
    """Saved-for-backward state of grouped_mlp_fwd (opaque device buffer).
    ``save_h``: written in the save-h mode (h stored as bf16) rather than the
    default recompute mode."""
    buf: torch.Tensor
    M: int
    H: int
    F: int
    E: int
    offsets: Optional[torch.Tensor] = None
    save_h: bool = False

    @property
    def padded_rows(self) -> int:
        return padded_rows_bound(self.M, self.E)

    def _off(self, which):
        off = int(lib().grouped_mlp_ctx_offset(which, self.M, self.H, self.F, self.E,
                                               _flags(self.save_h)))
        if off < 0:
            raise MxError("grouped_mlp_ctx_offset", 1, last_error())
        return off

    def h(self) -> torch.Tensor:
        """Saved gate-up pre-activation as bf16 [M, 2F] (save-h mode only),
        gathered from the library's 16 x 16 blocked layout (see MX_CTX_H in
        include/mxmoe.h)."""
        Mp, F = self.padded_rows, self.F
        raw = _region(self.buf, self._off(MX_CTX_H), (Mp // 16, F // 16, 4, 16, 2, 4),
                      torch.bfloat16)[0]
        hp = raw.permute(0, 3, 4, 1, 2, 5).reshape(Mp, 2 * F)
        poff = self.padded_offsets().cpu().tolist()
        offs = self.offsets.cpu().tolist()
        rows = [torch.arange(poff[e], poff[e] + (offs[e + 1] - offs[e]))
                for e in range(self.E)]
        idx = torch.cat(rows).to(hp.device) if rows else torch.zeros(0, dtype=torch.int64)
        return hp.index_select(0, idx)

    def xrow(self) -> MxTensor:
        """Rowwise MXFP8 copy of X kept for the recompute (default mode):
        codes [M, H], scales [M, H/32]."""
        return self._mx(MX_CTX_XROW, (self.M, self.H))

    def w1row(self) -> MxTensor:
        """Rowwise MXFP8 copy of W1: codes [E*2F, H], scales [E*2F, H/32]."""
        return self._mx(MX_CTX_W1ROW, (self.E * 2 * self.F, self.H))

    def w2row(self) -> MxTensor:
        """Rowwise MXFP8 copy of W2: codes [E*H, F], scales [E*H, F/32]."""
        return self._mx(MX_CTX_W2ROW, (self.E * self.H, self.F))

    def xcol(self) -> MxTensor:
        """Token-axis MXFP8 copy of X: codes [H, Mp], scales [H, Mp/32]
        (row-major copy of the tiled scales)."""
        return self._mx(MX_CTX_XCOL, (self.H, self.padded_rows))

    def zcol(self) -> MxTensor:
        """Token-axis MXFP8 copy of z: codes [F, Mp], scales [F, Mp/32]
        (row-major copy of the tiled scales)."""
        return self._mx(MX_CTX_ZCOL, (self.F, self.padded_rows))

    def w1col(self) -> MxTensor:
        """Columnwise MXFP8 copy of W1 made by the forward: codes [E*H, 2F]
        (row e*H + k is column k of expert e's W1), scales [E*H, 2F/32]."""
        return self._mx(MX_CTX_W1COL, (self.E * self.H, 2 * self.F))

    def w2col(self) -> MxTensor:
        """Columnwise MXFP8 copy of W2: codes [E*F, H], scales [E*F, H/32]."""
        return self._mx(MX_CTX_W2COL, (self.E * self.F, self.H))

    def padded_offsets(self) -> torch.Tensor:
        return _region(self.buf, self._off(MX_CTX_POFF), (self.E + 1,), torch.int64)[0]

    def _mx(self, which, shape):
        return _tiled_mx_view(self.buf, self._off(which), shape)


def _mlp_check(x, offsets, w1, w2, r):
    _need(x, torch.bfloat16, "x")
    dev = x.device
    _need(offsets, torch.int64, "offsets", dev)
    _need(w1, torch.bfloat16, "w1", dev)
    _need(w2, torch.bfloat16, "w2", dev)
    _need(r, torch.float32, "r", dev)
    M, H = x.shape
    E, F2, H1 = w1.shape
    E2, H2, F = w2.shape
    if H1 != H or H2 != H or E2 != E or F2 != 2 * F:
        raise ValueError("shape mismatch: x [M,H], w1 [E,2F,H], w2 [E,H,F]")
    if r.shape != (M,) or offsets.numel() != E + 1:
        raise ValueError("r must be [M] and offsets [E+1]")
    return dev, M, H, F, E


def ctx_bytes(M, H, F, E, save_h: bool = False) -> int:
    return int(lib().grouped_mlp_ctx_bytes(M, H, F, E, _flags(save_h)))


def fwd_ws_bytes(M, H, F, E, save_h: bool = False) -> int:
    return int(lib().grouped_mlp_fwd_ws_bytes(M, H, F, E, _flags(save_h)))


def bwd_ws_bytes(M, H, F, E, save_h: bool = False) -> int:
    return int(lib().grouped_mlp_bwd_ws_bytes(M, H, F, E, _flags(save_h)))


def grouped_mlp_fwd(x, offsets, w1, w2, r, ws: Optional[torch.Tensor] = None,
                    ctx_buf: Optional[torch.Tensor] = None, reuse_weights: bool = False,
                    save_h: bool = False):
    """Fused GroupedMLP forward.  Returns (y bf16 [M, H], MlpCtx).  ``ws`` and
    ``ctx_buf`` are optional caller-owned uint8 buffers (allocated when
    missing or too small).  ``reuse_weights``: use the MXFP8 weight copies an
    earlier call with the same weights (and the same ``save_h``) left in
    ``ctx_buf`` (which must then be given) instead of quantizing w1 and w2
    again.  ``save_h``: store h as bf16 for the backward instead of having the
    backward recompute it."""
    dev, M, H, F, E = _mlp_check(x, offsets, w1, w2, r)
    L = lib()
    fl = _flags(save_h)
    nctx = L.grouped_mlp_ctx_bytes(M, H, F, E, fl)
    nws = L.grouped_mlp_fwd_ws_bytes(M, H, F, E, fl)
    if nctx == 0 or nws == 0:
        raise MxError("grouped_mlp_fwd", 2, last_error())
    if reuse_weights and (ctx_buf is None or ctx_buf.numel() < nctx):
        raise ValueError("reuse_weights needs the ctx_buf of the earlier call")
    ctx = ctx_buf if ctx_buf is not None and ctx_buf.numel() >= nctx else \
        torch.empty(nctx, dtype=torch.uint8, device=dev)
    if ws is None or ws.numel() < nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    st = L.grouped_mlp_fwd_ex(_ptr(x), _ptr(offsets), E, M, H, F, _ptr(w1), _ptr(w2), _ptr(r),
                              _ptr(y), _ptr(ctx), ctx.numel(), _ptr(ws), ws.numel(),
                              fl | (MX_FWD_REUSE_WEIGHTS if reuse_weights else 0), _stream(dev))
    _check("grouped_mlp_fwd", st)
    return y, MlpCtx(ctx, M, H, F, E, offsets, save_h)


def grouped_mlp_bwd(dy, offsets, w1, w2, r, ctx: MlpCtx, ws: Optional[torch.Tensor] = None):
    """Fused GroupedMLP backward (in the mode the forward wrote ``ctx`` in).
    Returns (dx, dw1, dw2, dr)."""
    dev, M, H, F, E = _mlp_check(dy, offsets, w1, w2, r)
    if (ctx.M, ctx.H, ctx.F, ctx.E) != (M, H, F, E):
        raise ValueError("ctx was made for other sizes")
    L = lib()
    fl = _flags(ctx.save_h)
    nws = L.grouped_mlp_bwd_ws_bytes(M, H, F, E, fl)
    if ws is None or ws.numel() < nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    dx = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((E, 2 * F, H), dtype=torch.bfloat16, device=dev)
    dw2 = torch.empty((E, H, F), dtype=torch.bfloat16, device=dev)
    dr = torch.empty((M,), dtype=torch.float32, device=dev)
    st = L.grouped_mlp_bwd_ex(_ptr(dy), _ptr(offsets), E, M, H, F, _ptr(w1), _ptr(w2), _ptr(r),
                              _ptr(ctx.buf), ctx.buf.numel(), _ptr(dx), _ptr(dw1), _ptr(dw2),
                              _ptr(dr), _ptr(ws), ws.numel(), fl, _stream(dev))
    _check("grouped_mlp_bwd", st)
    return dx, dw1, dw2, dr


def _region(buf: torch.Tensor, off: int, shape, dtype):
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return buf[off:off + nbytes].view(dtype).view(*shape), (off + nbytes + 255) // 256 * 256


def _tiled_mx_view(buf: torch.Tensor, off: int, shape) -> MxTensor:
    """Codes [R, Kp] at ``off`` and the K-step tiled scales after them (the
    library's internal layout, see include/mxmoe.h), returned as row-major
    scales [R, Kp/32] (a gathered copy; codes are a view)."""
    R, Kp = shape
    codes, nxt = _region(buf, off, shape, torch.uint8)
    groups = (R + 31) // 32
    raw, _ = _region(buf, nxt, (groups, Kp // 128, 32, 4), torch.uint8)
    scales = raw.permute(0, 2, 1, 3).reshape(groups * 32, Kp // BLOCK)[:R]
    return MxTensor(codes, scales)


def ws_mx_view(ws: torch.Tensor, which: int, M, H, F, E, shape,
               save_h: bool = False) -> MxTensor:
    """MXFP8 tensor inside a forward/backward workspace: codes of ``shape``
    [R, Kp] at the documented offset, scales at the next 256-byte boundary in
    the K-step tiled layout, returned row-major [R, Kp/32] (see
    include/mxmoe.h)."""
    off = int(lib().grouped_mlp_ws_offset(which, M, H, F, E, _flags(save_h)))
    if off < 0:
        raise MxError("grouped_mlp_ws_offset", 1, last_error())
    return _tiled_mx_view(ws, off, shape)


# ---- routing around the expert path ------------------------------------------

def router(logits: torch.Tensor, k: int):
    """Top-k experts of every token (lower index among equal logits) and the
    softmax of their logits: (ids int32 [T, k], w fp32 [T, k])."""
    _need(logits, torch.float32, "logits")
    dev = logits.device
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    st = lib().moe_router(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(dev))
    _check("moe_router", st)
    return ids, w


def route_plan(ids: torch.Tensor, E: int, w: Optional[torch.Tensor] = None):
    """Sorted-row plan of a top-k routing ``ids`` int32 [T, k] over E experts.

    Returns (offsets int64 [E+1], row_of int32 [T, k], tok_of int32 [T*k],
    r_sorted fp32 [T*k] or None): rows sorted stably by (expert, token, slot);
    ``r_sorted`` holds ``w`` (fp32 [T, k]) in row order."""
    _need(ids, torch.int32, "ids")
    dev = ids.device
    if ids.dim() != 2:
        raise ValueError("ids must be [T, k]")
    T, k = ids.shape
    if w is not None:
        _need(w, torch.float32, "w", dev)
        if tuple(w.shape) != (T, k):
            raise ValueError("w must match ids")
    L = lib()
    nws = L.moe_route_ws_bytes(T, k, E)
    if nws == 0:
        raise MxError("moe_route_plan", 1, "bad sizes")
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int64, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    tok_of = torch.empty(T * k, dtype=torch.int32, device=dev)
    r_sorted = torch.empty(T * k, dtype=torch.float32, device=dev) if w is not None else None
    st = L.moe_route_plan(_ptr(ids), T, k, E, _ptr(w), _ptr(offsets), _ptr(row_of), _ptr(tok_of),
                          _ptr(r_sorted), _ptr(ws), nws, _stream(dev))
    _check("moe_route_plan", st)
    return offsets, row_of, tok_of, r_sorted


def route_plan_noalloc(ids: torch.Tensor, E: int, w: Optional[torch.Tensor] = None):
    """``route_plan`` through the entry point that allocates nothing on the
    device: the library's own scratch replaces the workspace (calls that
    overlap on one GPU race; see include/mxmoe.h).  The outputs are still
    allocated here, by torch."""
    _need(ids, torch.int32, "ids")
    dev = ids.device
    if ids.dim() != 2:
        raise ValueError("ids must be [T, k]")
    T, k = ids.shape
    if w is not None:
        _need(w, torch.float32, "w", dev)
        if tuple(w.shape) != (T, k):
            raise ValueError("w must match ids")
    offsets = torch.empty(E + 1, dtype=torch.int64, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    tok_of = torch.empty(T * k, dtype=torch.int32, device=dev)
    r_sorted = torch.empty(T * k, dtype=torch.float32, device=dev) if w is not None else None
    st = lib().moe_route_plan_noalloc(_ptr(ids), T, k, E, _ptr(w), _ptr(offsets), _ptr(row_of),
                                      _ptr(tok_of), _ptr(r_sorted), _stream(dev))
    _check("moe_route_plan_noalloc", st)
    return offsets, row_of, tok_of, r_sorted


def permute_quantize(x: torch.Tensor, tok_of: torch.Tensor, offsets: torch.Tensor, M: int,
                     rowwise: bool = True, colwise: bool = True):
    """MXFP8 copies of the sorted rows x[tok_of[row]] (x bf16 [T, H]), made
    straight from token order; same outputs as ``mxfp8_quantize`` of the
    sorted rows with ``offsets``: dict with ``row``, ``col`` and
    ``padded_offsets``."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    _need(tok_of, torch.int32, "tok_of", dev)
    _need(offsets, torch.int64, "offsets", dev)
    T, H = x.shape
    E = offsets.numel() - 1
    out = {}
    rc = rs = cc = cs = None
    ld = 0
    if rowwise:
        rc = torch.empty((M, H), dtype=torch.uint8, device=dev)
        rs = torch.empty((M, H // BLOCK), dtype=torch.uint8, device=dev)
        out["row"] = MxTensor(rc, rs)
    if colwise:
        ld = max(padded_rows_bound(M, E), TOKEN_ALIGN)
        cc = torch.empty((H, ld), dtype=torch.uint8, device=dev)
        cs = torch.empty((H, ld // BLOCK), dtype=torch.uint8, device=dev)
        out["col"] = MxTensor(cc, cs)
    poff = torch.empty(E + 1, dtype=torch.int64, device=dev)
    out["padded_offsets"] = poff
    st = lib().moe_permute_quantize(_ptr(x), T, H, _ptr(tok_of), M, _ptr(offsets), E, _ptr(rc),
                                    _ptr(rs), _ptr(cc), _ptr(cs), ld, _ptr(poff), _stream(dev))
    _check("moe_permute_quantize", st)
    return out


def combine(y: torch.Tensor, row_of: torch.Tensor, w: Optional[torch.Tensor] = None):
    """out bf16 [T, H] = sum_j c[t, j] * y[row_of[t, j]], c = w or 1."""
    _need(y, torch.bfloat16, "y")
    dev = y.device
    _need(row_of, torch.int32, "row_of", dev)
    if w is not None:
        _need(w, torch.float32, "w", dev)
    M, H = y.shape
    T, k = row_of.shape
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    st = lib().moe_combine(_ptr(y), M, H, _ptr(row_of), T, k, _ptr(w), _ptr(out), _stream(dev))
    _check("moe_combine", st)
    return out


def combine_bwd(dout: torch.Tensor, row_of: torch.Tensor, M: int,
                w: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None):
    """Backward of ``combine``: (dy bf16 [M, H], dw fp32 [T, k] or None).
    Unweighted it is the token -> sorted-row permute of ``dout``."""
    _need(dout, torch.bfloat16, "dout")
    dev = dout.device
    _need(row_of, torch.int32, "row_of", dev)
    T, H = dout.shape
    k = row_of.shape[1]
    if w is not None:
        _need(w, torch.float32, "w", dev)
    if y is not None:
        _need(y, torch.bfloat16, "y", dev)
    dy = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev) if (w is not None and
                                                                  y is not None) else None
    st = lib().moe_combine_bwd(_ptr(dout), T, H, k, _ptr(row_of), _ptr(w), _ptr(y), M, _ptr(dy),
                               _ptr(dw), _stream(dev))
    _check("moe_combine_bwd", st)
    return dy, dw


__all__ = ["lib", "last_error", "MxError", "MxTensor", "MlpCtx", "mxfp8_quantize",
           "grouped_linear_fwd", "fp8_tensor_quantize", "grouped_linear_fwd_fp8", "Fp8Tensor",
           "grouped_mlp_fwd", "grouped_mlp_bwd", "padded_rows_bound",
           "ws_mx_view", "ctx_bytes", "fwd_ws_bytes", "bwd_ws_bytes", "router", "route_plan",
           "route_plan_noalloc", "permute_quantize",
           "combine", "combine_bwd"]
