"""Host-side checks of the C ABI: the library loads, exports every function
the header declares, and rejects bad arguments with the documented status
before touching the device (no GPU needed: no kernel is launched)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxmoe.h")

MX_OK, MX_ERR_INVALID_ARG, MX_ERR_UNSUPPORTED, MX_ERR_WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x7f0000001000)       # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x7f0000002000)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s*]+(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for fn in ("mxfp8_quantize", "grouped_linear_fwd", "grouped_mlp_fwd", "grouped_mlp_bwd"):
        assert fn in names


def test_library_exports_every_declared_function(mxlib):
    missing = [n for n in declared_functions() if not hasattr(mxlib, n)]
    assert not missing, missing


def test_version_and_empty_error(mxlib):
    assert b"gfx950" in mxlib.mx_version()
    assert mxlib.mx_last_error() is not None


def test_padded_rows_bound_closed_form(mxlib):
    f = mxlib.mx_padded_rows_bound
    # sum ceil(n_e/a)*a <= M + G(a-1), rounded down to a multiple of a
    assert f(0, 1, 128) == 0
    assert f(1, 1, 128) == 128
    assert f(128, 1, 128) == 128
    assert f(129, 1, 128) == 256
    assert f(32768, 8, 128) == (32768 + 8 * 127) // 128 * 128
    assert f(-1, 1, 128) == -1 and f(5, 0, 128) == -1


def test_padded_bound_dominates_every_split(mxlib):
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(200):
        G = int(rng.integers(1, 70))
        counts = rng.integers(0, 400, G)
        M = int(counts.sum())
        padded = int(((counts + 127) // 128 * 128).sum())
        assert padded <= mxlib.mx_padded_rows_bound(M, G, 128)


SAVE_H = 2


def test_mlp_sizes(mxlib):
    M, H, F, E = 32768, 4096, 14336, 8
    Mp = mxlib.mx_padded_rows_bound(M, E, 128)
    weights = E * (2 * F * H + F * H) * 2 * (1 + 1 / 32)       # rowwise + columnwise copies
    tok = (H + F) * Mp * (1 + 1 / 32)                          # X and z token-axis copies
    # recompute mode: X rowwise copy (the backward recomputes h from it)
    ctx_r = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, 0)
    need_r = weights + tok + M * H * (1 + 1 / 32)
    assert need_r <= ctx_r <= need_r + 64 * 256
    # save-h mode: h (bf16, 16x16 blocks over padded rows: Mp*F*4 bytes)
    ctx_s = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, SAVE_H)
    need_s = weights + tok + Mp * F * 4
    assert need_s <= ctx_s <= need_s + 64 * 256
    for fl in (0, SAVE_H):
        assert mxlib.grouped_mlp_fwd_ws_bytes(M, H, F, E, fl) > 0
        assert mxlib.grouped_mlp_bwd_ws_bytes(M, H, F, E, fl) > 0
    # regions of each mode
    both = (1, 2, 3, 4, 5, 7, 8)
    for fl, own, other in ((0, 6, 0), (SAVE_H, 0, 6)):
        ctx = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, fl)
        for which in both + (own,):
            off = mxlib.grouped_mlp_ctx_offset(which, M, H, F, E, fl)
            assert 0 <= off < ctx and off % 256 == 0
        assert mxlib.grouped_mlp_ctx_offset(other, M, H, F, E, fl) == -1
        assert "mode" in _err(mxlib)
        assert mxlib.grouped_mlp_ctx_offset(9, M, H, F, E, fl) == -1
        for which in range(5):
            assert mxlib.grouped_mlp_ws_offset(which, M, H, F, E, fl) >= 0
        assert mxlib.grouped_mlp_ws_offset(5, M, H, F, E, fl) == -1
    # unsupported sizes and unknown flags give 0 / -1
    assert mxlib.grouped_mlp_ctx_bytes(M, 4000, F, E, 0) == 0
    assert mxlib.grouped_mlp_ctx_bytes(M, H, F, 0, 0) == 0
    assert mxlib.grouped_mlp_ctx_bytes(M, H, F, E, 1) == 0
    assert mxlib.grouped_mlp_fwd_ws_bytes(M, H, F, E, 4) == 0
    assert mxlib.grouped_mlp_ctx_offset(1, M, H, 100, E, 0) == -1
    assert mxlib.grouped_mlp_ctx_offset(1, M, H, F, E, 8) == -1
    assert "flags" in _err(mxlib)


def _err(mxlib):
    return mxlib.mx_last_error().decode()


def test_quantize_rejects_bad_arguments(mxlib):
    q = mxlib.mxfp8_quantize
    # NULL input
    assert q(None, 1, 64, 64, FAKE, FAKE2, None, 1, None, None, 0, None, None) == MX_ERR_INVALID_ARG
    assert "NULL" in _err(mxlib)
    # C not a multiple of 32
    assert q(FAKE, 1, 64, 48, FAKE, FAKE2, None, 1, None, None, 0, None, None) == MX_ERR_UNSUPPORTED
    # no output requested
    assert q(FAKE, 1, 64, 64, None, None, None, 1, None, None, 0, None, None) == MX_ERR_INVALID_ARG
    # codes without scales
    assert q(FAKE, 1, 64, 64, FAKE, None, None, 1, None, None, 0, None, None) == MX_ERR_INVALID_ARG
    # columnwise leading dimension too small / not a multiple of 128
    assert q(FAKE, 1, 300, 64, None, None, None, 1, FAKE, FAKE2, 128, None, None) == MX_ERR_INVALID_ARG
    assert q(FAKE, 1, 64, 64, None, None, None, 1, FAKE, FAKE2, 100, None, None) == MX_ERR_INVALID_ARG
    # grouped columnwise without padded-offsets output
    assert q(FAKE, 1, 64, 64, None, None, FAKE, 2, FAKE, FAKE2, 384, None, None) == MX_ERR_INVALID_ARG
    # groups with batch > 1
    assert q(FAKE, 2, 64, 64, None, None, FAKE, 2, FAKE, FAKE2, 384, FAKE, None) == MX_ERR_INVALID_ARG
    # too many groups
    assert q(FAKE, 1, 64, 64, None, None, FAKE, 5000, FAKE, FAKE2, 1 << 20, FAKE, None) == MX_ERR_UNSUPPORTED
    # misaligned input
    assert q(ctypes.c_void_p(0x7f0000001001), 1, 64, 64, FAKE, FAKE2, None, 1, None, None, 0,
             None, None) == MX_ERR_INVALID_ARG
    # misaligned scales
    assert q(FAKE, 1, 64, 64, FAKE, ctypes.c_void_p(0x7f0000002002), None, 1, None, None, 0,
             None, None) == MX_ERR_INVALID_ARG
    assert "scales" in _err(mxlib)
    assert q(FAKE, 1, 64, 64, None, None, None, 1, FAKE, ctypes.c_void_p(0x7f0000002001), 128,
             None, None) == MX_ERR_INVALID_ARG


def test_grouped_linear_rejects_bad_arguments(mxlib):
    f = mxlib.grouped_linear_fwd
    # NULL pointers
    assert f(0, None, None, FAKE, 4, 512, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG
    # unknown dtype
    assert f(7, FAKE, None, FAKE, 4, 512, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG
    # bf16 with scales
    assert f(0, FAKE, FAKE, FAKE, 4, 512, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG
    # bf16 K not a multiple of 32
    assert f(0, FAKE, None, FAKE, 4, 512, FAKE, None, 256, 100, None, FAKE, None) == MX_ERR_UNSUPPORTED
    # MXFP8 without scales; MXFP8 with K or N not a multiple of the 32-element block
    assert f(1, FAKE, None, FAKE, 4, 512, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG
    assert f(1, FAKE, FAKE, FAKE, 4, 512, FAKE, FAKE, 256, 100, None, FAKE, None) == MX_ERR_UNSUPPORTED
    assert f(1, FAKE, FAKE, FAKE, 4, 512, FAKE, FAKE, 250, 128, None, FAKE, None) == MX_ERR_UNSUPPORTED
    # E out of range, negative M
    assert f(0, FAKE, None, FAKE, 0, 512, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG
    assert f(0, FAKE, None, FAKE, 4, -1, FAKE, None, 256, 128, None, FAKE, None) == MX_ERR_INVALID_ARG


def test_grouped_mlp_rejects_bad_arguments(mxlib):
    fwd, bwd = mxlib.grouped_mlp_fwd, mxlib.grouped_mlp_bwd
    M, H, F, E = 1024, 256, 256, 4
    nctx = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, 0)
    nws = mxlib.grouped_mlp_fwd_ws_bytes(M, H, F, E, 0)
    nbws = mxlib.grouped_mlp_bwd_ws_bytes(M, H, F, E, 0)
    args = lambda **kw: [kw.get("x", FAKE), FAKE, kw.get("E", E), M, kw.get("H", H), F, FAKE,
                         FAKE, FAKE, FAKE, FAKE, kw.get("nctx", nctx), FAKE, kw.get("nws", nws),
                         None]
    assert fwd(*args(x=None)) == MX_ERR_INVALID_ARG
    assert fwd(*args(H=200)) == MX_ERR_UNSUPPORTED
    assert fwd(*args(E=0)) == MX_ERR_INVALID_ARG
    assert fwd(*args(E=2000)) == MX_ERR_UNSUPPORTED
    assert fwd(*args(nctx=nctx - 1)) == MX_ERR_WORKSPACE
    assert "ctx" in _err(mxlib)
    assert fwd(*args(nws=nws - 1)) == MX_ERR_WORKSPACE
    b = [FAKE, FAKE, E, M, H, F, FAKE, FAKE, FAKE, FAKE, nctx, FAKE, FAKE, FAKE, FAKE, FAKE,
         nbws - 1, None]
    assert bwd(*b) == MX_ERR_WORKSPACE
    b[0] = None
    assert bwd(*b) == MX_ERR_INVALID_ARG
    # the save-h backward needs the (larger) ctx of the save-h mode
    bex = mxlib.grouped_mlp_bwd_ex
    nctx_s = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, SAVE_H)
    nbws_s = mxlib.grouped_mlp_bwd_ws_bytes(M, H, F, E, SAVE_H)
    assert nctx_s > nctx
    b = [FAKE, FAKE, E, M, H, F, FAKE, FAKE, FAKE, FAKE, nctx, FAKE, FAKE, FAKE, FAKE, FAKE,
         nbws_s, SAVE_H, None]
    assert bex(*b) == MX_ERR_WORKSPACE
    b[17] = 4
    assert bex(*b) == MX_ERR_INVALID_ARG
    assert "flags" in _err(mxlib)


def test_grouped_mlp_fwd_ex_checks_flags_and_weights(mxlib):
    """The flags entry point validates on the host: unknown flag bits, weights
    required unless reused, workspace sizes (no GPU call is reached)."""
    fwd = mxlib.grouped_mlp_fwd_ex
    M, H, F, E = 1024, 256, 256, 4
    nctx = mxlib.grouped_mlp_ctx_bytes(M, H, F, E, 0)
    nws = mxlib.grouped_mlp_fwd_ws_bytes(M, H, F, E, SAVE_H)     # the larger of the two
    args = lambda flags, w=FAKE, n=nctx: [FAKE, FAKE, E, M, H, F, w, w, FAKE, FAKE, FAKE, n,
                                          FAKE, nws, flags, None]
    assert fwd(*args(4)) == MX_ERR_INVALID_ARG
    assert "flags" in _err(mxlib)
    assert fwd(*args(0, w=None)) == MX_ERR_INVALID_ARG
    assert fwd(*args(1, w=None, n=nctx - 1)) == MX_ERR_WORKSPACE
    # the save-h forward needs the save-h ctx
    assert fwd(*args(SAVE_H)) == MX_ERR_WORKSPACE
    assert fwd(*args(SAVE_H | 1, w=None)) == MX_ERR_WORKSPACE


def test_weight_regions_do_not_move_with_m(mxlib):
    """Reused weight copies sit at offsets that do not depend on M."""
    H, F, E = 256, 512, 4
    for fl in (0, SAVE_H):
        for which in (4, 5, 7, 8):     # the ctx regions of the weight copies
            offs = {mxlib.grouped_mlp_ctx_offset(which, M, H, F, E, fl)
                    for M in (0, 100, 4096, 9999)}
            assert len(offs) == 1 and offs.pop() >= 0


def test_routing_entry_points_reject_bad_arguments(mxlib):
    """Host-side validation of the routing entry points (no GPU call is
    reached)."""
    assert mxlib.moe_route_ws_bytes(100, 2, 8) == 1 * 8 * 4
    assert mxlib.moe_route_ws_bytes(1000, 2, 8) == 8 * 8 * 4     # ceil(2000/256) chunks
    assert mxlib.moe_route_ws_bytes(10, 0, 8) == 0
    assert mxlib.moe_route_ws_bytes(10, 2, 2000) == 0
    plan = mxlib.moe_route_plan
    nws = mxlib.moe_route_ws_bytes(100, 2, 8)
    base = [FAKE, 100, 2, 8, None, FAKE, FAKE, FAKE, None, FAKE, nws, None]
    a = list(base); a[3] = 2000
    assert plan(*a) == MX_ERR_UNSUPPORTED
    a = list(base); a[2] = 0
    assert plan(*a) == MX_ERR_INVALID_ARG
    a = list(base); a[4] = FAKE                     # weights without their sorted copy
    assert plan(*a) == MX_ERR_INVALID_ARG
    assert "go together" in _err(mxlib)
    a = list(base); a[10] = nws - 1
    assert plan(*a) == MX_ERR_WORKSPACE
    a = list(base); a[0] = None
    assert plan(*a) == MX_ERR_INVALID_ARG
    pq = mxlib.moe_permute_quantize
    args = [FAKE, 100, 256, FAKE, 200, FAKE, 8, FAKE, FAKE, None, None, 0, FAKE, None]
    a = list(args); a[2] = 100                      # H not a multiple of 32
    assert pq(*a) == MX_ERR_UNSUPPORTED
    a = list(args); a[7] = None                     # row codes without scales
    assert pq(*a) == MX_ERR_INVALID_ARG
    a = list(args); a[12] = None
    assert pq(*a) == MX_ERR_INVALID_ARG
    a = list(args); a[1] = 1 << 20; a[2] = 4096     # T*H*2 past 2^31
    assert pq(*a) == MX_ERR_UNSUPPORTED
    a = list(args); a[9] = FAKE; a[10] = FAKE; a[11] = 64   # col_ld not a multiple of 128
    assert pq(*a) == MX_ERR_INVALID_ARG
    comb = mxlib.moe_combine
    assert comb(FAKE, 200, 100, FAKE, 100, 2, None, FAKE, None) == MX_ERR_UNSUPPORTED
    assert comb(None, 200, 128, FAKE, 100, 2, None, FAKE, None) == MX_ERR_INVALID_ARG
    bwd = mxlib.moe_combine_bwd
    assert bwd(FAKE, 100, 128, 2, FAKE, None, None, 200, FAKE, FAKE, None) == MX_ERR_INVALID_ARG
    assert "needs" in _err(mxlib)
    fq = mxlib.fp8_tensor_quantize
    fargs = [FAKE, 1, 100, 64, FAKE, 4, FAKE, FAKE, FAKE, None]
    a = list(fargs); a[3] = 48                                  # C not a multiple of 32
    assert fq(*a) == MX_ERR_UNSUPPORTED
    a = list(fargs); a[1] = 2                                   # row groups with batch 2
    assert fq(*a) == MX_ERR_INVALID_ARG
    a = list(fargs); a[4] = None                                # matrices: G must equal batch
    assert fq(*a) == MX_ERR_INVALID_ARG
    a = list(fargs); a[5] = 2000
    assert fq(*a) == MX_ERR_UNSUPPORTED
    a = list(fargs); a[8] = None                                # no scale_inv buffer
    assert fq(*a) == MX_ERR_INVALID_ARG
    a = list(fargs); a[3] = 1 << 24                             # 256 * C past 2^31
    assert fq(*a) == MX_ERR_UNSUPPORTED
    lf = mxlib.grouped_linear_fwd_fp8
    largs = [FAKE, FAKE, FAKE, 8, 100, FAKE, FAKE, 256, 1024, None, FAKE, None]
    a = list(largs); a[8] = 1000                                # K not a multiple of 128
    assert lf(*a) == MX_ERR_UNSUPPORTED
    a = list(largs); a[6] = None                                # no w scale_inv
    assert lf(*a) == MX_ERR_INVALID_ARG
    a = list(largs); a[3] = 0
    assert lf(*a) == MX_ERR_INVALID_ARG
    a = list(largs); a[4] = 0                                   # no rows: nothing to do
    assert lf(*a) == MX_OK
    rt = mxlib.moe_router
    assert rt(FAKE, 100, 8, 0, FAKE, FAKE, None) == MX_ERR_INVALID_ARG       # k = 0
    assert rt(FAKE, 100, 8, 9, FAKE, FAKE, None) == MX_ERR_INVALID_ARG       # k > E
    assert rt(FAKE, 100, 2000, 2, FAKE, FAKE, None) == MX_ERR_UNSUPPORTED    # E > 1024
    assert rt(FAKE, 100, 128, 65, FAKE, FAKE, None) == MX_ERR_UNSUPPORTED    # k > 64
    assert rt(FAKE, 1 << 30, 8, 4, FAKE, FAKE, None) == MX_ERR_UNSUPPORTED   # T*k past 2^31
    assert rt(FAKE, 100, 8, 2, None, FAKE, None) == MX_ERR_INVALID_ARG
    assert rt(None, 0, 8, 2, None, None, None) == MX_OK                     # nothing to do


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import grouped_gemm_mxfp8_amd as gm
    monkeypatch.setattr(gm, "_lib", None)
    monkeypatch.setattr(gm, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        gm.lib()


def test_validate_offsets_on_host_crafted_arrays(mxlib):
    """The offsets check that MX_CHECK=1 runs on a copy of the device offsets:
    start at 0, never decrease, end at the row count."""
    import numpy as np

    def v(arr, M):
        a = np.ascontiguousarray(np.asarray(arr, dtype=np.int64))
        return mxlib.mx_validate_offsets(a.ctypes.data_as(ctypes.c_void_p), len(a) - 1, M)

    assert v([0, 3, 3, 10], 10) == MX_OK
    assert v([0, 0], 0) == MX_OK                        # one empty group
    assert v([0, 0, 0, 0], 0) == MX_OK
    assert v([1, 3, 10], 10) == MX_ERR_INVALID_ARG      # does not start at 0
    assert "offsets[0]" in _err(mxlib)
    assert v([0, 5, 4, 10], 10) == MX_ERR_INVALID_ARG   # decreases
    assert "decrease at group 1" in _err(mxlib)
    assert v([0, 3, 9], 10) == MX_ERR_INVALID_ARG       # does not end at M
    assert "expected the row count 10" in _err(mxlib)
    assert v([0, 3, 11], 10) == MX_ERR_INVALID_ARG
    assert v([0, -1, 10], 10) == MX_ERR_INVALID_ARG
    assert mxlib.mx_validate_offsets(None, 3, 10) == MX_ERR_INVALID_ARG
    rng = np.random.default_rng(1)
    for _ in range(100):
        counts = rng.integers(0, 50, int(rng.integers(1, 40)))
        off = np.concatenate([[0], np.cumsum(counts)])
        assert v(off, int(off[-1])) == MX_OK
        if len(counts) > 1 and counts.sum() > 0:
            i = int(rng.integers(1, len(off) - 1))
            bad = off.copy()
            bad[i] = off[-1] + 1                         # past the end: decreases after it
            assert v(bad, int(off[-1])) == MX_ERR_INVALID_ARG


def test_mlp_accepts_calls_past_two_gib_token_axis_copies(mxlib):
    """Descriptors are rebased per tile: M with 2F * Mp above 2^31 bytes (a
    token-axis copy of dh past 2 GiB) is accepted at the Mixtral shape; the
    limits are one expert's weights below 2^31 bytes and 65535 * 128 padded
    rows."""
    H, F = 4096, 14336
    for M, E in ((80000, 1), (1_000_000, 8), (8_388_480, 1)):
        Mp = mxlib.mx_padded_rows_bound(M, E, 128)
        assert 2 * F * Mp > 2 ** 31
        for fl in (0, SAVE_H):
            assert mxlib.grouped_mlp_ctx_bytes(M, H, F, E, fl) > 2 * F * Mp // 2
            assert mxlib.grouped_mlp_bwd_ws_bytes(M, H, F, E, fl) > 2 * F * Mp
    assert mxlib.grouped_mlp_ctx_bytes(8_388_481, H, F, 1, 0) == 0    # past the row bound
    assert "padded rows" in _err(mxlib)
    assert mxlib.grouped_mlp_ctx_bytes(1024, 32768, 32768, 1, 0) == 0  # 2F x H past 2^31
    assert "weights" in _err(mxlib)
