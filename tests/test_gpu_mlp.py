"""GPU parity of the fused GroupedMLP forward and backward against the FP64
oracle, at sizes the oracle finishes in seconds that still span several
tiles, ragged tails and empty experts.

Stage-wise bar (each GEMM against the oracle's GEMM on the same quantized
operands, the GPU's own codes): relative Frobenius error <= 1e-2 and
max |err| / rms(reference row) <= 5e-2, for h, Y, dX, dW1, dW2 (rows of the
stored matrices) and dr (one row).  Rows whose reference is exactly zero must
be exactly zero.

The intermediates z and dh are requantized from fp32 values on the GPU and
from fp64 values in the oracle; a value that sits next to an E4M3 rounding
boundary can land on the neighbouring code (the scaled FP8 MFMA accumulates
a little less exactly than fp32: the GPU's dz differs from the exact one by
~1e-5 relative, see the dr check).  The flip rate is bounded (< 2e-3), and
end to end (oracle fed only the bf16 inputs) the relative Frobenius bar of
1e-2 still holds, with a wider max-row bound of 0.1 because one flipped code
moves a whole output row by a few 1e-2 of its RMS.  The flip bound is a bound
on the probability of a flip: the count of flipped codes may exceed 2e-3 of
the codes by Poisson counting noise (four standard deviations plus three
codes), which matters for small experts only."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import mx_oracle as O
from workloads import make_mlp_case

pytestmark = pytest.mark.gpu

REL_F, ROW_MAX = 1e-2, 5e-2
E2E_ROW_MAX = 0.1
FLIP_MAX = 2e-3


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def deq(mx, n=None):
    c, s = mx.codes.cpu().numpy(), mx.scales.cpu().numpy()
    if n is not None:
        c, s = c[:, :n], s[:, : n // 32]
    return O.dequantize_lastdim(c, s)


class Report:
    def __init__(self):
        self.fails = []

    def check(self, name, got, ref, rel=REL_F, row=ROW_MAX):
        r, w = O.parity_metrics(got, ref)
        ok = r <= rel and w <= row
        print(f"  {name:10s} rel_fro={r:.3e} max_row={w:.3e} {'ok' if ok else 'FAIL'}",
              flush=True)
        if not ok:
            self.fails.append((name, r, w))

    def rate(self, name, mismatch, bound):
        """Requantized codes that differ from the oracle's (a boolean array):
        their probability is bounded by ``bound``; the count is held to that
        rate plus Poisson slack (four standard deviations and three codes),
        so that small samples are not failed by counting noise."""
        n = mismatch.size
        flips = int(np.count_nonzero(mismatch))
        limit = bound * n + 4.0 * np.sqrt(bound * n) + 3.0
        ok = flips <= limit
        print(f"  {name:10s} {flips / max(n, 1):.3e} ({flips} of {n}; at most {limit:.0f}) "
              f"{'ok' if ok else 'FAIL'}", flush=True)
        if not ok:
            self.fails.append((name, flips, n))

    def done(self):
        assert not self.fails, self.fails


def tok_rows(colmx, off_np, poff, n_rows):
    """[M, C] values of a token-axis copy (codes [C, Mp]) in row order."""
    full = deq(colmx, int(poff[-1]))
    out = np.zeros((n_rows, full.shape[0]))
    for e in range(len(off_np) - 1):
        n = off_np[e + 1] - off_np[e]
        out[off_np[e]:off_np[e + 1]] = full[:, poff[e]:poff[e] + n].T
    return out


def run_case(dev, case, save_h=False, reuse_from=None):
    """Forward and backward of ``case`` on the GPU, checked stage by stage
    and end to end against the oracle.  save_h: the save-h mode (h stored as
    bf16; the oracle's h_bf16 mode), else the recompute mode.  reuse_from:
    another case with the same weights whose forward runs first into the same
    ctx; this case's forward then reuses the weight copies it left there."""
    M, H, F, E = case.M, case.H, case.F, case.E
    off_np = case.offsets.numpy()
    poff = O.padded_offsets(off_np)
    x, w1, w2 = case.X.to(dev), case.W1.to(dev), case.W2.to(dev)
    r, off, dy = case.r.to(dev), case.offsets.to(dev), case.dY.to(dev)
    Mb = max(M, reuse_from.M) if reuse_from is not None else M
    # Workspaces and ctx start as 0xFF bytes (E8M0 NaN scales, E4M3 NaN
    # codes): anything the library reads without having written it shows.
    fws = torch.full((gm.fwd_ws_bytes(Mb, H, F, E, save_h),), 255, dtype=torch.uint8, device=dev)
    bws = torch.full((gm.bwd_ws_bytes(M, H, F, E, save_h),), 255, dtype=torch.uint8, device=dev)
    cbuf = torch.full((gm.ctx_bytes(Mb, H, F, E, save_h),), 255, dtype=torch.uint8, device=dev)
    if reuse_from is not None:
        a = reuse_from
        gm.grouped_mlp_fwd(a.X.to(dev), a.offsets.to(dev), w1, w2, a.r.to(dev), ws=fws,
                           ctx_buf=cbuf, save_h=save_h)
    y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws, ctx_buf=cbuf, save_h=save_h,
                                reuse_weights=reuse_from is not None)
    dx, dw1, dw2, dr = gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx, ws=bws)
    torch.cuda.synchronize()
    print(f"case M={M} H={H} F={F} E={E} counts={list(case.counts)} "
          f"mode={'save-h' if save_h else 'recompute'}"
          f"{' reusing weights' if reuse_from is not None else ''}", flush=True)

    X64, W164, W264, dY64 = to64(case.X), to64(case.W1), to64(case.W2), to64(case.dY)
    r64 = case.r.numpy().astype(np.float64)
    rep = Report()
    assert np.array_equal(ctx.padded_offsets().cpu().numpy(), poff)

    # ---- quantized copies of the bf16 inputs: bit-exact ----
    n = int(poff[-1])
    xc_o, xs_o, _ = O.quantize_tokens(X64, off_np)
    assert np.array_equal(ctx.xcol().codes.cpu().numpy()[:, :n], xc_o)
    assert np.array_equal(ctx.xcol().scales.cpu().numpy()[:, : n // 32], xs_o)
    if not save_h:
        # the rowwise X copy the backward recomputes h from
        c_ref, s_ref = O.quantize_lastdim(X64)
        assert np.array_equal(ctx.xrow().codes.cpu().numpy(), c_ref)
        assert np.array_equal(ctx.xrow().scales.cpu().numpy(), s_ref)
    # the weights' copies the forward saved: rowwise (blocks along H for W1,
    # along F for W2) and columnwise (blocks along 2F for W1, along H for W2)
    for got, w64 in ((ctx.w1row(), W164), (ctx.w2row(), W264),
                     (ctx.w1col(), W164.transpose(0, 2, 1)),
                     (ctx.w2col(), W264.transpose(0, 2, 1))):
        c_ref, s_ref = O.quantize_lastdim(w64)
        assert np.array_equal(got.codes.cpu().numpy(), c_ref.reshape(-1, c_ref.shape[-1]))
        assert np.array_equal(got.scales.cpu().numpy(), s_ref.reshape(-1, s_ref.shape[-1]))
    # the backward's dY copies: rowwise (dgrad) and token-axis (dW2)
    dyrow = gm.ws_mx_view(bws, gm.MX_WS_DYROW, M, H, F, E, (M, H), save_h)
    c_ref, s_ref = O.quantize_lastdim(dY64)
    assert np.array_equal(dyrow.codes.cpu().numpy(), c_ref)
    assert np.array_equal(dyrow.scales.cpu().numpy(), s_ref)
    dycol = gm.ws_mx_view(bws, gm.MX_WS_DYCOL, M, H, F, E, (H, ctx.padded_rows), save_h)
    c_ref, s_ref, _ = O.quantize_tokens(dY64, off_np)
    assert np.array_equal(dycol.codes.cpu().numpy()[:, :n], c_ref)
    assert np.array_equal(dycol.scales.cpu().numpy()[:, : n // 32], s_ref)

    # ---- forward, stage by stage ----
    qX, qW1, qW2 = O.qdq_lastdim(X64), O.qdq_lastdim(W164), O.qdq_lastdim(W264)
    h_ref = O.grouped_linear(qX, qW1, off_np)
    if save_h:
        h_gpu = to64(ctx.h())
        rep.check("h", h_gpu, h_ref)
    zrow = gm.ws_mx_view(fws, gm.MX_WS_ZROW, M, H, F, E, (M, F), save_h)
    rep.check("Y|z_gpu", to64(y), O.grouped_linear(deq(zrow), qW2, off_np))
    a, b = h_ref[:, :F], h_ref[:, F:]
    z_ref = r64[:, None] * a * O.sigmoid(a) * b
    rep.rate("z flips", zrow.codes.cpu().numpy() != O.quantize_lastdim(z_ref)[0], FLIP_MAX)
    rep.rate("zcol flips", ctx.zcol().codes.cpu().numpy()[:, :n]
             != O.quantize_tokens(z_ref, off_np)[0], FLIP_MAX)

    # ---- backward, stage by stage (on the GPU's own codes; the SwiGLU
    # backward on the h the GPU reads: bf16 saved h, or the exact h it
    # recomputes from the same codes) ----
    dz_ref = O.grouped_linear(O.qdq_lastdim(dY64), O.qdq_lastdim(W264.transpose(0, 2, 1)),
                              off_np)
    h_bwd = h_gpu if save_h else h_ref
    ag, bg = h_bwd[:, :F], h_bwd[:, F:]
    sg = O.sigmoid(ag)
    s_bwd = ag * sg * bg
    rep.check("dr", dr.cpu().numpy().astype(np.float64), (dz_ref * s_bwd).sum(axis=1))
    ds = r64[:, None] * dz_ref
    dh_ref = np.concatenate([ds * bg * sg * (1.0 + ag * (1.0 - sg)), ds * ag * sg], axis=1)
    dhrow = gm.ws_mx_view(bws, gm.MX_WS_DHROW, M, H, F, E, (M, 2 * F), save_h)
    rep.rate("dh flips", dhrow.codes.cpu().numpy() != O.quantize_lastdim(dh_ref)[0], FLIP_MAX)
    rep.check("dX|dh_gpu", to64(dx),
              O.grouped_linear(deq(dhrow), O.qdq_lastdim(W164.transpose(0, 2, 1)), off_np))
    dycol_rows = O.qdq_tokens(dY64, off_np)
    zt = tok_rows(ctx.zcol(), off_np, poff, M)
    dhcol = gm.ws_mx_view(bws, gm.MX_WS_DHCOL, M, H, F, E, (2 * F, ctx.padded_rows), save_h)
    rep.rate("dhcol flips", dhcol.codes.cpu().numpy()[:, :n]
             != O.quantize_tokens(dh_ref, off_np)[0], FLIP_MAX)
    dht = tok_rows(dhcol, off_np, poff, M)
    xt = O.qdq_tokens(X64, off_np)
    dW2_ref = np.zeros((E, H, F))
    dW1_ref = np.zeros((E, 2 * F, H))
    for e in range(E):
        lo, hi = off_np[e], off_np[e + 1]
        dW2_ref[e] = dycol_rows[lo:hi].T @ zt[lo:hi]
        dW1_ref[e] = dht[lo:hi].T @ xt[lo:hi]
    rep.check("dW2|z_gpu", to64(dw2), dW2_ref)
    rep.check("dW1|dh_gpu", to64(dw1), dW1_ref)
    for e in range(E):
        if case.counts[e] == 0:
            assert not dw1[e].any() and not dw2[e].any()

    # ---- end to end: the oracle sees only the bf16 inputs ----
    Yo, saved = O.grouped_mlp_fwd(X64, W164, W264, r64, off_np)
    go = O.grouped_mlp_bwd(dY64, X64, W164, W264, r64, off_np, saved, h_bf16=save_h)
    rep.check("Y e2e", to64(y), Yo, row=E2E_ROW_MAX)
    rep.check("dX e2e", to64(dx), go["dX"], row=E2E_ROW_MAX)
    # Weight gradients contract over one expert's tokens, which are
    # requantized along the token axis: when a 32-token block's amax sits next
    # to a power of two, fp32 and fp64 pick different block scales and all 32
    # codes move, shifting single elements of dW by up to ~1/sqrt(tokens) of
    # their row's RMS.  End to end they are held to the Frobenius bar per
    # expert (experts with >= 64 tokens); every element is covered by the
    # stage-wise check above.  The max-row figure is printed for the record.
    rep.check("dW1 e2e", to64(dw1), go["dW1"], row=np.inf)
    rep.check("dW2 e2e", to64(dw2), go["dW2"], row=np.inf)
    for e in range(E):
        if case.counts[e] >= 64:
            rep.check(f"dW1[{e}] e2e", to64(dw1[e]), go["dW1"][e], row=np.inf)
            rep.check(f"dW2[{e}] e2e", to64(dw2[e]), go["dW2"][e], row=np.inf)
    rep.check("dr e2e", dr.cpu().numpy().astype(np.float64), go["dr"], row=E2E_ROW_MAX)
    rep.done()
    return y, dx, dw1, dw2, dr


def small_case(counts, H, F, seed=0):
    """Token-sorted case with exact per-expert counts (top-2 routing, so no
    expert may hold more than half of the rows)."""
    k = 2
    M = sum(counts)
    T = (M + k - 1) // k
    if T * k != M:
        counts = list(counts)
        counts[-1] += T * k - M
    return make_mlp_case(None, seed=seed, T=T, k=k, E=len(counts), H=H, F=F,
                         routing="counts", counts=counts)


MODES = [pytest.param(False, id="recompute"), pytest.param(True, id="save_h")]


@pytest.mark.parametrize("save_h", MODES)
@pytest.mark.parametrize("counts,H,F", [
    ([300, 0, 257, 143], 256, 384),          # F/256 not integral: masked dz tiles (save-h)
    ([1, 33, 0, 250, 95, 0, 129, 6], 512, 256),
    ([600, 600], 384, 128),
    # 17 M-tiles x 16 F-tiles = 272 tiles: two per workgroup for some; K = H = 128
    # is one K step (the recompute backward's dz GEMM then runs its own prologue)
    ([2000, 1500, 700], 128, 2048),
])
def test_mlp_small(dev, counts, H, F, save_h):
    run_case(dev, small_case(counts, H, F, seed=H + F), save_h=save_h)


@pytest.mark.parametrize("save_h", MODES)
def test_mlp_zipf_scaled_down(dev, save_h):
    """Zipf(1.1) loads over 8 experts as in the Mixtral-shape workload, with
    T=2048 tokens, H=1024, F=1024."""
    case = make_mlp_case(None, seed=0, T=2048, k=2, E=8, H=1024, F=1024, routing="zipf",
                         zipf_s=1.1)
    run_case(dev, case, save_h=save_h)


def test_mlp_zero_routing_weight_rows(dev):
    case = small_case([200, 100, 100], 256, 256, seed=3)
    case.r[7] = 0.0
    case.r[250] = 0.0
    y, dx, dw1, dw2, dr = run_case(dev, case)
    assert not y[7].any() and not y[250].any()
    assert not dx[7].any()


@pytest.mark.parametrize("save_h", MODES)
def test_mlp_deterministic(dev, save_h):
    case = small_case([250, 200, 62], 256, 256, seed=4)
    a = run_case(dev, case, save_h=save_h)
    b = run_case(dev, case, save_h=save_h)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("save_h", MODES)
def test_mlp_zero_dy_gives_zero_gradients(dev, save_h):
    case = small_case([130, 70, 60], 256, 128, seed=5)
    case.dY.zero_()
    x, w1, w2 = case.X.to(dev), case.W1.to(dev), case.W2.to(dev)
    r, off, dy = case.r.to(dev), case.offsets.to(dev), case.dY.to(dev)
    y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, save_h=save_h)
    dx, dw1, dw2, dr = gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx)
    torch.cuda.synchronize()
    for t in (dx, dw1, dw2, dr):
        assert not t.any()


def test_recompute_and_save_h_agree_within_the_bar(dev):
    """The two modes differ only in the h the SwiGLU backward reads (exact
    fp32 accumulator vs its bf16 rounding): outputs agree within the
    end-to-end bar, the forward is identical."""
    case = small_case([300, 0, 257, 143], 256, 384, seed=9)
    x, w1, w2 = case.X.to(dev), case.W1.to(dev), case.W2.to(dev)
    r, off, dy = case.r.to(dev), case.offsets.to(dev), case.dY.to(dev)
    out = {}
    for sh in (False, True):
        y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, save_h=sh)
        out[sh] = (y,) + tuple(gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx))
    torch.cuda.synchronize()
    assert torch.equal(out[False][0], out[True][0])
    for name, u, v in zip(("dX", "dW1", "dW2", "dr"), out[False][1:], out[True][1:]):
        rel, _ = O.parity_metrics(to64(u), to64(v))
        print(f"  {name} recompute vs save-h rel_fro={rel:.3e}", flush=True)
        assert rel <= 3e-2, name


@pytest.mark.parametrize("save_h", MODES)
def test_mlp_reuse_weights_against_oracle(dev, save_h):
    """A forward that reuses the weight copies an earlier forward (another
    batch with another M, same weights) left in its ctx: every stage-wise and
    end-to-end check against the oracle, and the same bits as a forward that
    quantizes the weights itself, backward included."""
    H, F = 256, 384
    a = small_case([300, 0, 257, 143], H, F, seed=11)
    b = small_case([110, 40, 0, 78], H, F, seed=12)
    b.W1, b.W2 = a.W1, a.W2
    g_re = run_case(dev, b, save_h=save_h, reuse_from=a)
    xb, offb, rb, dyb = b.X.to(dev), b.offsets.to(dev), b.r.to(dev), b.dY.to(dev)
    w1, w2 = b.W1.to(dev), b.W2.to(dev)
    y_fr, ctx_fr = gm.grouped_mlp_fwd(xb, offb, w1, w2, rb, save_h=save_h)
    g_fr = (y_fr,) + tuple(gm.grouped_mlp_bwd(dyb, offb, w1, w2, rb, ctx_fr))
    torch.cuda.synchronize()
    for u, v in zip(g_re, g_fr):
        assert torch.equal(u, v)


@pytest.mark.parametrize("save_h", MODES)
def test_mlp_empty_batch(dev, save_h):
    """No routed rows at all (M = 0, every expert empty): the forward only
    quantizes the weights, the backward's weight gradients are exact zeros
    (outputs start poisoned)."""
    H, F, E = 256, 128, 3
    g = torch.Generator().manual_seed(7)
    w1 = (torch.randn((E, 2 * F, H), generator=g) * 0.02).to(torch.bfloat16).to(dev)
    w2 = (torch.randn((E, H, F), generator=g) * 0.02).to(torch.bfloat16).to(dev)
    x = torch.empty((0, H), dtype=torch.bfloat16, device=dev)
    r = torch.empty((0,), dtype=torch.float32, device=dev)
    off = torch.zeros(E + 1, dtype=torch.int64, device=dev)
    y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, save_h=save_h)
    dx, dw1, dw2, dr = gm.grouped_mlp_bwd(x, off, w1, w2, r, ctx)
    torch.cuda.synchronize()
    assert y.shape == (0, H) and dx.shape == (0, H) and dr.shape == (0,)
    assert not dw1.any() and not dw2.any()
    c_ref, s_ref = O.quantize_lastdim(to64(w1))
    assert np.array_equal(ctx.w1row().codes.cpu().numpy(), c_ref.reshape(-1, H))
