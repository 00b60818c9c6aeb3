"""GPU parity at the full sizes of the Mixtral-8x7B expert workload (T=16384
top-2, E=8, H=4096, F=14336, Zipf(1.1) loads, forward + backward) and of the
64-expert long-sequence workload (T=32768 top-8, E=64, H=2048, F=1408, 8
empty experts), run exactly as bench.py runs the headline workload: inputs
drawn on the GPU by the seeded generator, one grouped_mlp_fwd and one
grouped_mlp_bwd (recompute mode) on the library's default launch
configuration.

The FP64 oracle cannot run these sizes whole, so it runs on samples it can
compute exactly:

* stage-wise, at the spec's bar (relative Frobenius error <= 1e-2, max
  |err| / rms(reference row) <= 5e-2): each GEMM against the oracle's GEMM
  (FP64, dequantized operands) on the GPU's own MXFP8 codes, read back from
  ctx and the workspaces -- Y and dX on the sampled rows, the requantized z
  and dh codes (flip rate < 2e-3 against the oracle's SwiGLU forward and
  backward of the recomputed h), dr, and whole rows of dW1 and dW2: every
  row for small experts, 256-row slices (gate, up and tail rows) for the
  largest expert, whose weight gradients contract over its 13047 (31457)
  tokens, the longest K of the weight-gradient GEMMs.
* end to end (the oracle sees only the bf16 inputs, in worker processes
  while the GPU runs, see tests/_oracle_workers.py): whole experts and row
  subsets of the largest expert, with the end-to-end bars of
  test_gpu_mlp.py (max-row 0.1 for Y, dX and dr; weight gradients held to
  the Frobenius bar).

The Mixtral workload's split tail (the last round of output tiles of the
down GEMM and the gate-up dgrad, cut along K) falls in the last expert, which
is also the smallest and is compared whole.  Properties over the whole
output: every value finite, empty experts' weight gradients exactly zero."""
import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import mx_oracle as O
from tests._oracle_workers import expert_reference
from workloads import make_mlp_case

pytestmark = pytest.mark.gpu

REL_F, ROW_MAX, E2E_ROW_MAX = 1e-2, 5e-2, 0.1
FLIP_MAX = 2e-3
# exact value of every E4M3 code (the oracle's decode), for a fast gather
LUT = O.e4m3_decode(np.arange(256))


def deq(codes, scales):
    """The oracle's dequantization (code value times 2^(scale - 127) per
    block of 32 along the last axis) as a table lookup, float64."""
    codes = np.asarray(codes)
    v = LUT[codes].reshape(codes.shape[:-1] + (codes.shape[-1] // 32, 32))
    return (v * O.e8m0_decode(np.asarray(scales))[..., None]).reshape(codes.shape)


def rows_of(mx, lo, hi):
    """Codes and scales of rows [lo, hi) of a K-major MXFP8 view, on the CPU."""
    return mx.codes[lo:hi].cpu().numpy(), mx.scales[lo:hi].cpu().numpy()


def _np32(t):
    return t.float().cpu().numpy()


def _check(name, got, ref, row=ROW_MAX, rel=REL_F):
    r, worst = O.parity_metrics(np.asarray(got, dtype=np.float64), ref)
    print(f"    {name:26s} rel_fro={r:.3e} max_row={worst:.3e}", flush=True)
    assert r <= rel and worst <= row, (name, r, worst)


def _rate(name, mismatch):
    """Flipped requantized codes (boolean array): at most FLIP_MAX of them
    plus Poisson slack, as in test_gpu_mlp.py."""
    n = mismatch.size
    flips = int(np.count_nonzero(mismatch))
    limit = FLIP_MAX * n + 4.0 * np.sqrt(FLIP_MAX * n) + 3.0
    print(f"    {name:26s} {flips / n:.3e} ({flips} of {n}; at most {limit:.0f})", flush=True)
    assert flips <= limit, (name, flips, n)


def _jobs(case, samples):
    """End-to-end oracle inputs of each sample (label, expert, rows)."""
    off = case.offsets.cpu().numpy()
    out = []
    for label, e, rows, _ in samples:
        lo, hi = int(off[e]), int(off[e + 1])
        idx = np.arange(lo, hi) if rows is None else lo + np.asarray(rows)
        ti = torch.from_numpy(idx).to(case.X.device)
        out.append((label, e, rows is None, idx,
                    (_np32(case.X.index_select(0, ti)), _np32(case.W1[e]), _np32(case.W2[e]),
                     case.r.index_select(0, ti).cpu().numpy(), _np32(case.dY.index_select(0, ti)))))
    return out


def _stagewise(case, e, idx, wrows, views, outs):
    """Stage-wise checks of expert e on its sampled rows idx (global) and
    weight-gradient rows wrows (None: all rows)."""
    M, H, F = case.M, case.H, case.F
    y, dx, dw1, dw2, dr = outs
    v = views
    off = case.offsets.cpu().numpy()
    poff = v["poff"]
    lo, n = int(off[e]), int(off[e + 1] - off[e])
    p0 = int(poff[e])
    ti = torch.from_numpy(idx).to(y.device)
    sel = lambda mx: (mx.codes.index_select(0, ti).cpu().numpy(),
                      mx.scales.index_select(0, ti).cpu().numpy())
    r = case.r.index_select(0, ti).cpu().numpy().astype(np.float64)

    # forward: h = X W1^T on the GPU's codes (the recompute reads the same
    # codes), z requantized, Y = z W2^T
    h = deq(*sel(v["xrow"])) @ deq(*rows_of(v["w1row"], e * 2 * F, (e + 1) * 2 * F)).T
    a, b = h[:, :F], h[:, F:]
    sg = O.sigmoid(a)
    s = a * sg * b
    zc, zs = sel(v["zrow"])
    _rate("z flips", zc != O.quantize_lastdim(r[:, None] * s)[0])
    _check("Y | z codes", _np32(y.index_select(0, ti)),
           deq(zc, zs) @ deq(*rows_of(v["w2row"], e * H, (e + 1) * H)).T)
    # backward: dz = dY W2 on the GPU's codes, SwiGLU backward of the exact h
    dz = deq(*sel(v["dyrow"])) @ deq(*rows_of(v["w2col"], e * F, (e + 1) * F)).T
    _check("dr", dr.index_select(0, ti).cpu().numpy().astype(np.float64), (dz * s).sum(axis=1))
    ds = r[:, None] * dz
    dh = np.concatenate([ds * b * sg * (1.0 + a * (1.0 - sg)), ds * a * sg], axis=1)
    dhc, dhs = sel(v["dhrow"])
    _rate("dh flips", dhc != O.quantize_lastdim(dh)[0])
    _check("dX | dh codes", _np32(dx.index_select(0, ti)),
           deq(dhc, dhs) @ deq(*rows_of(v["w1col"], e * H, (e + 1) * H)).T)

    # weight gradients over the expert's whole token range, on the token-axis
    # codes (columns p0 .. p0 + n of the padded axis)
    if n == 0:
        return
    # p0 is a multiple of 128, so the expert's blocks start at column p0;
    # decode whole blocks of the padded range, then keep the n real tokens
    npad = (n + 31) // 32 * 32

    def tokvals(mx, rows):
        c = mx.codes[rows][:, p0:p0 + npad].cpu().numpy()
        s = mx.scales[rows][:, p0 // 32:(p0 + npad) // 32].cpu().numpy()
        return deq(c, s)[:, :n]

    all_h, all_f, all_2f = slice(0, H), slice(0, F), slice(0, 2 * F)
    w = wrows or {}
    r2, r1 = w.get("dW2", all_h), w.get("dW1", all_2f)
    # optional column slices, for token counts whose full FP64 operands would
    # not fit the host's memory
    c2, c1 = w.get("dW2_cols", all_f), w.get("dW1_cols", all_h)
    dyt = tokvals(v["dycol"], r2)                 # [rows of dW2, n]
    zt = tokvals(v["zcol"], c2)                   # [columns of dW2, n]
    _check(f"dW2[{e}] rows | codes", _np32(dw2[e][r2][:, c2]), dyt @ zt.T)
    del dyt, zt
    dht = tokvals(v["dhcol"], r1)                 # [rows of dW1, n]
    xt = tokvals(v["xcol"], c1)                   # [columns of dW1, n]
    _check(f"dW1[{e}] rows | codes", _np32(dw1[e][r1][:, c1]), dht @ xt.T)


def _run_full(dev, case, samples):
    M, H, F, E = case.M, case.H, case.F, case.E
    jobs = _jobs(case, samples)
    ctx_mp = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(len(jobs), 4), mp_context=ctx_mp) as pool:
        futs = [pool.submit(expert_reference, *args) for *_, args in jobs]
        print(f"full size M={M} H={H} F={F} E={E}: running the library", flush=True)
        # buffers start as 0xFF bytes: nothing unwritten may reach a result
        fws = torch.full((gm.fwd_ws_bytes(M, H, F, E),), 255, dtype=torch.uint8, device=dev)
        bws = torch.full((gm.bwd_ws_bytes(M, H, F, E),), 255, dtype=torch.uint8, device=dev)
        cbuf = torch.full((gm.ctx_bytes(M, H, F, E),), 255, dtype=torch.uint8, device=dev)
        y, ctx = gm.grouped_mlp_fwd(case.X, case.offsets, case.W1, case.W2, case.r, ws=fws,
                                    ctx_buf=cbuf)
        dx, dw1, dw2, dr = gm.grouped_mlp_bwd(case.dY, case.offsets, case.W1, case.W2, case.r,
                                              ctx, ws=bws)
        torch.cuda.synchronize()
        for t, name in ((y, "Y"), (dx, "dX"), (dw1, "dW1"), (dw2, "dW2"), (dr, "dr")):
            assert bool(torch.isfinite(t.float()).all()), f"{name} has non-finite values"
        for e in range(E):
            if int(case.counts[e]) == 0:
                assert not dw1[e].any() and not dw2[e].any(), f"empty expert {e}"
        print("  library outputs finite; empty experts' dW exactly zero", flush=True)
        Mp = ctx.padded_rows
        views = {"xrow": ctx.xrow(), "w1row": ctx.w1row(), "w2row": ctx.w2row(),
                 "w1col": ctx.w1col(), "w2col": ctx.w2col(), "xcol": ctx.xcol(),
                 "zcol": ctx.zcol(), "poff": ctx.padded_offsets().cpu().numpy(),
                 "zrow": gm.ws_mx_view(fws, gm.MX_WS_ZROW, M, H, F, E, (M, F)),
                 "dyrow": gm.ws_mx_view(bws, gm.MX_WS_DYROW, M, H, F, E, (M, H)),
                 "dycol": gm.ws_mx_view(bws, gm.MX_WS_DYCOL, M, H, F, E, (H, Mp)),
                 "dhrow": gm.ws_mx_view(bws, gm.MX_WS_DHROW, M, H, F, E, (M, 2 * F)),
                 "dhcol": gm.ws_mx_view(bws, gm.MX_WS_DHCOL, M, H, F, E, (2 * F, Mp))}
        outs = (y, dx, dw1, dw2, dr)
        for (label, e, whole, idx, _), (_, _, _, wrows), fut in zip(jobs, samples, futs):
            print(f" {label}: expert {e}, {len(idx)} rows", flush=True)
            print("  stage-wise (GPU codes)", flush=True)
            _stagewise(case, e, idx, wrows, views, outs)
            print("  end to end (bf16 inputs)", flush=True)
            Yr, dXr, drr, dW1r, dW2r = fut.result()
            ti = torch.from_numpy(idx).to(dev)
            _check("Y e2e", _np32(y.index_select(0, ti)), Yr, row=E2E_ROW_MAX)
            _check("dX e2e", _np32(dx.index_select(0, ti)), dXr, row=E2E_ROW_MAX)
            _check("dr e2e", dr.index_select(0, ti).cpu().numpy(), drr, row=E2E_ROW_MAX)
            if whole:
                _check("dW1[e] e2e", _np32(dw1[e]), dW1r, row=np.inf)
                _check("dW2[e] e2e", _np32(dw2[e]), dW2r, row=np.inf)


def _big_rows(n):
    return list(range(16)) + list(range(n // 2, n // 2 + 16)) + list(range(n - 32, n))


def _wslices(H, F):
    """256 rows of each weight gradient of the largest expert: the first and
    last 64 gate rows, the first and last 64 up rows of dW1 [2F, H]; the
    first, a middle and the last rows of dW2 [H, F]."""
    dw1 = np.r_[0:64, F - 64:F, F:F + 64, 2 * F - 64:2 * F]
    dw2 = np.r_[0:96, H // 2:H // 2 + 64, H - 96:H]
    return {"dW1": dw1, "dW2": dw2}


def test_mixtral_fwd_bwd_full_size(dev):
    case = make_mlp_case("mixtral_fwd_bwd", seed=0, device=dev)
    counts = [int(c) for c in case.counts]
    small, big = int(np.argmin(counts)), int(np.argmax(counts))
    # the split tail of the down GEMM and the gate-up dgrad is in the last
    # expert, the smallest one here, compared whole
    assert small == case.E - 1
    _run_full(dev, case, [("smallest expert, whole", small, None, None),
                          ("largest expert, 64 rows; dW row slices", big, _big_rows(counts[big]),
                           _wslices(case.H, case.F))])


def test_fine_grained_64e_full_size(dev):
    case = make_mlp_case("fine_grained_64e", seed=0, device=dev)
    counts = [int(c) for c in case.counts]
    assert sum(c == 0 for c in counts) == 8
    nz = [e for e in range(len(counts)) if counts[e] > 0]
    small = min(nz, key=lambda e: counts[e])
    big = max(nz, key=lambda e: counts[e])
    mid = sorted(nz, key=lambda e: counts[e])[len(nz) // 2]
    _run_full(dev, case, [("smallest expert, whole", small, None, None),
                          ("median expert, whole", mid, None, None),
                          ("largest expert, 64 rows; dW row slices", big,
                           _big_rows(counts[big]), _wslices(case.H, case.F))])


def test_mixtral_full_size_deterministic(dev):
    """Two runs of the Mixtral fwd+bwd at full size, the second with other
    buffers (fresh ctx and workspaces holding other bytes), give the same bits
    in every output: no atomics, fixed reduction orders."""
    case = make_mlp_case("mixtral_fwd_bwd", seed=0, device=dev)
    M, H, F, E = case.M, case.H, case.F, case.E
    outs = []
    for fill in (255, 0):
        fws = torch.full((gm.fwd_ws_bytes(M, H, F, E),), fill, dtype=torch.uint8, device=dev)
        bws = torch.full((gm.bwd_ws_bytes(M, H, F, E),), fill, dtype=torch.uint8, device=dev)
        cbuf = torch.full((gm.ctx_bytes(M, H, F, E),), fill, dtype=torch.uint8, device=dev)
        y, ctx = gm.grouped_mlp_fwd(case.X, case.offsets, case.W1, case.W2, case.r, ws=fws,
                                    ctx_buf=cbuf)
        g = gm.grouped_mlp_bwd(case.dY, case.offsets, case.W1, case.W2, case.r, ctx, ws=bws)
        torch.cuda.synchronize()
        outs.append((y,) + tuple(g))
        del fws, bws, cbuf, ctx
    for name, u, v in zip(("Y", "dX", "dW1", "dW2", "dr"), *outs):
        assert torch.equal(u, v), name
    print("  Mixtral fwd+bwd bitwise identical across two runs", flush=True)


def test_past_two_gib_token_axis_copies(dev):
    """One expert with 80,000 routed rows at H=4096, F=14336: the token-axis
    dh copy (2F x Mp bytes = 2.29e9) and dW1's contraction are past 2^31 bytes,
    which calls used to be refused for.  Stage-wise and end to end on 64 rows,
    and 256-row slices of dW1 and dW2 over 2048 of their columns, contracted
    over all 80,000 tokens."""
    n = 80000
    case = make_mlp_case(None, seed=5, T=n, k=1, E=1, H=4096, F=14336, routing="counts",
                         counts=[n], device=dev)
    assert 2 * case.F * gm.padded_rows_bound(n, 1) > 2 ** 31
    w = _wslices(case.H, case.F)
    w["dW2_cols"] = np.r_[0:1024, case.F - 1024:case.F]
    w["dW1_cols"] = np.r_[0:1024, case.H - 1024:case.H]
    _run_full(dev, case, [("80,000-row expert, 64 rows; dW row slices", 0, _big_rows(n), w)])
