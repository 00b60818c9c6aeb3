"""GPU parity of the per-tensor FP8 path (quantizer and GroupedLinear)
against oracle/fp8_tensor.py.  Codes, amax and scale_inv bit-exact (both
sides take every rounding in fp32); the GEMM on the same codes within one
bf16 rounding plus the fp32 accumulation (the tighter stage-wise bar of the
MXFP8 GroupedLinear tests), and within the spec's bar against the oracle."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import fp8_tensor as P
from oracle import mx_oracle as O
from workloads import make_linear_case

pytestmark = pytest.mark.gpu


def bf16(rng, shape, std=1.0, outliers=0.0):
    v = rng.standard_normal(shape) * std
    if outliers:
        v = np.where(rng.random(shape) < outliers, v * 100.0, v)
    return torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)


def offsets_of(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def check_quant(q, x, offsets=None):
    """Bit-exact codes, amax and scale_inv (offsets start at row 0)."""
    codes, amax, sinv = P.quantize_groups(x.double().numpy(), offsets)
    got = q.codes.cpu().numpy()
    assert np.array_equal(got, codes)
    assert np.array_equal(q.amax.cpu().numpy().view(np.uint32), amax.view(np.uint32))
    assert np.array_equal(q.scale_inv.cpu().numpy().view(np.uint32), sinv.view(np.uint32))


@pytest.mark.parametrize("counts,C", [
    ([300, 0, 17, 129, 1, 553], 256), ([1000], 64), ([5, 0, 0, 7], 32),
    ([128] * 8, 1024), ([0, 0], 96),
])
def test_quantize_groups_matches_oracle(dev, counts, C):
    rng = np.random.default_rng(sum(counts) + C)
    offs = offsets_of(counts)
    x = bf16(rng, (int(offs[-1]), C), outliers=0.01)
    q = gm.fp8_tensor_quantize(x.to(dev), torch.from_numpy(offs).to(dev))
    torch.cuda.synchronize()
    check_quant(q, x, offs)


def test_quantize_many_groups_and_edge_values(dev):
    """1024 groups of 0..7 rows; one group all zero, one tiny (448 / amax
    overflows fp32), one with a single huge value."""
    rng = np.random.default_rng(7)
    counts = rng.integers(0, 8, size=1024)
    counts[3] = 5
    offs = offsets_of(counts)
    x = bf16(rng, (int(offs[-1]), 64)).float()
    x[offs[3]:offs[4]] = 0.0
    j = int(np.flatnonzero(counts > 0)[5])
    x[offs[j]:offs[j + 1]] = 2.0 ** -130
    k = int(np.flatnonzero(counts > 0)[9])
    x[offs[k], 3] = 3.0e38
    x = x.to(torch.bfloat16)
    q = gm.fp8_tensor_quantize(x.to(dev), torch.from_numpy(offs).to(dev))
    torch.cuda.synchronize()
    check_quant(q, x, offs)


def test_quantize_rows_outside_the_groups_are_left_alone(dev):
    rng = np.random.default_rng(9)
    offs = np.array([40, 100, 250], dtype=np.int64)       # rows [0, 40) and [250, 300) uncovered
    x = bf16(rng, (300, 128))
    q = gm.fp8_tensor_quantize(x.to(dev), torch.from_numpy(offs).to(dev))
    torch.cuda.synchronize()
    sub_offs = offs - offs[0]
    codes, amax, sinv = P.quantize_groups(x.double().numpy()[40:250], sub_offs)
    got = q.codes.cpu().numpy()
    assert np.array_equal(got[40:250], codes)
    assert np.array_equal(q.amax.cpu().numpy(), amax)
    assert np.array_equal(q.scale_inv.cpu().numpy(), sinv)


@pytest.mark.parametrize("G,R,C", [(4, 96, 128), (8, 1, 32), (3, 200, 160), (2, 0, 64)])
def test_quantize_matrices_matches_oracle(dev, G, R, C):
    rng = np.random.default_rng(G * R + C)
    w = bf16(rng, (G, R, C), std=0.02)
    q = gm.fp8_tensor_quantize(w.to(dev))
    torch.cuda.synchronize()
    check_quant(q, w)


def gemm_case(rng, counts, K, N, row_scale):
    offs = offsets_of(counts)
    M, E = int(offs[-1]), len(counts)
    x = bf16(rng, (M, K), outliers=0.01)
    w = bf16(rng, (E, N, K), std=0.02)
    r = torch.from_numpy(rng.random(M).astype(np.float32)) if row_scale else None
    return offs, x, w, r


@pytest.mark.parametrize("counts,K,N,row_scale", [
    ([300, 0, 17, 129, 1, 553], 256, 96, False), ([700, 300], 512, 320, True),
    ([1], 128, 32, False), ([257, 0, 0, 1000], 1024, 64, True),
    # K not a multiple of 128 (zero-padded copies)
    ([300, 17, 0, 44], 160, 96, True), ([513], 992, 64, False),
])
def test_grouped_linear_fp8_matches_oracle(dev, counts, K, N, row_scale):
    rng = np.random.default_rng(sum(counts) + K + N)
    offs, x, w, r = gemm_case(rng, counts, K, N, row_scale)
    od = torch.from_numpy(offs).to(dev)
    xq = gm.fp8_tensor_quantize(x.to(dev), od)
    wq = gm.fp8_tensor_quantize(w.to(dev))
    y = gm.grouped_linear_fwd_fp8(xq, od, wq, None if r is None else r.to(dev))
    torch.cuda.synchronize()
    got = y.double().cpu().numpy()
    rr = None if r is None else r.double().numpy()
    # stage-wise: the oracle's GEMM on the device's codes and scales
    ref_same = P.grouped_linear_fp8(xq.codes.cpu().numpy(), xq.scale_inv.cpu().numpy(),
                                    wq.codes.cpu().numpy(), wq.scale_inv.cpu().numpy(), offs, rr)
    rel, row = O.parity_metrics(got, ref_same)
    assert rel <= 4e-3 and row <= 3e-2, (rel, row)
    # end to end: the oracle quantizes the bf16 inputs itself
    xc, _, xs = P.quantize_groups(x.double().numpy(), offs)
    wc, _, ws = P.quantize_groups(w.double().numpy())
    ref = P.grouped_linear_fp8(xc, xs, wc, ws, offs, rr)
    rel, row = O.parity_metrics(got, ref)
    assert rel <= 1e-2 and row <= 5e-2, (rel, row)
    # and against the unquantized product (the FP8 error itself, for scale)
    exact = O.grouped_linear(x.double().numpy(), w.double().numpy(), offs, row_scale=rr)
    assert O.parity_metrics(got, exact)[0] < 0.1


def test_grouped_linear_fp8_full_size_sampled(dev):
    """The MXFP8 GroupedLinear workload (T=8192 top-2, E=8, K=1024, N=2816,
    1% outliers x100) in per-tensor FP8: all of amax / scale_inv, 64 sampled
    rows of codes, and 64 sampled rows of y against the oracle."""
    case = make_linear_case("mxfp8_linear", seed=0)
    offs = case.offsets.numpy()
    od = case.offsets.to(dev)
    xq = gm.fp8_tensor_quantize(case.X.to(dev), od)
    wq = gm.fp8_tensor_quantize(case.W.to(dev))
    y = gm.grouped_linear_fwd_fp8(xq, od, wq)
    torch.cuda.synchronize()
    x64 = case.X.double().numpy()
    amax = np.array([np.max(np.abs(x64[offs[e]:offs[e + 1]]), initial=0.0)
                     for e in range(len(offs) - 1)], dtype=np.float32)
    assert np.array_equal(xq.amax.cpu().numpy(), amax)
    sinv = np.array([P.tensor_scale(a)[1] for a in amax], dtype=np.float32)
    assert np.array_equal(xq.scale_inv.cpu().numpy(), sinv)
    _, wamax, wsinv = P.quantize_groups(case.W.double().numpy())
    assert np.array_equal(wq.amax.cpu().numpy(), wamax)
    assert np.array_equal(wq.scale_inv.cpu().numpy(), wsinv)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(len(x64), size=64, replace=False))
    grp = np.searchsorted(offs, rows, side="right") - 1
    xcodes = xq.codes.cpu().numpy()
    wcodes = wq.codes.cpu().numpy()
    got = y.double().cpu().numpy()[rows]
    ref = np.zeros_like(got)
    for i, (m, e) in enumerate(zip(rows, grp)):
        assert np.array_equal(xcodes[m], P.encode(x64[m], P.tensor_scale(amax[e])[0]))
        ref[i] = (O.e4m3_decode(xcodes[m]) @ O.e4m3_decode(wcodes[e]).T) * (
            float(sinv[e]) * float(wsinv[e]))
    wc_ref, _, _ = P.quantize_groups(case.W.double().numpy())
    assert np.array_equal(wcodes, wc_ref)
    rel, row = O.parity_metrics(got, ref)
    assert rel <= 4e-3 and row <= 3e-2, (rel, row)
