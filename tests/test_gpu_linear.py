"""GPU parity of GroupedLinear (BF16 and MXFP8) against the FP64 oracle.

Bar: relative Frobenius error <= 1e-2 and max |err| / rms(reference row)
<= 5e-2.  The MXFP8 path is also checked stage-wise: the oracle's GEMM on the
very codes the GPU produced (exact in FP64) against the GPU output, where the
only differences are fp32 accumulation and the final bf16 rounding (at most
2^-9 of |y|, i.e. about 2e-3 in Frobenius norm and up to a few 1e-2 of a
row's RMS for the largest entries), hence the tighter 4e-3 / 3e-2 there."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import mx_oracle as O
from workloads import make_linear_case

pytestmark = pytest.mark.gpu

REL_F, ROW_MAX = 1e-2, 5e-2


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def deq(mx: gm.MxTensor):
    return O.dequantize_lastdim(mx.codes.cpu().numpy(), mx.scales.cpu().numpy())


def assert_parity(got, ref, rel=REL_F, row=ROW_MAX):
    r, w = O.parity_metrics(got, ref)
    assert r <= rel and w <= row, (r, w)
    return r, w


def test_tiny_bf16_linear(dev):
    """T=256 top-2, E=4, K=128, N=256, BF16 (no quantization)."""
    case = make_linear_case("tiny_bf16_linear", seed=0)
    off = case.offsets.to(dev)
    y = gm.grouped_linear_fwd(case.X.to(dev), off, case.W.to(dev))
    torch.cuda.synchronize()
    ref = O.grouped_linear(to64(case.X), to64(case.W), case.offsets.numpy())
    r, w = assert_parity(to64(y), ref)
    assert r < 5e-3        # only the bf16 output rounding differs
    yr = gm.grouped_linear_fwd(case.X.to(dev), off, case.W.to(dev), row_scale=case.r.to(dev))
    torch.cuda.synchronize()
    ref_r = O.grouped_linear(to64(case.X), to64(case.W), case.offsets.numpy(),
                             row_scale=case.r.numpy())
    assert_parity(to64(yr), ref_r)


def test_bf16_grouped_equals_per_expert_loop(dev):
    rng = np.random.default_rng(3)
    counts = [0, 70, 1, 0, 129, 64]
    off_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M, K, N, E = off_np[-1], 96, 80, len(counts)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((E, N, K)).astype(np.float32) * 0.1).to(torch.bfloat16)
    y = gm.grouped_linear_fwd(x.to(dev), torch.from_numpy(off_np).to(dev), w.to(dev))
    torch.cuda.synchronize()
    for e in range(E):
        lo, hi = off_np[e], off_np[e + 1]
        if hi == lo:
            continue
        ye = gm.grouped_linear_fwd(x[lo:hi].contiguous().to(dev),
                                   torch.tensor([0, hi - lo], dtype=torch.int64, device=dev),
                                   w[e:e + 1].contiguous().to(dev))
        torch.cuda.synchronize()
        assert torch.equal(ye, y[lo:hi])


def _mx_case(dev, counts, K, N, seed, outliers=False):
    rng = np.random.default_rng(seed)
    off_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M, E = int(off_np[-1]), len(counts)
    xf = rng.standard_normal((M, K))
    if outliers:
        xf[rng.random((M, K)) < 0.01] *= 100.0
    x = torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)).to(
        torch.bfloat16)
    return x, w, off_np


@pytest.mark.parametrize("counts,K,N", [
    ([256], 128, 256),                       # one full tile
    ([300, 0, 17, 511], 256, 320),           # ragged M tails, an empty expert, N tail
    ([0, 0, 1, 0], 384, 64),                 # a single row
    ([1000, 2000, 3], 512, 544),
    # K not a multiple of the 128-wide K step: zero-padded copies
    ([300, 0, 17, 511], 96, 320),
    ([1000, 5, 700], 544, 256),
    ([64, 129], 1056, 64),
])
def test_mxfp8_linear_small(dev, counts, K, N):
    x, w, off_np = _mx_case(dev, counts, K, N, seed=K + N, outliers=True)
    off = torch.from_numpy(off_np).to(dev)
    xq = gm.mxfp8_quantize(x.to(dev), rowwise=True)["row"]
    wq = gm.mxfp8_quantize(w.to(dev), rowwise=True)["row"]
    r = torch.rand(x.shape[0], generator=torch.Generator().manual_seed(1)).to(dev)
    y = gm.grouped_linear_fwd(xq, off, wq)
    ys = gm.grouped_linear_fwd(xq, off, wq, row_scale=r)
    torch.cuda.synchronize()
    # stage-wise: the oracle's GEMM on the GPU's own codes
    stage = O.grouped_linear(deq(xq), deq(wq), off_np)
    assert_parity(to64(y), stage, rel=4e-3, row=3e-2)
    # end to end: the oracle quantizes bf16 inputs itself
    ref = O.grouped_linear_mxfp8(to64(x), to64(w), off_np)
    assert_parity(to64(y), ref)
    ref_s = O.grouped_linear_mxfp8(to64(x), to64(w), off_np, row_scale=r.cpu().numpy())
    assert_parity(to64(ys), ref_s)


@pytest.mark.parametrize("K", [128, 256, 384])
def test_mxfp8_linear_chained_tiles(dev, K):
    """More tiles than workgroups (273 M-tiles x 2 N-tiles = 546 tiles on 256
    workgroups), so each workgroup runs a chain of tiles whose last K steps
    fetch the next tile's first ones; K = 128, 256, 384 are 1, 2 and 3 K
    steps (a chain link needs two)."""
    counts = [40000, 37, 0, 29000, 5]
    x, w, off_np = _mx_case(dev, counts, K, 512, seed=K, outliers=True)
    off = torch.from_numpy(off_np).to(dev)
    xq = gm.mxfp8_quantize(x.to(dev), rowwise=True)["row"]
    wq = gm.mxfp8_quantize(w.to(dev), rowwise=True)["row"]
    r = torch.rand(x.shape[0], generator=torch.Generator().manual_seed(2)).to(dev)
    y = gm.grouped_linear_fwd(xq, off, wq)
    ys = gm.grouped_linear_fwd(xq, off, wq, row_scale=r)
    torch.cuda.synchronize()
    stage = O.grouped_linear(deq(xq), deq(wq), off_np)
    assert_parity(to64(y), stage, rel=4e-3, row=3e-2)
    assert_parity(to64(ys), stage * r.cpu().numpy().astype(np.float64)[:, None],
                  rel=4e-3, row=3e-2)
    ref = O.grouped_linear_mxfp8(to64(x), to64(w), off_np)
    assert_parity(to64(y), ref)


def test_mxfp8_linear_full_workload(dev):
    """T=8192 top-2 (M=16384), E=8, K=1024, N=2816 with 1% outliers, the
    launch bench.py times for this workload."""
    case = make_linear_case("mxfp8_linear", seed=0)
    off = case.offsets.to(dev)
    xq = gm.mxfp8_quantize(case.X.to(dev), rowwise=True)["row"]
    wq = gm.mxfp8_quantize(case.W.to(dev), rowwise=True)["row"]
    y = gm.grouped_linear_fwd(xq, off, wq)
    torch.cuda.synchronize()
    ref = O.grouped_linear_mxfp8(to64(case.X), to64(case.W), case.offsets.numpy())
    assert_parity(to64(y), ref)


def test_mxfp8_linear_deterministic(dev):
    x, w, off_np = _mx_case(dev, [700, 300], 256, 256, seed=5)
    off = torch.from_numpy(off_np).to(dev)
    xq = gm.mxfp8_quantize(x.to(dev), rowwise=True)["row"]
    wq = gm.mxfp8_quantize(w.to(dev), rowwise=True)["row"]
    a = gm.grouped_linear_fwd(xq, off, wq)
    b = gm.grouped_linear_fwd(xq, off, wq)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
