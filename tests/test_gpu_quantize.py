"""GPU parity of the MXFP8 quantizer: codes and scales bit-exact against the
FP64 oracle, rowwise and columnwise (token-axis, per-expert padded) copies."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import mx_oracle as O
from workloads import make_linear_case

pytestmark = pytest.mark.gpu


def bf16_from_bits(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def all_finite_bf16_bits():
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return b[np.isfinite(f)].astype(np.uint16)


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def exhaustive_blocks(seed):
    """Every finite bf16 pattern, shuffled into 32-blocks, plus copies whose
    blocks are anchored by a large, a unit and a tiny amax so each value is
    also quantized under very different shared scales."""
    rng = np.random.default_rng(seed)
    bits = all_finite_bf16_bits()
    parts = []
    for anchor in (None, 0x4380, 0x3f80, 0x0100, 0x7f7f):   # 256, 1, tiny, max
        b = rng.permutation(bits)
        b = b[: len(b) // 32 * 32].reshape(-1, 32)
        if anchor is not None:
            b = b.copy()
            b[:, 0] = anchor
        parts.append(b)
    blocks = np.concatenate(parts)
    blocks = blocks[: len(blocks) // 8 * 8]
    return blocks.reshape(-1, 256)          # rows of 256 values = 8 blocks


def test_rowwise_exhaustive_bf16(dev):
    bits = exhaustive_blocks(0)
    x = bf16_from_bits(bits).to(dev)
    out = gm.mxfp8_quantize(x, rowwise=True)
    torch.cuda.synchronize()
    codes, scales = O.quantize_lastdim(to64(x))
    assert np.array_equal(out["row"].codes.cpu().numpy(), codes)
    assert np.array_equal(out["row"].scales.cpu().numpy(), scales)


def test_tile_pass_rowwise_matches_flat_pass(dev):
    bits = exhaustive_blocks(1)[:4096]
    x = bf16_from_bits(bits).to(dev)
    a = gm.mxfp8_quantize(x, rowwise=True)["row"]
    b = gm.mxfp8_quantize(x, rowwise=True, colwise=True)["row"]
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


def test_columnwise_exhaustive_bf16(dev):
    bits = exhaustive_blocks(2)[:1216, :128]                 # [1216, 128]
    x = bf16_from_bits(np.ascontiguousarray(bits.T)).to(dev)     # blocks run down columns
    x = x.contiguous()
    R = x.shape[0]
    out = gm.mxfp8_quantize(x, rowwise=False, colwise=True)
    torch.cuda.synchronize()
    off = np.array([0, R])
    codes, scales, poff = O.quantize_tokens(to64(x), off, align=128)
    n = int(poff[-1])
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], codes)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], scales)


@pytest.mark.parametrize("counts", [
    [0, 1, 31, 32, 33, 0, 127, 128, 129, 300],
    [0, 0, 5],
    [257, 0, 0, 1000, 64],
    [1] * 40,
])
def test_grouped_token_axis(dev, counts):
    rng = np.random.default_rng(sum(counts))
    M, C = sum(counts), 192
    xf = rng.standard_normal((M, C)) * np.exp(rng.uniform(-8, 8, (M, 1)))
    xf[rng.random((M, C)) < 0.01] *= 100.0
    x = torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16).to(dev)
    off_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    off = torch.from_numpy(off_np).to(dev)
    out = gm.mxfp8_quantize(x, rowwise=True, colwise=True, offsets=off)
    torch.cuda.synchronize()
    x64 = to64(x)
    codes, scales, poff = O.quantize_tokens(x64, off_np, align=128)
    n = int(poff[-1])
    assert np.array_equal(out["padded_offsets"].cpu().numpy(), poff)
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], codes)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], scales)
    rc, rs = O.quantize_lastdim(x64)
    assert np.array_equal(out["row"].codes.cpu().numpy(), rc)
    assert np.array_equal(out["row"].scales.cpu().numpy(), rs)


@pytest.mark.parametrize("R,C", [(200, 96), (1, 32), (129, 224), (256, 64)])
def test_tile_pass_ragged_shapes(dev, R, C):
    """One tile pass (rowwise + token-axis) on shapes with a ragged last row
    tile, a half-used last column tile and an odd number of scale blocks."""
    rng = np.random.default_rng(R * 1000 + C)
    xf = rng.standard_normal((R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))
    x = torch.from_numpy(xf.astype(np.float32)).to(torch.bfloat16).to(dev)
    out = gm.mxfp8_quantize(x, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    x64 = to64(x)
    rc, rs = O.quantize_lastdim(x64)
    assert np.array_equal(out["row"].codes.cpu().numpy(), rc)
    assert np.array_equal(out["row"].scales.cpu().numpy(), rs)
    codes, scales, poff = O.quantize_tokens(x64, np.array([0, R]), align=128)
    n = int(poff[-1])
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], codes)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], scales)


def test_batched_columnwise_weights(dev):
    rng = np.random.default_rng(7)
    E, R, C = 3, 384, 160
    w = torch.from_numpy((rng.standard_normal((E, R, C)) * 0.02).astype(np.float32)).to(
        torch.bfloat16).to(dev)
    out = gm.mxfp8_quantize(w, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    w64 = to64(w)
    for e in range(E):
        codes, scales = O.quantize_lastdim(w64[e].T)
        assert np.array_equal(out["col"].codes[e].cpu().numpy()[:, :R], codes)
        assert np.array_equal(out["col"].scales[e].cpu().numpy()[:, : R // 32], scales)
        rc, rs = O.quantize_lastdim(w64[e])
        assert np.array_equal(out["row"].codes[e].cpu().numpy(), rc)
        assert np.array_equal(out["row"].scales[e].cpu().numpy(), rs)


def test_mxfp8_linear_workload_inputs_bit_exact(dev):
    """X of the T=8192, K=1024 outlier workload (1% of entries x100) and its
    expert weights [8, 2816, 1024]: rowwise and token-axis copies."""
    case = make_linear_case("mxfp8_linear", seed=0)
    x = case.X.to(dev)
    off = case.offsets.to(dev)
    out = gm.mxfp8_quantize(x, rowwise=True, colwise=True, offsets=off)
    wq = gm.mxfp8_quantize(case.W.to(dev), rowwise=True)
    torch.cuda.synchronize()
    x64 = to64(case.X)
    rc, rs = O.quantize_lastdim(x64)
    assert np.array_equal(out["row"].codes.cpu().numpy(), rc)
    assert np.array_equal(out["row"].scales.cpu().numpy(), rs)
    codes, scales, poff = O.quantize_tokens(x64, case.offsets.numpy(), align=128)
    n = int(poff[-1])
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], codes)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], scales)
    wc, ws = O.quantize_lastdim(to64(case.W))
    assert np.array_equal(wq["row"].codes.cpu().numpy(), wc)
    assert np.array_equal(wq["row"].scales.cpu().numpy(), ws)
