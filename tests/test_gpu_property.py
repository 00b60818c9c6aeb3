"""Property-based ragged expert loads (hypothesis, derandomized so every run
draws the same examples): random per-expert row counts, empty experts
included, through the grouped quantizer (bit-exact against the oracle),
MXFP8 GroupedLinear (the spec's bar on the GPU's own codes) and the fused
GroupedMLP in both modes (every stage-wise and end-to-end check of
test_gpu_mlp.py)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import grouped_gemm_mxfp8_amd as gm
from oracle import mx_oracle as O
from tests.test_gpu_mlp import run_case
from workloads import make_mlp_case

pytestmark = pytest.mark.gpu

SETTINGS = dict(derandomize=True, deadline=None, database=None,
                suppress_health_check=[HealthCheck.function_scoped_fixture,
                                       HealthCheck.too_slow])
counts_st = st.lists(st.integers(0, 300), min_size=1, max_size=10).filter(lambda c: sum(c) > 0)


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


@settings(max_examples=25, **SETTINGS)
@given(counts=counts_st, cb=st.integers(1, 8), seed=st.integers(0, 2 ** 16))
def test_grouped_quantizer_ragged(dev, counts, cb, seed):
    C = 32 * cb
    off = _offsets(counts)
    M = int(off[-1])
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((M, C), generator=g) * torch.exp(torch.randn((M, 1), generator=g))
         ).to(torch.bfloat16)
    out = gm.mxfp8_quantize(x.to(dev), rowwise=True, colwise=True,
                            offsets=torch.from_numpy(off).to(dev))
    torch.cuda.synchronize()
    x64 = x.double().numpy()
    rc, rs = O.quantize_lastdim(x64)
    assert np.array_equal(out["row"].codes.cpu().numpy(), rc)
    assert np.array_equal(out["row"].scales.cpu().numpy(), rs)
    cc, cs, poff = O.quantize_tokens(x64, off)
    n = int(poff[-1])
    assert np.array_equal(out["padded_offsets"].cpu().numpy(), poff)
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], cc)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], cs)


@settings(max_examples=15, **SETTINGS)
@given(counts=counts_st, kb=st.integers(1, 3), nb=st.integers(1, 10), seed=st.integers(0, 2 ** 16))
def test_mxfp8_linear_ragged(dev, counts, kb, nb, seed):
    K, N = 128 * kb, 32 * nb
    off = _offsets(counts)
    M, E = int(off[-1]), len(counts)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn((E, N, K), generator=g) * 0.05).to(torch.bfloat16).to(dev)
    r = torch.rand(M, generator=g).to(dev)
    mx, mw = gm.mxfp8_quantize(x)["row"], gm.mxfp8_quantize(w)["row"]
    y = gm.grouped_linear_fwd(mx, torch.from_numpy(off).to(dev), mw, row_scale=r)
    torch.cuda.synchronize()
    deq = lambda t: O.dequantize_lastdim(t.codes.cpu().numpy(), t.scales.cpu().numpy())
    ref = O.grouped_linear(deq(mx), deq(mw), off, row_scale=r.cpu().numpy().astype(np.float64))
    rel, worst = O.parity_metrics(y.float().cpu().numpy().astype(np.float64), ref)
    assert rel <= 1e-2 and worst <= 5e-2, (counts, K, N, rel, worst)


@settings(max_examples=10, **SETTINGS)
@given(counts=st.lists(st.integers(0, 300), min_size=1, max_size=8).filter(lambda c: sum(c) > 0),
       h=st.sampled_from([128, 256]), f=st.sampled_from([128, 256, 384]),
       save_h=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_mlp_ragged(dev, counts, h, f, save_h, seed):
    # top-1 routing, so any count vector is a valid routing of M tokens
    case = make_mlp_case(None, seed=seed, T=sum(counts), k=1, E=len(counts), H=h, F=f,
                         routing="counts", counts=counts)
    run_case(dev, case, save_h=save_h)
