"""MX_CHECK=1: entry points that take device offsets copy them to the host
and refuse bad ones (not starting at 0, decreasing, not ending at the row
count) with MX_ERR_INVALID_ARG before launching anything; good offsets give
the same results as without the check.  Bad offsets only ever reach the
checked calls: without MX_CHECK they would be undefined behaviour."""
import re

import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from workloads import make_mlp_case

pytestmark = pytest.mark.gpu


def test_mx_check_refuses_bad_device_offsets(dev, monkeypatch):
    g = torch.Generator().manual_seed(0)
    M, K, N, E = 300, 128, 256, 3
    x = torch.randn((M, K), generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn((E, N, K), generator=g) * 0.05).to(torch.bfloat16).to(dev)
    good = torch.tensor([0, 100, 100, 300], dtype=torch.int64, device=dev)
    y_plain = gm.grouped_linear_fwd(x, good, w)
    torch.cuda.synchronize()
    monkeypatch.setenv("MX_CHECK", "1")
    assert torch.equal(gm.grouped_linear_fwd(x, good, w), y_plain)
    for bad, msg in (([0, 200, 100, 300], "decrease"), ([0, 100, 100, 299], "row count"),
                     ([5, 100, 100, 300], "offsets[0]")):
        off = torch.tensor(bad, dtype=torch.int64, device=dev)
        with pytest.raises(gm.MxError, match="status 1") as ei:
            gm.grouped_linear_fwd(x, off, w)
        assert msg in str(ei.value)
        mx = gm.mxfp8_quantize(x)["row"]
        mw = gm.mxfp8_quantize(w)["row"]
        with pytest.raises(gm.MxError, match=re.escape(msg)):
            gm.grouped_linear_fwd(mx, off, mw)
        with pytest.raises(gm.MxError, match=re.escape(msg)):
            gm.mxfp8_quantize(x, rowwise=False, colwise=True, offsets=off)
    # the fused MLP refuses them too, forward and backward
    case = make_mlp_case(None, seed=1, T=150, k=2, E=3, H=128, F=128, routing="counts",
                         counts=[150, 0, 150])
    xm, w1, w2, r, dy = (case.X.to(dev), case.W1.to(dev), case.W2.to(dev), case.r.to(dev),
                         case.dY.to(dev))
    off = case.offsets.to(dev)
    y, ctx = gm.grouped_mlp_fwd(xm, off, w1, w2, r)
    gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx)
    torch.cuda.synchronize()
    bad = torch.tensor([0, 150, 150, 250], dtype=torch.int64, device=dev)
    with pytest.raises(gm.MxError, match="row count"):
        gm.grouped_mlp_fwd(xm, bad, w1, w2, r)
    with pytest.raises(gm.MxError, match="row count"):
        gm.grouped_mlp_bwd(dy, bad, w1, w2, r, ctx)
