"""The routing plan's entry point that allocates nothing
(moe_route_plan_noalloc, the library's own scratch in place of the
workspace), against the entry point with a workspace (moe_route_plan):
bit-identical offsets, rows, tokens and sorted weights, on two calls in a
row, the second smaller than the first (the scratch keeps the first call's
counts), and a host-side rejection of a plan larger than the scratch."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm

pytestmark = pytest.mark.gpu


def _ids(seed, T, k, E, dev, unrouted=0.0):
    g = torch.Generator().manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if unrouted:
        drop = torch.rand((T, k), generator=g) < unrouted
        ids[drop] = -1
    w = torch.rand((T, k), generator=g, dtype=torch.float32)
    return ids.to(dev), w.to(dev)


def _same(a, b):
    """offsets and row_of whole; tok_of and r_sorted on the M routed rows
    the plan writes (entries past M are not outputs)."""
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    M = int(a[0][-1])
    assert torch.equal(a[2][:M], b[2][:M])
    if a[3] is None:
        assert b[3] is None
    else:
        assert torch.equal(a[3][:M], b[3][:M])


def test_noalloc_plan_matches_workspace_plan_twice(dev):
    # first call: 8192 tokens top-2 over 64 experts (64 chunks x 64 counters),
    # some slots unrouted; second: a smaller plan (fewer chunks, fewer experts)
    for seed, T, k, E, unrouted in ((1, 8192, 2, 64, 0.05), (2, 700, 4, 16, 0.0)):
        ids, w = _ids(seed, T, k, E, dev, unrouted)
        got = gm.route_plan_noalloc(ids, E, w)
        ref = gm.route_plan(ids, E, w)
        torch.cuda.synchronize()
        print(f"  T={T} k={k} E={E}: offsets {got[0][:4].tolist()}...", flush=True)
        _same(got, ref)
        counts = np.bincount(ids.cpu().numpy().ravel()[ids.cpu().numpy().ravel() >= 0],
                             minlength=E)
        assert np.array_equal(np.diff(got[0].cpu().numpy()), counts)
    # without routing weights
    ids, _ = _ids(3, 300, 2, 8, dev)
    _same(gm.route_plan_noalloc(ids, 8), gm.route_plan(ids, 8))


def test_noalloc_plan_rejects_plans_larger_than_its_scratch(dev):
    L = gm.lib()
    # ceil(T*k/256) * E > 2^20 counters: T*k = 256 * 1025, E = 1024
    T, k, E = 256 * 1025 // 2, 2, 1024
    st = L.moe_route_plan_noalloc(None, T, k, E, None, None, None, None, None, None)
    assert st != 0
    st = L.moe_route_plan_noalloc(ctypes_ptr(1 << 40), T, k, E, None, ctypes_ptr(1 << 40),
                                  ctypes_ptr(1 << 40), ctypes_ptr(1 << 40), None, None)
    assert st == 2 and "scratch" in gm.last_error()


def ctypes_ptr(v):
    import ctypes
    return ctypes.c_void_p(v)
