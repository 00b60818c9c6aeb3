"""GPU parity at the full sizes of the Mixtral-8x7B expert workload (T=16384
top-2, E=8, H=4096, F=14336, Zipf(1.1) loads, forward + backward) and of the
64-expert long-sequence workload (T=32768 top-8, E=64, H=2048, F=1408, 8
empty experts), run exactly as bench.py runs the headline workload: inputs
drawn on the GPU by the seeded generator, one grouped_mlp_fwd and one
grouped_mlp_bwd on the library's default launch configuration.

The FP64 oracle cannot run these sizes whole, so it is run on samples it can
compute exactly (see tests/_oracle_workers.py): whole experts (every output
of the expert, including dW1[e] and dW2[e]) and row subsets of the largest
expert (Y, dX and dr of those rows), in worker processes while the GPU runs.
Bars as in test_gpu_mlp.py end to end: relative Frobenius error <= 1e-2 for
every compared tensor, max |err| / rms(reference row) <= 0.1 for Y, dX and
dr (a requantized intermediate code can flip next to a rounding boundary),
weight gradients held to the Frobenius bar per expert.  Properties over the
whole output: every value finite, empty experts' weight gradients exactly
zero."""
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

REL_F, E2E_ROW_MAX = 1e-2, 0.1


def _np32(t):
    return t.float().cpu().numpy()


def _check(name, got, ref, row=E2E_ROW_MAX):
    rel, worst = O.parity_metrics(np.asarray(got, dtype=np.float64), ref)
    print(f"  {name:24s} rel_fro={rel:.3e} max_row={worst:.3e}", flush=True)
    assert rel <= REL_F and worst <= row, (name, rel, worst)


def _jobs(case, samples):
    """Oracle inputs of each sample: (label, expert, row indices or None)."""
    off = case.offsets.cpu().numpy()
    out = []
    for label, e, rows in samples:
        lo, hi = int(off[e]), int(off[e + 1])
        idx = np.arange(lo, hi) if rows is None else lo + np.asarray(rows)
        ti = torch.from_numpy(idx).to(case.X.device)
        out.append((label, e, rows is None, idx,
                    (_np32(case.X.index_select(0, ti)), _np32(case.W1[e]), _np32(case.W2[e]),
                     case.r.index_select(0, ti).cpu().numpy(), _np32(case.dY.index_select(0, ti)))))
    return out


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
        cbuf = torch.full((gm.ctx_bytes(M, H, F, E),), 255,
                          dtype=torch.uint8, device=dev)
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
        for (label, e, whole, idx, _), fut in zip(jobs, futs):
            Yr, dXr, drr, dW1r, dW2r = fut.result()
            ti = torch.from_numpy(idx).to(dev)
            print(f" {label}: expert {e}, {len(idx)} rows", flush=True)
            _check("Y", _np32(y.index_select(0, ti)), Yr)
            _check("dX", _np32(dx.index_select(0, ti)), dXr)
            _check("dr", dr.index_select(0, ti).cpu().numpy(), drr)
            if whole:
                _check("dW1[e]", _np32(dw1[e]), dW1r, row=np.inf)
                _check("dW2[e]", _np32(dw2[e]), dW2r, row=np.inf)


def test_mixtral_fwd_bwd_full_size(dev):
    case = make_mlp_case("mixtral_fwd_bwd", seed=0, device=dev)
    counts = [int(c) for c in case.counts]
    small, big = int(np.argmin(counts)), int(np.argmax(counts))
    n = counts[big]
    rows = list(range(16)) + list(range(n // 2, n // 2 + 16)) + list(range(n - 32, n))
    _run_full(dev, case, [("smallest expert, whole", small, None),
                          ("largest expert, 64 rows", big, rows)])


def test_fine_grained_64e_full_size(dev):
    case = make_mlp_case("fine_grained_64e", seed=0, device=dev)
    counts = [int(c) for c in case.counts]
    assert sum(c == 0 for c in counts) == 8
    nz = [e for e in range(len(counts)) if counts[e] > 0]
    small = min(nz, key=lambda e: counts[e])
    big = max(nz, key=lambda e: counts[e])
    mid = sorted(nz, key=lambda e: counts[e])[len(nz) // 2]
    n = counts[big]
    rows = list(range(16)) + list(range(n // 2, n // 2 + 16)) + list(range(n - 32, n))
    _run_full(dev, case, [("smallest expert, whole", small, None),
                          ("median expert, whole", mid, None),
                          ("largest expert, 64 rows", big, rows)])
