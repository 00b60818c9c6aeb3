"""Pins of the oracle's GroupedMLP forward and backward.

* Unquantized mode: reduces to a dense Mixtral-style expert FFN computed with
  torch, and its backward equals torch.autograd in float64 and central finite
  differences.
* Quantized mode: which axis each GEMM operand is blocked along is pinned by
  inputs that are exactly MXFP8-representable along the intended axis and
  lossy along every other axis; a wrong axis changes the result.
* Invariants: r_i dr_i = <Y_i, dY_i>, zero rows, empty experts, dY = 0.
"""
import numpy as np
import torch

from oracle import mx_oracle as O
from tests.test_oracle_codec import exact_block_values


def rand_case(rng, M_counts, H, F, wstd=0.1):
    offsets = np.concatenate([[0], np.cumsum(M_counts)]).astype(np.int64)
    M, E = int(offsets[-1]), len(M_counts)
    X = rng.standard_normal((M, H))
    W1 = rng.standard_normal((E, 2 * F, H)) * wstd
    W2 = rng.standard_normal((E, H, F)) * wstd
    r = rng.uniform(0.1, 1.0, M)
    dY = rng.standard_normal((M, H))
    return X, W1, W2, r, offsets, dY


def torch_mlp(X, W1, W2, r, offsets):
    """Independent torch formulation (float64) of the unquantized MLP."""
    F = W2.shape[2]
    outs = []
    for e in range(W1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        x = X[lo:hi]
        g = x @ W1[e, :F].T
        u = x @ W1[e, F:].T
        outs.append((torch.nn.functional.silu(g) * u * r[lo:hi, None])
                    @ W2[e].T)
    return torch.cat(outs, 0)


def test_fwd_single_expert_dense_ffn():
    rng = np.random.default_rng(20)
    X, W1, W2, r, off, _ = rand_case(rng, [37], 64, 32)
    r[:] = 1.0
    Y, _ = O.grouped_mlp_fwd(X, W1, W2, r, off, quantize=False)
    w1, w3 = torch.from_numpy(W1[0, :32]), torch.from_numpy(W1[0, 32:])
    x = torch.from_numpy(X)
    ref = (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ torch.from_numpy(
        W2[0]).T
    assert np.allclose(Y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_bwd_unquantized_matches_autograd():
    rng = np.random.default_rng(21)
    X, W1, W2, r, off, dY = rand_case(rng, [5, 0, 17, 10], 64, 32)
    Y, saved = O.grouped_mlp_fwd(X, W1, W2, r, off, quantize=False)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved, quantize=False)

    tX, tW1, tW2, tr = (torch.tensor(a, requires_grad=True)
                        for a in (X, W1, W2, r))
    tY = torch_mlp(tX, tW1, tW2, tr, off)
    assert np.allclose(Y, tY.detach().numpy(), rtol=1e-12, atol=1e-12)
    (tY * torch.from_numpy(dY)).sum().backward()
    for name, t in (("dX", tX), ("dW1", tW1), ("dW2", tW2), ("dr", tr)):
        assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10,
                           atol=1e-12), name
    assert not g["dW1"][1].any() and not g["dW2"][1].any()


def test_bwd_unquantized_finite_differences():
    rng = np.random.default_rng(22)
    X, W1, W2, r, off, dY = rand_case(rng, [6, 9], 32, 32)
    _, saved = O.grouped_mlp_fwd(X, W1, W2, r, off, quantize=False)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved, quantize=False)

    def loss(X_, W1_, W2_, r_):
        return float((O.grouped_mlp_fwd(X_, W1_, W2_, r_, off,
                                        quantize=False)[0] * dY).sum())

    eps = 1e-6
    checks = [("dX", 0, (3, 7)), ("dX", 0, (12, 30)), ("dW1", 1, (1, 5, 9)),
              ("dW1", 1, (0, 40, 3)), ("dW2", 2, (1, 2, 31)), ("dr", 3, (4,)),
              ("dr", 3, (14,))]
    args = [X, W1, W2, r]
    for name, which, idx in checks:
        p, m = [a.copy() for a in args], [a.copy() for a in args]
        p[which][idx] += eps
        m[which][idx] -= eps
        fd = (loss(*p) - loss(*m)) / (2 * eps)
        assert abs(fd - g[name][idx]) <= 1e-6 * max(1.0, abs(fd)), name


def test_bwd_routing_weight_invariant():
    rng = np.random.default_rng(23)
    X, W1, W2, r, off, dY = rand_case(rng, [8, 8, 3], 64, 64)
    Y, saved = O.grouped_mlp_fwd(X, W1, W2, r, off, quantize=False)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved, quantize=False)
    assert np.allclose(r * g["dr"], (Y * dY).sum(axis=1), rtol=1e-10,
                       atol=1e-12)


def test_quantized_zero_rows_empty_experts_zero_dy():
    rng = np.random.default_rng(24)
    X, W1, W2, r, off, dY = rand_case(rng, [40, 0, 33], 64, 64)
    r[5] = 0.0
    Y, saved = O.grouped_mlp_fwd(X, W1, W2, r, off)
    assert not Y[5].any()
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved)
    assert not g["dW1"][1].any() and not g["dW2"][1].any()
    z = O.grouped_mlp_bwd(np.zeros_like(dY), X, W1, W2, r, off, saved)
    for name in ("dX", "dW1", "dW2", "dr"):
        assert not z[name].any(), name


def test_quantized_close_to_unquantized():
    rng = np.random.default_rng(25)
    X, W1, W2, r, off, dY = rand_case(rng, [64, 29, 0, 100], 128, 64)
    Yq, sq = O.grouped_mlp_fwd(X, W1, W2, r, off)
    Yu, su = O.grouped_mlp_fwd(X, W1, W2, r, off, quantize=False)
    assert O.parity_metrics(Yq, Yu)[0] < 0.15
    gq = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, sq)
    gu = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, su, quantize=False)
    for name in ("dX", "dW1", "dW2", "dr"):
        assert O.parity_metrics(gq[name], gu[name])[0] < 0.2, name


def lossy_elsewhere(rng, shape, axis):
    """Exactly representable along 32-blocks of ``axis``; exponents jump by
    up to 40 between neighbouring blocks, so blocking along any other axis
    loses values."""
    moved = np.moveaxis(np.zeros(shape), axis, -1)
    v = exact_block_values(rng, moved.shape, -20, 20)
    return np.moveaxis(v, -1, axis)


def test_fwd_quantization_axes():
    rng = np.random.default_rng(26)
    H, F = 64, 64
    off = np.array([0, 32, 96])
    X = rng.standard_normal((96, H))
    W1 = lossy_elsewhere(rng, (2, 2 * F, H), 2)       # exact along H
    W2 = lossy_elsewhere(rng, (2, H, F), 2)           # exact along F
    assert not np.array_equal(O.qdq_lastdim(np.swapaxes(W1, 1, 2)),
                              np.swapaxes(W1, 1, 2))
    r = rng.uniform(0.2, 1.0, 96)
    Y, s = O.grouped_mlp_fwd(X, W1, W2, r, off)
    assert np.array_equal(s["h"], O.grouped_linear(O.qdq_lastdim(X), W1, off))
    assert np.array_equal(Y, O.grouped_linear(O.qdq_lastdim(s["z"]), W2, off))


def test_bwd_dgrad_quantization_axes():
    rng = np.random.default_rng(27)
    H, F = 64, 64
    off = np.array([0, 40, 96])
    X = rng.standard_normal((96, H))
    W1 = lossy_elsewhere(rng, (2, 2 * F, H), 1)       # exact along 2F
    W2 = lossy_elsewhere(rng, (2, H, F), 1)           # exact along H
    assert not np.array_equal(O.qdq_lastdim(W2), W2)
    r = rng.uniform(0.2, 1.0, 96)
    dY = rng.standard_normal((96, H))
    _, s = O.grouped_mlp_fwd(X, W1, W2, r, off)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, s)
    assert np.array_equal(
        g["dz"], O.grouped_linear(O.qdq_lastdim(dY), W2.transpose(0, 2, 1),
                                  off))
    assert np.array_equal(
        g["dX"], O.grouped_linear(O.qdq_lastdim(g["dh"]),
                                  W1.transpose(0, 2, 1), off))


def test_bwd_wgrad_token_axis():
    rng = np.random.default_rng(28)
    H, F = 64, 32
    off = np.array([0, 64, 160])                      # 32-aligned experts
    X = lossy_elsewhere(rng, (160, H), 0)              # exact along tokens
    dY = lossy_elsewhere(rng, (160, H), 0)
    assert not np.array_equal(O.qdq_lastdim(X), X)
    W1 = rng.standard_normal((2, 2 * F, H)) * 0.1
    W2 = rng.standard_normal((2, H, F)) * 0.1
    r = rng.uniform(0.2, 1.0, 160)
    _, s = O.grouped_mlp_fwd(X, W1, W2, r, off)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, s)
    zt = O.qdq_tokens(s["z"], off)
    dht = O.qdq_tokens(g["dh"], off)
    for e in range(2):
        lo, hi = off[e], off[e + 1]
        assert np.array_equal(g["dW2"][e], dY[lo:hi].T @ zt[lo:hi])
        assert np.array_equal(g["dW1"][e], dht[lo:hi].T @ X[lo:hi])


def test_parity_metrics_definition():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    got = np.array([[3.0, 4.5], [0.0, 0.0]])
    rel, worst = O.parity_metrics(got, ref)
    assert abs(rel - 0.1) < 1e-12
    assert abs(worst - 0.5 / np.sqrt(12.5)) < 1e-12
    got[1, 0] = 1e-30
    assert O.parity_metrics(got, ref)[1] == np.inf


def test_single_expert_slices_equal_the_full_computation():
    """The full-size GPU tests compare against the oracle run on one expert
    alone, or on a subset of one expert's rows: pin that this equals the
    corresponding slice of the oracle run on all experts (weight gradients
    only for whole experts)."""
    from tests._oracle_workers import expert_reference
    rng = np.random.default_rng(11)
    counts = [70, 0, 129, 33]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M, H, F, E = int(off[-1]), 64, 96, len(counts)
    bf = lambda *s, std=1.0: O.round_bf16(rng.standard_normal(s) * std)
    X, dY = bf(M, H), bf(M, H)
    W1, W2 = bf(E, 2 * F, H, std=0.05), bf(E, H, F, std=0.05)
    r = rng.uniform(0.1, 1.0, M)
    Y, saved = O.grouped_mlp_fwd(X, W1, W2, r, off)
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved)
    # equal up to fp64 summation order (BLAS may block a sub-problem differently)
    same = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-10,
                                                   atol=1e-12 * max(1.0, np.abs(b).max()))
    for e in (0, 2, 3):
        lo, hi = off[e], off[e + 1]
        Ye, dXe, dre, dW1e, dW2e = expert_reference(X[lo:hi], W1[e], W2[e], r[lo:hi], dY[lo:hi])
        same(Ye, Y[lo:hi]); same(dXe, g["dX"][lo:hi]); same(dre, g["dr"][lo:hi])
        same(dW1e, g["dW1"][e]); same(dW2e, g["dW2"][e])
    # a row subset of expert 2 (rows 0..4, 64..69, 120..128): row-local outputs
    lo = off[2]
    rows = np.r_[0:5, 64:70, 120:129]
    Ys, dXs, drs, _, _ = expert_reference(X[lo + rows], W1[2], W2[2], r[lo + rows],
                                          dY[lo + rows])
    same(Ys, Y[lo + rows]); same(dXs, g["dX"][lo + rows]); same(drs, g["dr"][lo + rows])


def _load_h_rounding_case():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mlp_bwd_h_rounding.txt")
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            kv[key] = vals
    H, F = int(kv["H"][0]), int(kv["F"][0])
    X = np.zeros((1, H))
    for t in kv["x"]:
        i, v = t.split(":")
        X[0, int(i)] = float(v)
    W1 = np.zeros((1, 2 * F, H))
    for t in kv["w1"]:
        i, j, v = t.split(":")
        W1[0, int(i), int(j)] = float(v)
    W2 = np.zeros((1, H, F))
    for t in kv["w2"]:
        i, j, v = t.split(":")
        W2[0, int(i), int(j)] = float(v)
    dY = np.zeros((1, H))
    for t in kv["dy"]:
        i, v = t.split(":")
        dY[0, int(i)] = float(v)
    r = np.array([float(kv["r"][0])])
    exp = {}
    for mode in ("recompute", "saved_h"):
        codes = np.zeros(2 * F, dtype=np.uint8)
        lead = [int(c, 16) for c in kv["codes_" + mode]]
        codes[:len(lead)] = lead
        exp[mode] = (codes, np.array([int(s) for s in kv["scales_" + mode]], dtype=np.uint8))
    return X, W1, W2, dY, r, exp


def test_bwd_h_rounding_golden_codes():
    """Hand-derived dh codes (tests/golden/mlp_bwd_h_rounding.txt): the
    default backward uses the exact h (its code 1 is 0x39); the saved-h mode
    reads bf16(h) (code 1 is 0x38).  A rounding of h dropped from one mode or
    added to the other, or a bf16 rounding of dz or dh, changes a code."""
    X, W1, W2, dY, r, exp = _load_h_rounding_case()
    off = np.array([0, 1], dtype=np.int64)
    # the inputs are MXFP8-exact, so the quantizers leave them unchanged
    for t in (X, W1, W2.transpose(0, 2, 1), dY):
        assert np.array_equal(O.qdq_lastdim(t), t)
    Y, saved = O.grouped_mlp_fwd(X, W1, W2, r, off)
    assert saved["h"][0, 32] == 288.0 and saved["h"][0, 33] == 1.0634765625
    for mode, kw in (("recompute", {}), ("saved_h", {"h_bf16": True})):
        g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved, **kw)
        codes, scales = O.quantize_lastdim(g["dh"])
        assert np.array_equal(codes[0], exp[mode][0]), (mode, codes[0][:4])
        assert np.array_equal(scales[0], exp[mode][1]), (mode, scales[0])
        assert g["dr"][0] == 0.0                      # s = silu(0) b = 0
    assert not np.array_equal(exp["recompute"][0], exp["saved_h"][0])


def test_bwd_h_bf16_mode_reads_the_rounded_h():
    """The saved-h mode equals the default backward run on bf16(h), and the
    two differ once h is not bf16-representable."""
    rng = np.random.default_rng(29)
    X, W1, W2, r, off, dY = rand_case(rng, [40, 0, 57], 64, 64)
    _, saved = O.grouped_mlp_fwd(X, W1, W2, r, off)
    g_s = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved, h_bf16=True)
    rounded = dict(saved, h=O.round_bf16(saved["h"]))
    g_r = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, rounded)
    for name in ("dX", "dW1", "dW2", "dr", "dh"):
        assert np.array_equal(g_s[name], g_r[name]), name
    g = O.grouped_mlp_bwd(dY, X, W1, W2, r, off, saved)
    assert not np.array_equal(g["dh"], g_s["dh"])
