"""Pins of oracle/moe_route.py against definitions it does not share code
with: pure-Python loops on small inputs, permutation invariants, closed forms
of the combine, and torch autograd (float64) for the combine's backward."""
import numpy as np
import pytest
import torch

from oracle import moe_route as R


def loop_plan(ids, E):
    """Rows handed out expert by expert, walking tokens then slots in order."""
    T, k = len(ids), len(ids[0])
    row_of = [[-1] * k for _ in range(T)]
    tok_of, offsets = [], [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t][j] == e:
                    row_of[t][j] = len(tok_of)
                    tok_of.append(t)
        offsets.append(len(tok_of))
    return offsets, row_of, tok_of


def random_ids(rng, T, k, E, distinct=True, skip=()):
    live = [e for e in range(E) if e not in skip]
    if distinct and k <= len(live):
        return np.array([rng.choice(live, size=k, replace=False) for _ in range(T)])
    return rng.choice(live, size=(T, k))


@pytest.mark.parametrize("T,k,E,distinct,skip", [
    (1, 1, 1, True, ()), (7, 2, 4, True, ()), (20, 2, 8, True, (0, 5)),
    (33, 4, 6, True, (2,)), (16, 3, 3, False, ()), (50, 8, 16, True, (15,)),
])
def test_plan_matches_loops(T, k, E, distinct, skip):
    rng = np.random.default_rng(T * 31 + k)
    ids = random_ids(rng, T, k, E, distinct, skip)
    offs, row_of, tok_of = R.route_plan(ids, E)
    lo, lr, lt = loop_plan(ids.tolist(), E)
    assert offs.tolist() == lo and row_of.tolist() == lr and tok_of.tolist() == lt


def test_plan_invariants():
    rng = np.random.default_rng(3)
    T, k, E = 200, 2, 8
    ids = random_ids(rng, T, k, E, skip=(6,))
    offs, row_of, tok_of = R.route_plan(ids, E)
    M = T * k
    assert sorted(row_of.reshape(-1).tolist()) == list(range(M))      # a bijection
    assert np.all(np.diff(offs) == np.bincount(ids.reshape(-1), minlength=E))
    assert offs[6] == offs[7]                                         # empty expert
    for t in range(T):
        for j in range(k):
            row = row_of[t, j]
            assert tok_of[row] == t
            assert offs[ids[t, j]] <= row < offs[ids[t, j] + 1]
    # within an expert, token order is kept
    for e in range(E):
        seg = tok_of[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) >= 0)


def test_sorted_weights_follow_rows():
    ids = np.array([[2, 0], [0, 1], [2, 1]])
    w = np.array([[0.7, 0.3], [0.6, 0.4], [0.9, 0.1]])
    offs, row_of, tok_of = R.route_plan(ids, 3)
    # rows: expert 0 -> (t0,j1), (t1,j0); expert 1 -> (t1,j1), (t2,j1); expert 2 -> (t0,j0), (t2,j0)
    assert offs.tolist() == [0, 2, 4, 6]
    assert R.sorted_weights(w, row_of).tolist() == [0.3, 0.6, 0.4, 0.1, 0.7, 0.9]
    assert tok_of.tolist() == [0, 1, 1, 2, 0, 2]


def test_combine_closed_forms():
    rng = np.random.default_rng(5)
    T, k, E, H = 40, 3, 5, 6
    ids = random_ids(rng, T, k, E)
    x = rng.standard_normal((T, H))
    offs, row_of, tok_of = R.route_plan(ids, E)
    xs = R.permute_rows(x, tok_of)
    # unweighted combine of the permuted rows: every token counted k times
    assert np.allclose(R.combine(xs, row_of), k * x, rtol=0, atol=1e-12)
    # weights summing to one per token give the token back
    w = rng.random((T, k))
    w /= w.sum(axis=1, keepdims=True)
    assert np.allclose(R.combine(xs, row_of, w), x, rtol=0, atol=1e-12)
    # k = 1, unweighted: the inverse permutation, exactly
    ids1 = ids[:, :1]
    o1, r1, t1 = R.route_plan(ids1, E)
    assert np.array_equal(R.combine(R.permute_rows(x, t1), r1), x)


def test_combine_matches_loop():
    rng = np.random.default_rng(9)
    T, k, E, H = 12, 2, 4, 5
    ids = random_ids(rng, T, k, E)
    y = rng.standard_normal((T * k, H))
    w = rng.random((T, k))
    _, row_of, _ = R.route_plan(ids, E)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            for h in range(H):
                ref[t, h] += w[t, j] * y[row_of[t, j], h]
    assert np.allclose(R.combine(y, row_of, w), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("weighted", [False, True])
def test_combine_bwd_matches_autograd(weighted):
    rng = np.random.default_rng(11 + weighted)
    T, k, E, H = 25, 2, 6, 7
    ids = random_ids(rng, T, k, E, skip=(1,))
    _, row_of, _ = R.route_plan(ids, E)
    y = torch.tensor(rng.standard_normal((T * k, H)), dtype=torch.float64, requires_grad=True)
    w = torch.tensor(rng.random((T, k)), dtype=torch.float64, requires_grad=True)
    dout = rng.standard_normal((T, H))
    idx = torch.tensor(row_of)
    out = (w.unsqueeze(-1) if weighted else torch.ones(T, k, 1, dtype=torch.float64)) * y[idx]
    out.sum(dim=1).backward(torch.tensor(dout))
    dy, dw = R.combine_bwd(dout, row_of, w.detach().numpy() if weighted else None,
                           y.detach().numpy())
    assert np.allclose(dy, y.grad.numpy(), rtol=0, atol=1e-12)
    if weighted:
        assert np.allclose(dw, w.grad.numpy(), rtol=0, atol=1e-12)
    else:
        assert dw is None


def test_permute_is_the_unweighted_combine_backward():
    rng = np.random.default_rng(13)
    T, k, E, H = 30, 2, 5, 4
    ids = random_ids(rng, T, k, E)
    x = rng.standard_normal((T, H))
    _, row_of, tok_of = R.route_plan(ids, E)
    dy, _ = R.combine_bwd(x, row_of)
    assert np.array_equal(dy, R.permute_rows(x, tok_of))


def test_router_selection_matches_stable_sort():
    """Selection pass by pass equals a stable descending sort (ties to the
    lower index), including heavy ties."""
    rng = np.random.default_rng(17)
    for T, E, k in [(30, 8, 2), (20, 16, 5), (10, 4, 4), (15, 64, 8)]:
        logits = np.round(rng.standard_normal((T, E)) * 2) / 2      # many equal values
        ids, w = R.router_topk_softmax(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)


def test_router_weights_closed_forms():
    rng = np.random.default_rng(19)
    logits = rng.standard_normal((40, 12))
    ids, w = R.router_topk_softmax(logits, 3)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)                    # selection order = weight order
    _, w2 = R.router_topk_softmax(logits + 7.25, 3)           # shift invariance
    assert np.allclose(w, w2, rtol=0, atol=1e-15)
    # two equal selected logits split evenly; k = 1 gives weight 1
    ids1, w1 = R.router_topk_softmax(np.array([[0.5, 2.0, 2.0, -1.0]]), 2)
    assert ids1.tolist() == [[1, 2]] and np.allclose(w1, [[0.5, 0.5]])
    _, wk1 = R.router_topk_softmax(logits, 1)
    assert np.all(wk1 == 1.0)
    # k = E: the full softmax over the row (sorted)
    full = np.exp(logits - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    idsE, wE = R.router_topk_softmax(logits, 12)
    assert np.allclose(wE, np.take_along_axis(full, idsE, axis=1), rtol=0, atol=1e-15)
