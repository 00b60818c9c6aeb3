"""GPU parity of the routing steps around the expert path (sorted-row plan,
permute + quantize, combine and its backward) against oracle/moe_route.py
and the MXFP8 oracle.  Integer and byte results bit-exact; bf16 results within
one rounding of the fp64 reference plus the fp32 accumulation bound."""
import numpy as np
import pytest
import torch

import grouped_gemm_mxfp8_amd as gm
from oracle import moe_route as R
from oracle import mx_oracle as O

pytestmark = pytest.mark.gpu


def routing(rng, T, k, E, skip=(), invalid=0):
    """Top-k ids with distinct experts per token (k <= live experts), an
    optional set of never-chosen experts, and ``invalid`` slots set to ids
    outside [0, E)."""
    live = np.array([e for e in range(E) if e not in skip])
    ids = np.stack([rng.choice(live, size=k, replace=False) for _ in range(T)]) if T else \
        np.zeros((0, k), dtype=np.int64)
    w = rng.random((T, k))
    if invalid:
        flat = ids.reshape(-1)
        pick = rng.choice(flat.size, size=invalid, replace=False)
        flat[pick[: invalid // 2]] = -1
        flat[pick[invalid // 2:]] = E
    return ids.astype(np.int32), w.astype(np.float32)


def bf16(rng, shape, scale=1.0):
    return torch.tensor(rng.standard_normal(shape) * scale, dtype=torch.float32).to(torch.bfloat16)


def oracle_plan(ids, E):
    """The oracle's plan over the routed slots only (ids in [0, E))."""
    T, k = ids.shape
    ok = (ids >= 0) & (ids < E)
    key = np.where(ok, ids, E)                      # unrouted slots sort last
    offs, row_of, tok_of = R.route_plan(key, E + 1)
    M = int(offs[E])
    return offs[:E + 1], np.where(ok, row_of, -1), tok_of[:M], M


@pytest.mark.parametrize("T,k,E,skip,invalid", [
    (0, 2, 4, (), 0), (1, 1, 1, (), 0), (300, 2, 8, (3,), 0), (1000, 8, 64, (7, 15, 63), 0),
    (2500, 4, 1024, (), 0), (777, 2, 16, (1,), 40),
])
def test_route_plan_matches_oracle(dev, T, k, E, skip, invalid):
    rng = np.random.default_rng(T + 17 * k + E)
    ids, w = routing(rng, T, k, E, skip, invalid)
    offs, row_of, tok_of, r_sorted = gm.route_plan(torch.from_numpy(ids).to(dev), E,
                                                    torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    o_offs, o_row, o_tok, M = oracle_plan(ids, E)
    assert np.array_equal(offs.cpu().numpy(), o_offs)
    assert np.array_equal(row_of.cpu().numpy(), o_row)
    assert np.array_equal(tok_of.cpu().numpy()[:M], o_tok)
    ok = o_row >= 0
    r_ref = np.zeros(M, dtype=np.float32)
    r_ref[o_row[ok]] = w[ok]
    assert np.array_equal(r_sorted.cpu().numpy()[:M], r_ref)        # bits of w, moved


@pytest.mark.parametrize("T,k,E,H,skip", [
    (200, 2, 4, 256, (2,)), (513, 2, 8, 96, ()), (64, 8, 16, 512, (0, 9)), (1, 1, 1, 32, ()),
])
def test_permute_quantize_matches_oracle(dev, T, k, E, H, skip):
    rng = np.random.default_rng(T * H + k)
    ids, _ = routing(rng, T, k, E, skip)
    x = bf16(rng, (T, H))
    offs, row_of, tok_of, _ = gm.route_plan(torch.from_numpy(ids).to(dev), E)
    M = T * k
    out = gm.permute_quantize(x.to(dev), tok_of, offs, M)
    torch.cuda.synchronize()
    o_offs, _, o_tok, _ = oracle_plan(ids, E)
    xs = R.permute_rows(x.double().numpy(), o_tok)
    rc, rs = O.quantize_lastdim(xs)
    assert np.array_equal(out["row"].codes.cpu().numpy(), rc)
    assert np.array_equal(out["row"].scales.cpu().numpy(), rs)
    cc, cs, poff = O.quantize_tokens(xs, o_offs)
    n = int(poff[-1])
    assert np.array_equal(out["padded_offsets"].cpu().numpy(), poff)
    assert np.array_equal(out["col"].codes.cpu().numpy()[:, :n], cc)
    assert np.array_equal(out["col"].scales.cpu().numpy()[:, : n // 32], cs)


def test_permute_quantize_equals_quantizing_sorted_rows(dev):
    """Same bytes as the plain quantizer applied to rows gathered by torch."""
    rng = np.random.default_rng(5)
    T, k, E, H = 1500, 2, 8, 1024
    ids, _ = routing(rng, T, k, E)
    x = bf16(rng, (T, H), 3.0).to(dev)
    offs, row_of, tok_of, _ = gm.route_plan(torch.from_numpy(ids).to(dev), E)
    a = gm.permute_quantize(x, tok_of, offs, T * k)
    b = gm.mxfp8_quantize(x[tok_of.long()], rowwise=True, colwise=True, offsets=offs)
    torch.cuda.synchronize()
    assert torch.equal(a["row"].codes, b["row"].codes)
    assert torch.equal(a["row"].scales, b["row"].scales)
    # columnwise: the padded token range (columns past it are not written)
    n = int(a["padded_offsets"][-1].item())
    assert torch.equal(a["padded_offsets"], b["padded_offsets"])
    assert torch.equal(a["col"].codes[:, :n], b["col"].codes[:, :n])
    assert torch.equal(a["col"].scales[:, : n // 32], b["col"].scales[:, : n // 32])


def combine_bound(terms_abs, ref):
    """One bf16 rounding of the result plus the fp32 accumulation error."""
    return np.abs(ref) * 2.0 ** -8 + terms_abs * 2.0 ** -20


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("T,k,E,H,invalid", [(300, 2, 8, 256, 0), (97, 8, 16, 64, 30),
                                              (0, 2, 4, 64, 0)])
def test_combine_matches_oracle(dev, weighted, T, k, E, H, invalid):
    rng = np.random.default_rng(T + k + H + weighted)
    ids, w = routing(rng, T, k, E, (), invalid)
    offs, row_of, tok_of, _ = gm.route_plan(torch.from_numpy(ids).to(dev), E)
    M = int(offs[-1].item()) if T else 0
    y = bf16(rng, (max(M, 1), H))[:M]
    out = gm.combine(y.to(dev), row_of, torch.from_numpy(w).to(dev) if weighted else None)
    torch.cuda.synchronize()
    _, o_row, _, _ = oracle_plan(ids, E)
    y64 = y.double().numpy()
    wv = w.astype(np.float64) if weighted else np.ones((T, k))
    ref = np.zeros((T, H))
    terms = np.zeros((T, H))
    for j in range(k):
        ok = o_row[:, j] >= 0
        ref[ok] += wv[ok, j:j + 1] * y64[o_row[ok, j]]
        terms[ok] += np.abs(wv[ok, j:j + 1] * y64[o_row[ok, j]])
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= combine_bound(terms, ref))


def test_combine_single_slot_is_exact_inverse_permute(dev):
    rng = np.random.default_rng(7)
    T, E, H = 400, 6, 128
    ids, _ = routing(rng, T, 1, E)
    x = bf16(rng, (T, H)).to(dev)
    offs, row_of, tok_of, _ = gm.route_plan(torch.from_numpy(ids).to(dev), E)
    xs, _ = gm.combine_bwd(x, row_of, T)                 # token -> sorted rows
    back = gm.combine(xs, row_of)
    torch.cuda.synchronize()
    assert torch.equal(xs, x[tok_of.long()])
    assert torch.equal(back, x)


@pytest.mark.parametrize("weighted", [False, True])
def test_combine_bwd_matches_oracle(dev, weighted):
    rng = np.random.default_rng(21 + weighted)
    T, k, E, H = 350, 4, 12, 320
    ids, w = routing(rng, T, k, E, (5,), 20)
    offs, row_of, tok_of, _ = gm.route_plan(torch.from_numpy(ids).to(dev), E)
    M = int(offs[-1].item())
    dout = bf16(rng, (T, H))
    y = bf16(rng, (M, H))
    wd = torch.from_numpy(w).to(dev) if weighted else None
    dy, dw = gm.combine_bwd(dout.to(dev), row_of, M, wd, y.to(dev) if weighted else None)
    torch.cuda.synchronize()
    _, o_row, _, _ = oracle_plan(ids, E)
    d64, y64 = dout.double().numpy(), y.double().numpy()
    got = dy.double().cpu().numpy()
    for t in range(T):
        for j in range(k):
            row = o_row[t, j]
            if row < 0:
                continue
            if weighted:
                ref = float(w[t, j]) * d64[t]
                assert np.all(np.abs(got[row] - ref) <= np.abs(ref) * 2.0 ** -8)
            else:
                assert np.array_equal(got[row], d64[t])
    if weighted:
        ok = o_row >= 0
        ref = np.zeros((T, k))
        mag = np.zeros((T, k))
        for j in range(k):
            sel = ok[:, j]
            ref[sel, j] = np.sum(d64[sel] * y64[o_row[sel, j]], axis=1)
            mag[sel, j] = np.sum(np.abs(d64[sel] * y64[o_row[sel, j]]), axis=1)
        assert np.all(np.abs(dw.double().cpu().numpy() - ref) <= mag * 2.0 ** -18 + 1e-30)
    else:
        assert dw is None


def test_mixtral_shape_round_trip(dev):
    """The Mixtral-shape routing (T=16384 top-2, E=8, H=4096) through plan,
    permute + quantize and combine: bytes of sampled sorted rows against the
    oracle, and the unweighted combine of the permuted rows is 2 x."""
    rng = np.random.default_rng(0)
    T, k, E, H = 16384, 2, 8, 4096
    ids, w = routing(rng, T, k, E)
    x = bf16(rng, (T, H)).to(dev)
    ids_d = torch.from_numpy(ids).to(dev)
    offs, row_of, tok_of, r_sorted = gm.route_plan(ids_d, E, torch.from_numpy(w).to(dev))
    q = gm.permute_quantize(x, tok_of, offs, T * k)
    xs, _ = gm.combine_bwd(x, row_of, T * k)
    twice = gm.combine(xs, row_of)
    torch.cuda.synchronize()
    o_offs, o_row, o_tok, M = oracle_plan(ids, E)
    assert np.array_equal(offs.cpu().numpy(), o_offs)
    assert np.array_equal(tok_of.cpu().numpy(), o_tok)
    rows = rng.choice(M, size=64, replace=False)
    xs_ref = R.permute_rows(x.double().cpu().numpy(), o_tok[rows])
    rc, rs = O.quantize_lastdim(xs_ref)
    assert np.array_equal(q["row"].codes[torch.from_numpy(rows).to(dev)].cpu().numpy(), rc)
    assert np.array_equal(q["row"].scales[torch.from_numpy(rows).to(dev)].cpu().numpy(), rs)
    assert torch.equal(twice.float(), (2.0 * x.float()))   # x + x is exact in bf16


@pytest.mark.parametrize("T,E,k,ties", [
    (0, 8, 2, False), (1, 1, 1, False), (333, 8, 2, False), (1000, 64, 8, True),
    (257, 1024, 64, True), (500, 100, 7, False), (64, 65, 65 - 1, True), (128, 16, 16, True),
])
def test_router_matches_oracle(dev, T, E, k, ties):
    """Expert ids bit-exact (ties to the lower index); weights within a few
    fp32 roundings of the fp64 softmax."""
    rng = np.random.default_rng(T * 7 + E + k)
    lg = rng.standard_normal((T, E)) * 3
    if ties:
        lg = np.round(lg * 2) / 2                      # many equal logits per token
    lg = lg.astype(np.float32)
    ids, w = gm.router(torch.from_numpy(lg).to(dev), k)
    torch.cuda.synchronize()
    o_ids, o_w = R.router_topk_softmax(lg.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    assert np.all(np.abs(w.double().cpu().numpy() - o_w) <= o_w * 2.0 ** -18)


def test_router_feeds_the_plan(dev):
    """Router output straight into the plan: every token's slots land in its
    experts' row ranges, and the sorted weights are the router's."""
    rng = np.random.default_rng(23)
    T, E, k = 4096, 8, 2
    lg = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).to(dev)
    ids, w = gm.router(lg, k)
    offs, row_of, tok_of, r_sorted = gm.route_plan(ids, E, w)
    torch.cuda.synchronize()
    o_ids, _ = R.router_topk_softmax(lg.double().cpu().numpy(), k)
    o_offs, o_row, o_tok, M = oracle_plan(o_ids.astype(np.int32), E)
    assert np.array_equal(offs.cpu().numpy(), o_offs)
    assert np.array_equal(row_of.cpu().numpy(), o_row)
    assert np.array_equal(r_sorted.cpu().numpy()[o_row.reshape(-1)], w.cpu().numpy().reshape(-1))
