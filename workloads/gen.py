"""Seeded input generators for the five workloads of the MXFP8 MoE expert path.

All draws use a CPU ``torch.Generator`` seeded once per case, in a fixed order
(x, W1, W2, routing, outlier mask, dY), so a case is bit-identical on any
machine.  FP32 samples are rounded to bfloat16 by torch's RNE cast.

Workloads (sizes follow the Mixtral-8x7B expert shape that the pages name as
the scale-up target, and a fine-grained 64-expert long-sequence case):

* ``tiny_bf16_linear``   T=256, top-2, E=4, K=128, N=256, BF16, no quantization
* ``mxfp8_linear``       T=8192, top-2, E=8, K=1024, N=2816, 1% outliers x100
* ``mixtral_fwd``        T=16384, top-2, E=8, H=4096, F=14336, Zipf(1.1) loads
* ``mixtral_fwd_bwd``    as above plus dY
* ``fine_grained_64e``   T=32768, top-8, E=64, H=2048, F=1408, 8 empty experts,
                         largest expert ~12% of assignments
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

CONFIGS = {
    "tiny_bf16_linear": dict(T=256, k=2, E=4, K=128, N=256,
                             routing="topk_normal"),
    "mxfp8_linear": dict(T=8192, k=2, E=8, K=1024, N=2816,
                         routing="topk_uniform", outlier_frac=0.01,
                         outlier_scale=100.0),
    "mixtral_fwd": dict(T=16384, k=2, E=8, H=4096, F=14336, routing="zipf",
                        zipf_s=1.1),
    "mixtral_fwd_bwd": dict(T=16384, k=2, E=8, H=4096, F=14336,
                            routing="zipf", zipf_s=1.1),
    "fine_grained_64e": dict(T=32768, k=8, E=64, H=2048, F=1408,
                             routing="skewed_empty", max_share=0.12),
}

W_STD = 0.02


# --------------------------------------------------------------------------
# Routing (harness side: produces rows, offsets and routing weights).
# --------------------------------------------------------------------------

def topk_softmax_routing(logits: np.ndarray, k: int):
    """Top-k experts per token (ties to the lower index) and the softmax of
    the k selected logits.  Returns (ids [T,k] int64, w [T,k] float64)."""
    logits = np.asarray(logits, dtype=np.float64)
    # stable argsort of -logits keeps the lower index first among ties
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, ids, axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    w = np.exp(sel)
    return ids.astype(np.int64), w / w.sum(axis=1, keepdims=True)


def sort_by_expert(ids: np.ndarray, w: np.ndarray, E: int):
    """Stable sort of the T*k (token, expert) slots by (expert, token).

    Returns (token index [M], routing weight [M] float32, counts [E],
    offsets [E+1] int64)."""
    T, k = ids.shape
    tok = np.repeat(np.arange(T), k)
    exp = ids.reshape(-1)
    wt = w.reshape(-1)
    order = np.lexsort((tok, exp))         # primary key expert, then token
    counts = np.bincount(exp, minlength=E).astype(np.int64)
    return (tok[order].astype(np.int64), wt[order].astype(np.float32),
            counts, offsets_from_counts(counts))


def offsets_from_counts(counts) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def largest_remainder(weights: np.ndarray, total: int) -> np.ndarray:
    """Integer apportionment of ``total`` proportional to ``weights``."""
    q = weights / weights.sum() * total
    base = np.floor(q).astype(np.int64)
    short = total - int(base.sum())
    frac = q - base
    order = np.argsort(-frac, kind="stable")
    base[order[:short]] += 1
    return base


def zipf_counts(M: int, E: int, s: float) -> np.ndarray:
    """Expert loads proportional to rank^-s (expert e has rank e+1)."""
    return largest_remainder(np.arange(1, E + 1, dtype=np.float64) ** -s, M)


def skewed_counts_with_empty(M: int, E: int, max_share: float, cap: int):
    """Experts with e % 8 == 7 get no rows; the others get loads proportional
    to rank^-p with p solved so the largest expert holds ``max_share`` of
    the M assignments (and no expert exceeds ``cap``)."""
    active = np.array([e for e in range(E) if e % 8 != 7])
    ranks = np.arange(1, len(active) + 1, dtype=np.float64)
    lo, hi = 0.0, 5.0
    for _ in range(200):
        p = 0.5 * (lo + hi)
        share = 1.0 / (ranks ** -p).sum()
        if share < max_share:
            lo = p
        else:
            hi = p
    c = largest_remainder(ranks ** -p, M)
    if c.max() > cap:
        raise ValueError("load above per-token cap")
    counts = np.zeros(E, dtype=np.int64)
    counts[active] = c
    return counts


def slot_grid_routing(counts: np.ndarray, T: int, k: int,
                      gen: torch.Generator):
    """Token->expert assignment with exactly ``counts`` rows per expert.

    The k*T slot grid is filled in row-major order with expert ids repeated
    counts[e] times; every counts[e] <= T, so the k slots of a token hold
    distinct experts.  Tokens are then permuted with a seeded permutation and
    the k routing weights of each token are the softmax of k N(0,1) logits.
    """
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.sum() == T * k and counts.max() <= T
    grid = np.repeat(np.arange(len(counts)), counts).reshape(k, T).T  # [T,k]
    perm = torch.randperm(T, generator=gen).numpy()
    ids = grid[perm]
    logits = torch.randn(T, k, generator=gen, dtype=torch.float64).numpy()
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return ids.astype(np.int64), w / w.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Case builders.
# --------------------------------------------------------------------------

def _randn_bf16(gen, shape, std=1.0):
    """N(0, std^2) samples drawn in FP32 then rounded to bfloat16 (on the
    generator's device)."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


@dataclasses.dataclass
class LinearCase:
    X: torch.Tensor            # [M, K] bf16, token-sorted rows
    W: torch.Tensor            # [E, N, K] bf16
    r: torch.Tensor            # [M] float32 routing weight of each row
    offsets: torch.Tensor      # [E+1] int64
    counts: np.ndarray
    token: np.ndarray          # [M] source token of each row
    T: int
    k: int


@dataclasses.dataclass
class MlpCase:
    X: torch.Tensor            # [M, H] bf16, token-sorted rows
    W1: torch.Tensor           # [E, 2F, H] bf16 (gate rows, then up rows)
    W2: torch.Tensor           # [E, H, F] bf16
    r: torch.Tensor            # [M] float32
    offsets: torch.Tensor      # [E+1] int64
    dY: Optional[torch.Tensor] # [M, H] bf16
    counts: np.ndarray
    token: np.ndarray
    T: int
    k: int

    @property
    def M(self):
        return int(self.offsets[-1])

    @property
    def E(self):
        return self.W1.shape[0]

    @property
    def H(self):
        return self.W1.shape[2]

    @property
    def F(self):
        return self.W2.shape[2]


def make_linear_case(name="tiny_bf16_linear", seed=0, **over) -> LinearCase:
    cfg = dict(CONFIGS[name]) if name else {}
    cfg.update(over)
    T, k, E, K, N = cfg["T"], cfg["k"], cfg["E"], cfg["K"], cfg["N"]
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(T, K, generator=gen, dtype=torch.float32)
    W = _randn_bf16(gen, (E, N, K), W_STD)
    routing = cfg.get("routing", "topk_normal")
    if routing == "topk_normal":
        logits = torch.randn(T, E, generator=gen, dtype=torch.float64).numpy()
        ids, w = topk_softmax_routing(logits, k)
    elif routing == "topk_uniform":
        logits = torch.rand(T, E, generator=gen, dtype=torch.float64).numpy()
        ids, w = topk_softmax_routing(logits, k)
    elif routing == "counts":
        ids, w = slot_grid_routing(np.asarray(cfg["counts"]), T, k, gen)
    else:
        raise ValueError(routing)
    frac = cfg.get("outlier_frac", 0.0)
    if frac:
        mask = torch.rand(T, K, generator=gen) < frac
        x = torch.where(mask, x * cfg.get("outlier_scale", 100.0), x)
    xb = x.to(torch.bfloat16)
    tok, r, counts, offs = sort_by_expert(ids, w, E)
    return LinearCase(X=xb[torch.from_numpy(tok)].contiguous(), W=W,
                      r=torch.from_numpy(r), offsets=torch.from_numpy(offs),
                      counts=counts, token=tok, T=T, k=k)


def make_mlp_case(name="mixtral_fwd_bwd", seed=0, with_dy=True, device=None,
                  **over) -> MlpCase:
    """Build a GroupedMLP case.  ``over`` overrides config keys, e.g. a
    scaled-down shape for parity tests: make_mlp_case(None, T=300, k=2, E=4,
    H=256, F=256, routing="counts", counts=[...]).

    With ``device`` (a GPU), x, W1, W2 and dY are drawn there by a generator
    of that device seeded with ``seed`` (same distributions, other values than
    the CPU draw); routing is always drawn on the CPU."""
    cfg = dict(CONFIGS[name]) if name else {}
    cfg.update(over)
    T, k, E, H, F = cfg["T"], cfg["k"], cfg["E"], cfg["H"], cfg["F"]
    M = T * k
    gen = torch.Generator().manual_seed(seed)
    tgen = gen if device is None else torch.Generator(device=device).manual_seed(seed)
    x = _randn_bf16(tgen, (T, H))
    W1 = _randn_bf16(tgen, (E, 2 * F, H), W_STD)
    W2 = _randn_bf16(tgen, (E, H, F), W_STD)
    routing = cfg.get("routing", "zipf")
    if routing == "zipf":
        counts = zipf_counts(M, E, cfg.get("zipf_s", 1.1))
        ids, w = slot_grid_routing(counts, T, k, gen)
    elif routing == "skewed_empty":
        counts = skewed_counts_with_empty(M, E, cfg.get("max_share", 0.12), T)
        ids, w = slot_grid_routing(counts, T, k, gen)
    elif routing == "counts":
        ids, w = slot_grid_routing(np.asarray(cfg["counts"]), T, k, gen)
    elif routing == "topk_normal":
        logits = torch.randn(T, E, generator=gen, dtype=torch.float64).numpy()
        ids, w = topk_softmax_routing(logits, k)
    else:
        raise ValueError(routing)
    tok, r, counts, offs = sort_by_expert(ids, w, E)
    dY = _randn_bf16(tgen, (M, H)) if with_dy else None
    tok_t = torch.from_numpy(tok).to(x.device)
    r_t, off_t = torch.from_numpy(r), torch.from_numpy(offs)
    if device is not None:
        r_t, off_t = r_t.to(device), off_t.to(device)
    return MlpCase(X=x[tok_t].contiguous(), W1=W1, W2=W2, r=r_t, offsets=off_t,
                   dY=dY, counts=counts, token=tok, T=T, k=k)
