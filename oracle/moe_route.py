"""FP64 CPU oracle for the steps on either side of the expert path: the
token sort that gathers each expert's rows, and the combine that brings the
expert outputs back to token order.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it imports nothing from the product path.

Sources (cited by page title): "MoE-Training für biologische Grundmodelle
optimieren" (hyper.ai, German) -- the paragraph on GroupedLinear: the caller
hands over the number of tokens of every expert and the expert inputs are
gathered into one grouped call; "NVIDIA apresenta técnicas para tornar mais
eficiente o treinamento de modelos biológicos baseados em arquitetura MoE"
(conexaotc, Portuguese) -- third paragraph: the routing weights send each
token to its experts, and the GroupedMLP applies the routing-weight scaling
itself.

The pages give no algorithm for either step.  Readings (also listed in the
design notes of the repository):

* R-sort     token t's k routing slots (expert ids[t, j]) become M = T*k
             rows sorted stably by (expert, token, slot): expert e owns rows
             [offsets[e], offsets[e+1]); within an expert, tokens keep their
             order, and a token routed twice to one expert keeps slot order.
* R-combine  out[t] = sum_j c[t, j] * Y[row_of[t, j]] with c = w (the routing
             weights) when the expert path did not apply them, or c = 1 when it
             did (the GroupedMLP scales z by r); j ascending.
* R-router   token t's experts are its k largest logits, taken one at a time
             (the largest remaining, the lower expert index among equal
             values), and its routing weights are the softmax of those k
             logits.
* R-bwd      the combine's backward: dY[row_of[t, j]] = c[t, j] * dout[t], and
             for the weighted combine dw[t, j] = <dout[t], Y[row_of[t, j]]>.
             Gathering token rows into sorted order (the permute) is the same
             map as this dY with c = 1.

Functions are float64/int64, written for reading; the one library primitive
used as a step is numpy's stable sort.

Functions with no independent pin: none (see tests/test_oracle_moe_route.py).
"""
from __future__ import annotations

import numpy as np


def router_topk_softmax(logits, k):
    """Top-k experts of every token and the softmax of their logits (R-router).

    logits [T, E].  Returns ids int64 [T, k] (selection order) and w float64
    [T, k].
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k))
    for t in range(T):
        taken = [False] * E
        for j in range(k):
            best = -1
            for e in range(E):
                if not taken[e] and (best < 0 or logits[t, e] > logits[t, best]):
                    best = e                      # strictly larger: ties keep the lower index
            taken[best] = True
            ids[t, j] = best
        sel = logits[t, ids[t]]
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
    return ids, w


def route_plan(ids, E):
    """Sorted-row plan of a top-k routing (R-sort).

    ids int [T, k] with values in [0, E).  Returns offsets int64 [E+1],
    row_of int64 [T, k] (the sorted row of each slot) and tok_of int64 [M]
    (the token of each sorted row).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)                       # slot t*k + j, token order
    order = np.argsort(flat, kind="stable")      # sorted row -> slot
    row_of = np.empty(T * k, dtype=np.int64)
    row_of[order] = np.arange(T * k)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return offsets, row_of.reshape(T, k), order // k


def sorted_weights(w, row_of):
    """Routing weight of every sorted row: r[row_of[t, j]] = w[t, j]."""
    w = np.asarray(w, dtype=np.float64)
    r = np.empty(w.size, dtype=np.float64)
    r[np.asarray(row_of).reshape(-1)] = w.reshape(-1)
    return r


def permute_rows(x, tok_of):
    """Token rows in sorted order: X_sorted[row] = x[tok_of[row]]."""
    return np.asarray(x, dtype=np.float64)[np.asarray(tok_of)]


def combine(y, row_of, w=None):
    """out[t] = sum_j c[t, j] * y[row_of[t, j]], j ascending (R-combine)."""
    y = np.asarray(y, dtype=np.float64)
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        c = 1.0 if w is None else np.asarray(w, dtype=np.float64)[:, j:j + 1]
        out += c * y[row_of[:, j]]
    return out


def combine_bwd(dout, row_of, w=None, y=None):
    """Backward of combine (R-bwd).  Returns dY [M, H] and, for the weighted
    combine (w given, y needed), dw [T, k]."""
    dout = np.asarray(dout, dtype=np.float64)
    row_of = np.asarray(row_of)
    T, k = row_of.shape
    dy = np.zeros((T * k, dout.shape[1]))
    dw = None if w is None else np.zeros((T, k))
    for j in range(k):
        c = 1.0 if w is None else np.asarray(w, dtype=np.float64)[:, j:j + 1]
        dy[row_of[:, j]] = c * dout
        if w is not None:
            dw[:, j] = np.sum(dout * np.asarray(y, dtype=np.float64)[row_of[:, j]], axis=1)
    return dy, dw
