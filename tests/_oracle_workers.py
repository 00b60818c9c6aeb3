"""Oracle jobs run in worker processes by the full-size parity tests (CPU
only: these processes never touch the GPU).

An expert's slice of the fused GroupedMLP depends only on that expert's rows,
weights, routing weights and output gradients: every GEMM is grouped per
expert and the token-axis blocks restart at each expert's first row.  So the
oracle run on one expert alone (offsets [0, n]) gives exactly that expert's
Y, dX, dr, dW1[e] and dW2[e] of the full computation.  Run on a subset of an
expert's rows it gives those rows' Y, dX and dr exactly (they are row-local);
its weight gradients then belong to the subset and are not compared."""
import numpy as np

from oracle import mx_oracle as O


def expert_reference(X, W1e, W2e, r, dY):
    """X [n, H], W1e [2F, H], W2e [H, F], r [n], dY [n, H] (bf16 values as
    float32) -> (Y, dX, dr, dW1e, dW2e) in float64."""
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    X, W1e, W2e, r, dY = f64(X), f64(W1e), f64(W2e), f64(r), f64(dY)
    off = np.array([0, X.shape[0]], dtype=np.int64)
    Y, saved = O.grouped_mlp_fwd(X, W1e[None], W2e[None], r, off)
    g = O.grouped_mlp_bwd(dY, X, W1e[None], W2e[None], r, off, saved)
    return Y, g["dX"], g["dr"], g["dW1"][0], g["dW2"][0]
