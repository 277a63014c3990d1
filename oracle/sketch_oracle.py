"""CPU oracle for the sketched-weight matrix multiply (float64, numpy).

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The library itself never
calls it, and this module imports nothing from the library: it shares no code,
tables or constants with the HIP path.

What is computed, and where the pages define it
------------------------------------------------
Sources: "SpaLLM: Unified Compressive Adaptation of Large Language Models with
Sketching" (arXiv 2410.06364v1; called *SpaLLM* below) and the OpenReview
discussion of the same method, "Sketch to Adapt: Fine-Tunable Sketches for
Efficient LLM Adaptation" (called *Sketch to Adapt* below).

* Row-wise sketch (SpaLLM, section 2.2, Eq. (1)): a weight row theta in R^d is
  approximated as Pi w, where w in R^k is the sketched parameter (the lookup
  table) and Pi in R^{d x k} has one-hot rows. Storing the position of the one
  in each row of Pi as a b-bit integer gives ``idx[i, j]`` with k = 2^b, so
  ``W[i, j] = w_i[idx[i, j]]``.
* Groups per row (SpaLLM, section 2.2, "Scaling up learning power ..."; Sketch
  to Adapt, reply W2 on sub-rows): each row is cut into ``gpr`` contiguous,
  non-overlapping sub-rows of ``d / gpr`` columns, each with its own table, so
  ``W[i, j] = LUT[i, j // (d / gpr), idx[i, j]]``.
* Forward (SpaLLM, abstract and section 2.3: a single compressed matmul per
  layer; Sketch to Adapt, reply on Eq. (6): y = w M X): with tokens as rows of
  X, ``Y = X W^T``.
* Gradient of the tables (Sketch to Adapt, corrected Eq. (6)):
  dL/dw = dL/dy (M X)^T. For row i this sums ``dW[i, j] = sum_t dY[t, i]
  X[t, j]`` over the columns that map to each table entry:
  ``dLUT[i, g, c] = sum_{j in g, idx[i, j] = c} dW[i, j]``. The mapping Pi is
  frozen (SpaLLM, section 2.3), so there is no gradient for the indices.
* Gradient of the input: the chain rule through ``Y = X W^T`` gives
  ``dX = dY W``; the pages use it implicitly to train lower layers.
* Several adapters over one mapping (SpaLLM, section 2.3, the paragraph on
  dynamic maintenance of multiple adapters): each task owns its own set of
  tables in the same format while the mapping Pi is shared, so a batch can mix
  tasks; token t then uses table set s(t): ``Y[t, i] = sum_j X[t, j]
  W_{s(t)}[i, j]``.

* Fine-tuning updates only the tables (SpaLLM, section 2.3); the pages list
  the learning rates tried (SpaLLM, appendix B.1, Table 7) but name no
  optimizer. ``adam_step`` follows Adam as Kingma & Ba state it (their
  Algorithm 1: moment estimates, bias correction, step) with the decoupled
  weight decay of Loshchilov & Hutter (AdamW); ``sgd_step`` is gradient descent
  with heavy-ball momentum and an L2 term added to the gradient. Both work on
  fp32 master tables in the library; here they are carried in float64.

* Sketch construction (SpaLLM, section 2.2, "Weighted Lloyd's algorithm ..."
  and "Learning the sketching matrix"; Sketch to Adapt, reply to Concern 1):
  with H = X^T X from sample inputs X of the layer, the table of each (row,
  group) holds the k centroids of Lloyd's algorithm over the group's weights,
  each weight counted with weight 1 / [H^-1]_jj of its column; then the
  columns of the row are mapped one at a time, in order, to the nearest table
  entry, and the error of each mapped weight is spread over the columns not
  yet mapped by the update of Frantar et al. (GPTQ): with H^-1 = U^T U (U upper
  triangular), err = (w_j - q_j) / U_jj and w_{j'} -= err * U_{j j'} for
  j' > j. ``hessian_factor``, ``column_weights``, ``weighted_lloyd`` and
  ``map_error_compensated`` follow these steps.

Readings where the pages leave a step open (listed with the design notes):
the packed bit order is little-endian (field j at bits b*j .. b*j+b-1 of the
row's byte stream, LSB first); gradients of shared entries are summed, as the
chain rule of the corrected Eq. (6) gives, not averaged.

Every function here is pinned in ``tests/test_oracle_pins.py`` against facts
the pages or plain mathematics fix (the identity example, a dense special case,
finite differences, invariants, brute force on tiny inputs).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# index stream
# ---------------------------------------------------------------------------

def unpack_indices(idx_packed: np.ndarray, d: int, b: int) -> np.ndarray:
    """b-bit little-endian fields of each row's byte stream -> int64 ``[n][d]``.

    Bit p of a row's stream is bit ``p % 8`` of byte ``p // 8``; field j is the
    integer whose bit q is stream bit ``b*j + q``.
    """
    packed = np.ascontiguousarray(idx_packed, dtype=np.uint8)
    n = packed.shape[0]
    if packed.shape[1] * 8 < d * b:
        raise ValueError("packed rows too short for d*b bits")
    bits = np.unpackbits(packed, axis=1, bitorder="little")[:, : d * b]
    fields = bits.reshape(n, d, b).astype(np.int64)
    weights = (1 << np.arange(b, dtype=np.int64))
    return fields @ weights


def pack_indices(idx: np.ndarray, b: int) -> np.ndarray:
    """Inverse of :func:`unpack_indices`: int ``[n][d]`` in ``[0, 2^b)`` -> uint8 stream."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    if idx.min(initial=0) < 0 or idx.max(initial=0) >= (1 << b):
        raise ValueError("index out of range for b bits")
    if (d * b) % 8:
        raise ValueError("d*b must be a multiple of 8")
    bits = ((idx[:, :, None] >> np.arange(b, dtype=np.int64)) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(n, d * b), axis=1, bitorder="little")


# ---------------------------------------------------------------------------
# dequantisation (SpaLLM Eq. (1) with groups per row)
# ---------------------------------------------------------------------------

def group_of_column(d: int, gpr: int) -> np.ndarray:
    """g(j) = floor(j / (d / gpr)): contiguous, equal, non-overlapping sub-rows."""
    if gpr < 1 or d % gpr:
        raise ValueError("d must be a multiple of gpr")
    return np.arange(d, dtype=np.int64) // (d // gpr)


def dequantize(idx_packed: np.ndarray, lut: np.ndarray, d: int, b: int, gpr: int) -> np.ndarray:
    """W[i, j] = LUT[i, g(j), idx[i, j]] in float64 (exact for f32/f16/bf16 tables)."""
    lut = np.asarray(lut, dtype=np.float64)
    n = lut.shape[0]
    if lut.shape != (n, gpr, 1 << b):
        raise ValueError(f"lut shape {lut.shape} != {(n, gpr, 1 << b)}")
    idx = unpack_indices(idx_packed, d, b)
    g = group_of_column(d, gpr)
    rows = np.arange(n, dtype=np.int64)[:, None]
    return lut[rows, g[None, :], idx]


# ---------------------------------------------------------------------------
# forward and backward
# ---------------------------------------------------------------------------

def forward(X: np.ndarray, idx_packed: np.ndarray, lut: np.ndarray, b: int, gpr: int) -> np.ndarray:
    """Y[t, i] = sum_j X[t, j] W[i, j]  (float64)."""
    X = np.asarray(X, dtype=np.float64)
    W = dequantize(idx_packed, lut, X.shape[1], b, gpr)
    return X @ W.T


def forward_multi(X: np.ndarray, idx_packed: np.ndarray, luts: np.ndarray, lut_set, b: int,
                  gpr: int) -> np.ndarray:
    """Y[t, i] = sum_j X[t, j] W_{s(t)}[i, j], with W_s dequantised from table
    set luts[s] over the shared indices and s(t) = lut_set[t]  (float64)."""
    X = np.asarray(X, dtype=np.float64)
    luts = np.asarray(luts)
    m, d = X.shape
    Y = np.zeros((m, idx_packed.shape[0]), dtype=np.float64)
    for t in range(m):
        W = dequantize(idx_packed, luts[int(lut_set[t])], d, b, gpr)
        Y[t] = W @ X[t]
    return Y


def backward_dx(dY: np.ndarray, idx_packed: np.ndarray, lut: np.ndarray, d: int, b: int, gpr: int) -> np.ndarray:
    """dX[t, j] = sum_i dY[t, i] W[i, j]  (float64)."""
    dY = np.asarray(dY, dtype=np.float64)
    W = dequantize(idx_packed, lut, d, b, gpr)
    return dY @ W


def weight_gradient(dY: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Gradient of every virtual parameter: dW[i, j] = sum_t dY[t, i] X[t, j]."""
    return np.asarray(dY, dtype=np.float64).T @ np.asarray(X, dtype=np.float64)


def backward_dlut_loop(dY: np.ndarray, X: np.ndarray, idx_packed: np.ndarray, b: int, gpr: int) -> np.ndarray:
    """dLUT by an explicit loop over every virtual parameter (tiny shapes only).

    Each virtual parameter W[i, j] hands its gradient to the table entry it is
    mapped to; entries shared by several columns receive the sum.
    """
    dW = weight_gradient(dY, X)
    n, d = dW.shape
    idx = unpack_indices(idx_packed, d, b)
    g = group_of_column(d, gpr)
    out = np.zeros((n, gpr, 1 << b), dtype=np.float64)
    for i in range(n):
        for j in range(d):
            out[i, g[j], idx[i, j]] += dW[i, j]
    return out


def backward_dlut(dY: np.ndarray, X: np.ndarray, idx_packed: np.ndarray, b: int, gpr: int) -> np.ndarray:
    """Same sum as :func:`backward_dlut_loop`, binned row by row with ``np.bincount``."""
    dW = weight_gradient(dY, X)
    n, d = dW.shape
    k = 1 << b
    idx = unpack_indices(idx_packed, d, b)
    g = group_of_column(d, gpr)
    out = np.empty((n, gpr, k), dtype=np.float64)
    for i in range(n):
        out[i] = np.bincount(g * k + idx[i], weights=dW[i], minlength=gpr * k).reshape(gpr, k)
    return out


# ---------------------------------------------------------------------------
# scoring
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# sketch construction (the step before the path)
# ---------------------------------------------------------------------------

def hessian_factor(Xs: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """Upper-triangular U with U^T U = (X^T X + damp * mean(diag) * I)^-1, float64 ``[d][d]``.

    X^T X of the sample inputs ``Xs`` ``[s][d]``; the damping term keeps it invertible (the pages do not
    say; 1 % of the mean diagonal is GPTQ's choice).
    """
    X = np.asarray(Xs, dtype=np.float64)
    H = X.T @ X
    H = H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    Hinv = np.linalg.inv(H)
    L = np.linalg.cholesky(Hinv)      # Hinv = L L^T
    return L.T


def column_weights(U: np.ndarray) -> np.ndarray:
    """1 / [H^-1]_jj for every column, from the factor U (H^-1 = U^T U, so [H^-1]_jj = sum_k U_kj^2)."""
    U = np.asarray(U, dtype=np.float64)
    return 1.0 / np.sum(U * U, axis=0)


def lloyd_init(x: np.ndarray, k: int) -> np.ndarray:
    """k starting centroids spread evenly over [min x, max x] (cell midpoints)."""
    lo, hi = float(np.min(x)), float(np.max(x))
    return lo + (np.arange(k, dtype=np.float64) + 0.5) * ((hi - lo) / k)


def lloyd_group(x: np.ndarray, wt: np.ndarray, k: int, iters: int):
    """Weighted Lloyd's algorithm on one group: (centroids, iterations run).

    Each iteration assigns every value to its nearest centroid (ties to the lower index) and moves every
    centroid to the weighted mean of its values; a centroid with no values stays. Stops after ``iters``
    iterations or when the centroids no longer change.
    """
    x = np.asarray(x, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    c = lloyd_init(x, k)
    for it in range(iters):
        a = np.argmin(np.abs(x[:, None] - c[None, :]), axis=1)
        sw = np.bincount(a, weights=wt, minlength=k)
        swx = np.bincount(a, weights=wt * x, minlength=k)
        new = np.where(sw > 0, swx / np.where(sw > 0, sw, 1.0), c)
        if np.array_equal(new, c):
            return c, it
        c = new
    return c, iters


def weighted_lloyd(W: np.ndarray, h: np.ndarray, gpr: int, k: int, iters: int) -> np.ndarray:
    """Tables ``[n][gpr][k]``: weighted Lloyd centroids of every (row, group); column j weighs h[j]."""
    W = np.asarray(W, dtype=np.float64)
    n, d = W.shape
    G = d // gpr
    out = np.empty((n, gpr, k), dtype=np.float64)
    for i in range(n):
        for g in range(gpr):
            out[i, g], _ = lloyd_group(W[i, g * G:(g + 1) * G], h[g * G:(g + 1) * G], k, iters)
    return out


def map_error_compensated(W: np.ndarray, U: np.ndarray, lut: np.ndarray, gpr: int) -> np.ndarray:
    """Indices ``[n][d]``: columns in order, each weight to its nearest table entry (ties to the lower
    index) after the errors of the columns before it were spread by the update err = (w_j - q_j) / U_jj,
    w_{j'} -= err * U_{j j'} (j' > j)."""
    w = np.array(W, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    lut = np.asarray(lut, dtype=np.float64)
    n, d = w.shape
    G = d // gpr
    rows = np.arange(n)
    idx = np.empty((n, d), dtype=np.int64)
    for j in range(d):
        t = lut[:, j // G, :]
        a = np.argmin(np.abs(w[:, j:j + 1] - t), axis=1)
        idx[:, j] = a
        err = (w[:, j] - t[rows, a]) / U[j, j]
        w[:, j + 1:] -= err[:, None] * U[j, j + 1:][None, :]
    return idx


# ---------------------------------------------------------------------------
# optimizer steps on the tables (textbook rules; the pages name none)
# ---------------------------------------------------------------------------

def adam_step(master: np.ndarray, grad: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray, step: int,
              lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
              grad_scale: float = 1.0):
    """One Adam step with decoupled weight decay; returns (master, exp_avg, exp_avg_sq) as new float64 arrays.

    Kingma & Ba, Algorithm 1: m <- beta1 m + (1 - beta1) g; v <- beta2 v + (1 - beta2) g^2;
    m_hat = m / (1 - beta1^t); v_hat = v / (1 - beta2^t); theta <- theta - lr m_hat / (sqrt(v_hat) + eps).
    The decay shrinks theta by (1 - lr * weight_decay) before the step (Loshchilov & Hutter).
    """
    p = np.asarray(master, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64) * grad_scale
    m = beta1 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(exp_avg_sq, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p * (1.0 - lr * weight_decay)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def sgd_step(master: np.ndarray, grad: np.ndarray, lr: float, momentum: float = 0.0, weight_decay: float = 0.0,
             grad_scale: float = 1.0, momentum_buf=None):
    """One SGD step; returns (master, momentum_buf) as new float64 arrays (buf None without momentum).

    g = grad * grad_scale + weight_decay * theta; with momentum, buf <- momentum * buf + g and the step
    uses buf (a zero buffer before the first step makes the first step use g itself); theta <- theta - lr g.
    """
    p = np.asarray(master, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64) * grad_scale + weight_decay * p
    buf = None
    if momentum != 0.0:
        prev = np.zeros_like(p) if momentum_buf is None else np.asarray(momentum_buf, dtype=np.float64)
        buf = momentum * prev + g
        g = buf
    return p - lr * g, buf


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero).

    The parity score of every comparison with this oracle: the largest
    absolute error over the largest absolute reference value, both taken over
    the whole output tensor. The pages print no tolerance rule; this is the
    acceptance measure stated for the path (5e-3 for 16-bit inputs, 1e-5 for
    fp32). Shapes must match exactly (no broadcasting); an all-zero reference
    scores 0 against an exact result and infinity against anything else.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
