"""Sketch construction: the tables and index stream of a layer from its dense weights.

SpaLLM section 2.2 ("Weighted Lloyd's algorithm for learning sketched
parameters", "Learning the sketching matrix") and the Sketch to Adapt reply to
Concern 1: the tables are weighted Lloyd centroids per (row, group), each
weight counted with 1 / [H^-1]_jj of its column; the indices come from a
sweep over the columns that maps each weight to its nearest entry and spreads
its error over the later columns with the update of Frantar et al.

H = X^T X of sample inputs X of the layer, plus a damping of ``damp`` times
its mean diagonal (the pages do not say how H is kept invertible; 1 % is
GPTQ's choice). H is one plain float64 GEMM (the vendor BLAS through
torch.matmul); the upper-triangular factor U (H^-1 = U^T U) and the three
sketching steps run in the HIP library: the factor (blocked Cholesky and
triangular inverse in float64), column weights, Lloyd, and the mapping sweep.
"""
from __future__ import annotations

import torch

from . import _lib


def hessian_factor(Xs, damp: float = 0.01):
    """Upper-triangular U (fp32, [d, d]) with U^T U = (X^T X + damp * mean(diag) * I)^-1."""
    X = Xs.to(torch.float64)
    return _lib.sketch_hessian_factor(X.T @ X, damp)


def build_sketch(W, b: int, gpr: int, Xs=None, U=None, iters: int = 30, lut_dtype=torch.float16,
                 damp: float = 0.01):
    """(idx_packed [n, d*b/8] uint8, lut [n, gpr, 2^b] lut_dtype) of the fp32 weights W [n, d].

    Give either the sample inputs Xs [s, d] or the factor U. W is not modified.
    """
    if U is None:
        if Xs is None:
            raise ValueError("build_sketch needs the sample inputs Xs or the factor U")
        U = hessian_factor(Xs, damp)
    W = W.to(torch.float32).contiguous()
    h = _lib.sketch_column_weights(U)
    lut = _lib.sketch_lloyd(W, h, b, gpr, iters, lut_dtype=lut_dtype)
    idx = _lib.sketch_map(W.clone(), U, lut, b, gpr)
    return idx, lut
