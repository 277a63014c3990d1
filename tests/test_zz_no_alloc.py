"""The backward entry point that allocates nothing (library-owned scratch) against sketch_matmul_bwd.

Two calls in a row on one GPU, the second smaller, each compared with sketch_matmul_bwd on the same
inputs (bit-identical: the same kernels) and with the oracle (the 16-bit tolerance). The cases need
scratch: row exponents of bf16 dY with f16 tables, and the table gradient split over token ranges.
"""
import numpy as np
import pytest

import oracle
from lut_sketched_matmul_amd import synthetic as syn

from gpu_util import to_dev, to_f64

pytestmark = pytest.mark.gpu

TOL16 = 5e-3


def _case(tag, n, d, b, gpr, m, io, lut_dtype):
    idx = syn.random_packed_indices(f"{tag}/idx", n, d, b)
    lut = syn.random_lut(f"{tag}/lut", n, gpr, b, 0.02, lut_dtype)
    X = syn.random_normal(f"{tag}/X", (m, d), 1.0, io)
    dY = syn.random_normal(f"{tag}/dY", (m, n), 1e-2, io)
    return idx, lut, X, dY


def test_noalloc_matches_bwd_twice():
    import torch
    import lut_sketched_matmul_amd as skm
    from lut_sketched_matmul_amd import _lib
    cases = [("noalloc/big", 256, 1024, 4, 1, 640, "bf16", "f16"),     # exponents + 5 token ranges
             ("noalloc/small", 128, 512, 2, 1, 320, "bf16", "f16")]    # exponents + 2 token ranges
    for tag, n, d, b, gpr, m, io, ldt in cases:
        assert _lib.sketch_matmul_bwd_workspace(m, n, d, b, gpr, _lib.SKM_BF16, _lib.SKM_F16) > m * 4
        idx, lut, X, dY = _case(tag, n, d, b, gpr, m, io, ldt)
        gi, gl, gx, gdy = to_dev(idx, "u8"), to_dev(lut, ldt), to_dev(X, io), to_dev(dY, io)
        dX = torch.full((m, d), float("nan"), dtype=torch.float32, device="cuda:0")
        dL = torch.full((n, gpr, 1 << b), float("nan"), dtype=torch.float32, device="cuda:0")
        _lib.sketch_matmul_bwd_noalloc(gdy, gx, gi, gl, b, gpr, dx_out=dX, dlut_out=dL)
        rX, rL = skm.sketch_matmul_bwd(gdy, gx, gi, gl, b, gpr)
        torch.cuda.synchronize()
        assert bool((dX == rX).all()) and bool((dL == rL).all()), tag
        L64, X64, dY64 = syn.to_float64(lut, ldt), syn.to_float64(X, io), syn.to_float64(dY, io)
        assert oracle.rel_err(to_f64(dX), oracle.backward_dx(dY64, idx, L64, d, b, gpr)) <= TOL16
        assert oracle.rel_err(to_f64(dL), oracle.backward_dlut(dY64, X64, idx, b, gpr)) <= TOL16


def test_noalloc_accumulate():
    import torch
    import lut_sketched_matmul_amd as skm
    from lut_sketched_matmul_amd import _lib
    n, d, b, gpr, m = 256, 1024, 4, 1, 640
    idx, lut, X, dY = _case("noalloc/acc", n, d, b, gpr, m, "bf16", "f16")
    gi, gl, gx, gdy = to_dev(idx, "u8"), to_dev(lut, "f16"), to_dev(X, "bf16"), to_dev(dY, "bf16")
    base = torch.from_numpy(np.random.default_rng(1).normal(size=(n, gpr, 16)).astype(np.float32)).to("cuda:0")
    got = base.clone()
    _lib.sketch_matmul_bwd_noalloc(gdy, gx, gi, gl, b, gpr, dlut_out=got, accumulate=True)
    want = base.clone()
    skm.sketch_matmul_bwd(gdy, gx, gi, gl, b, gpr, need_dx=False, dlut_out=want, accumulate=True)
    torch.cuda.synchronize()
    assert bool((got == want).all())
