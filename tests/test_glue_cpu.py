"""Host-side checks of the fine-tuning and construction glue (no GPU): CPU tensors are refused before
any library call, so no step can silently run on the host."""
import numpy as np
import pytest
import torch

from lut_sketched_matmul_amd import construct, finetune
from lut_sketched_matmul_amd import synthetic as syn


def _layer_inputs():
    idx = torch.from_numpy(syn.random_packed_indices("cpu-glue/idx", 16, 256, 4))
    lut = torch.from_numpy(syn.random_lut("cpu-glue/lut", 16, 2, 4, 0.02, "f32"))
    return idx, lut


def test_sketched_linear_refuses_host_tensors():
    idx, lut = _layer_inputs()
    layer = finetune.SketchedLinear(idx, lut, 256, 4, 2)
    assert layer.lut_master.dtype == torch.float32 and layer.lut.dtype == torch.float16
    with pytest.raises(ValueError, match="GPU"):
        layer(torch.zeros(2, 256, dtype=torch.float16))


def test_sketched_linear_checks_shapes():
    idx, lut = _layer_inputs()
    with pytest.raises(ValueError):
        finetune.SketchedLinear(idx, lut[:, :1], 256, 4, 2)       # tables of 1 group, gpr = 2
    with pytest.raises(ValueError):
        finetune.SketchedLinear(idx, lut, 512, 4, 2)              # d does not match the packed rows


def test_optimizers_refuse_host_tensors():
    p = torch.nn.Parameter(torch.zeros(64))
    p.grad = torch.ones(64)
    with pytest.raises(ValueError, match="GPU"):
        finetune.LutAdam([p], lr=1e-3).step()
    with pytest.raises(ValueError, match="GPU"):
        finetune.LutSGD([p], lr=1e-3, momentum=0.9).step()


def test_construction_refuses_host_tensors():
    W = torch.zeros(16, 256)
    U = torch.eye(256)
    with pytest.raises(ValueError, match="GPU"):
        construct.build_sketch(W, 4, 2, U=U)
    assert np.all(W.numpy() == 0)


# ---- the binding checks every tensor against the sizes it passes to the C ABI
# (host tensors of the right shape get past these checks and are then refused
# as host memory, so a shape error is always reported first)

from lut_sketched_matmul_amd import _lib  # noqa: E402


def _mm_inputs(m=4, n=16, d=256, b=4, gpr=2, dt=torch.float16):
    X = torch.zeros(m, d, dtype=dt)
    idx = torch.zeros(n, d * b // 8, dtype=torch.uint8)
    lut = torch.zeros(n, gpr, 1 << b, dtype=torch.float16)
    dY = torch.zeros(m, n, dtype=dt)
    return X, idx, lut, dY


def test_fwd_checks_shapes_before_the_call():
    X, idx, lut, _ = _mm_inputs()
    with pytest.raises(ValueError, match="GPU"):
        _lib.sketch_matmul_fwd(X, idx, lut, 4, 2)                     # right shapes: refused as host memory
    with pytest.raises(ValueError, match="out"):
        _lib.sketch_matmul_fwd(X, idx, lut, 4, 2, out=torch.zeros(4, 15, dtype=torch.float16))
    with pytest.raises(TypeError, match="out"):
        _lib.sketch_matmul_fwd(X, idx, lut, 4, 2, out=torch.zeros(4, 16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lut"):
        _lib.sketch_matmul_fwd(X, idx, lut[:, :1], 4, 2)              # one group's tables for gpr = 2
    with pytest.raises(ValueError, match="idx_packed"):
        _lib.sketch_matmul_fwd(X, idx[:, :64], lut, 4, 2)             # rows of 128 columns for d = 256
    with pytest.raises(TypeError, match="idx_packed"):
        _lib.sketch_matmul_fwd(X, idx.to(torch.int16), lut, 4, 2)
    with pytest.raises(ValueError, match="bit width"):
        _lib.sketch_matmul_fwd(X, idx, lut, 5, 2)
    with pytest.raises(ValueError, match="matrix"):
        _lib.sketch_matmul_fwd(X[0], idx, lut, 4, 2)


def test_fwd_multi_checks_shapes():
    X, idx, lut, _ = _mm_inputs()
    luts = torch.stack([lut, lut])
    sets = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        _lib.sketch_matmul_fwd_multi(X, idx, luts, sets, 4, 2)
    with pytest.raises(ValueError, match="luts"):
        _lib.sketch_matmul_fwd_multi(X, idx, luts[:, :8], sets, 4, 2)
    with pytest.raises(ValueError, match="lut_set"):
        _lib.sketch_matmul_fwd_multi(X, idx, luts, sets[:3], 4, 2)


def test_bwd_checks_shapes_and_dtypes():
    X, idx, lut, dY = _mm_inputs()
    with pytest.raises(ValueError, match="GPU"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut, 4, 2)
    with pytest.raises(TypeError, match="X"):
        _lib.sketch_matmul_bwd(dY.float(), X, idx, lut, 4, 2)         # fp32 dY with 16-bit X
    with pytest.raises(ValueError, match="X"):
        _lib.sketch_matmul_bwd(dY, X[:3], idx, lut, 4, 2)             # X of 3 tokens, dY of 4
    with pytest.raises(ValueError, match="dlut_out"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut, 4, 2, dlut_out=torch.zeros(16, 2, 8))
    with pytest.raises(TypeError, match="dlut_out"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut, 4, 2, dlut_out=torch.zeros(16, 2, 16, dtype=torch.float16))
    with pytest.raises(ValueError, match="lut"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut[:8], 4, 2)
    with pytest.raises(ValueError, match="idx_packed"):
        _lib.sketch_matmul_bwd(dY, X, idx[:15], lut, 4, 2)            # dY has 16 output columns
    with pytest.raises(ValueError, match="needs X"):
        _lib.sketch_matmul_bwd(dY, None, idx, lut, 4, 2, d=256)
    with pytest.raises(ValueError, match="d = 128"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut, 4, 2, d=128)
    with pytest.raises(TypeError, match="workspace"):
        _lib.sketch_matmul_bwd(dY, X, idx, lut, 4, 2, workspace=torch.zeros(64, dtype=torch.float32))


def test_checking_aids_and_construction_check_shapes():
    _, idx, lut, _ = _mm_inputs()
    with pytest.raises(ValueError, match="idx_packed"):
        _lib.sketch_dequant(idx, lut, 512, 4, 2)
    with pytest.raises(ValueError, match="idx_packed"):
        _lib.sketch_unpack_indices(idx, 512, 4)
    W = torch.zeros(16, 256)
    with pytest.raises(ValueError, match="h"):
        _lib.sketch_lloyd(W, torch.ones(255), 4, 2, 10)
    with pytest.raises(ValueError, match="U"):
        _lib.sketch_map(W, torch.eye(255), lut, 4, 2)
    with pytest.raises(ValueError, match="U"):
        _lib.sketch_column_weights(torch.zeros(4, 5))
