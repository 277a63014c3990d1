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
