"""Fine-tuning glue: autograd, trainable sketched layers and table optimizers.

Fine-tuning trains only the table values; the mapping stays frozen (SpaLLM,
section 2.3). A :class:`SketchedLinear` keeps the trained values as an fp32
master :class:`torch.nn.Parameter` and a 16-bit compute copy that the forward
and backward kernels read. Its gradient is the fp32 table gradient of the
backward kernel. :class:`LutAdam` and :class:`LutSGD` update the master and
refresh the copy in one fused pass. The pages list the learning rates they
tried (SpaLLM, appendix B.1, Table 7) but name no optimizer.

Every compute step runs in the HIP library (forward, dX, dLUT, optimizer
step); this module only marshals arguments. Two small torch operations remain
in the glue: the fp32 input gradient is cast to the activations' dtype (autograd
requires a gradient in its input's dtype), and a grouped layer's output
gradient is made contiguous before the backward launch.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence

import torch

from . import _lib


class SketchMatmulFunction(torch.autograd.Function):
    """Y = X Wᵀ with W[i, j] = lut[i, j // G, idx[i, j]]; gradients for X and the master tables.

    Inputs: X [m, d]; lut_master [n, gpr, 2^b] fp32 (receives dLUT); lut [n, gpr, 2^b], the compute
    copy the kernels read (fp32 for the fp32 path, else f16/bf16); idx_packed [n, d*b/8] uint8.
    """

    @staticmethod
    def forward(ctx, X, lut_master, lut, idx_packed, b: int, gpr: int):
        Y = _lib.sketch_matmul_fwd(X.contiguous(), idx_packed, lut, b, gpr)
        ctx.save_for_backward(X, lut, idx_packed)
        ctx.b, ctx.gpr = b, gpr
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, lut, idx_packed = ctx.saved_tensors
        need_dx, need_dlut = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_dx or need_dlut):
            return None, None, None, None, None, None
        dY = dY.contiguous()
        if dY.dtype != X.dtype:
            raise TypeError("the output gradient must have the activations' dtype")
        dX, dL = _lib.sketch_matmul_bwd(dY, X.contiguous() if need_dlut else None, idx_packed, lut, ctx.b, ctx.gpr,
                                        d=X.shape[1], need_dx=need_dx, need_dlut=need_dlut)
        if dX is not None and dX.dtype != X.dtype:
            dX = dX.to(X.dtype)
        return dX, dL, None, None, None, None


def sketch_matmul(X, lut_master, lut, idx_packed, b: int, gpr: int):
    """Functional form of :class:`SketchMatmulFunction`."""
    return SketchMatmulFunction.apply(X, lut_master, lut, idx_packed, b, gpr)


class SketchedLinear(torch.nn.Module):
    """A linear layer whose weight is a frozen mapping into trainable per-group tables.

    idx_packed: [n, d*b/8] uint8 on the GPU (frozen). lut: [n, gpr, 2^b] initial table values.
    compute_dtype: dtype of the copy the kernels read (torch.float16 / torch.bfloat16, or torch.float32
    for the fp32 path, where the master itself is read).
    """

    def __init__(self, idx_packed, lut, d: int, b: int, gpr: int, compute_dtype=torch.float16):
        super().__init__()
        n = idx_packed.shape[0]
        if tuple(lut.shape) != (n, gpr, 1 << b) or idx_packed.shape[1] * 8 != d * b:
            raise ValueError("table or index shape does not match (n, gpr, 2^b) / (n, d*b/8)")
        self.d, self.b, self.gpr = d, b, gpr
        self.register_buffer("idx_packed", idx_packed.contiguous())
        self.lut_master = torch.nn.Parameter(lut.detach().to(torch.float32).contiguous().clone())
        if compute_dtype == torch.float32:
            self.lut = None
        else:
            self.register_buffer("lut", self.lut_master.detach().to(compute_dtype))
        self._link_copy()

    def _link_copy(self) -> None:
        # the optimizers below find the compute copy through this attribute (set again on every
        # forward, since moving the module replaces its buffers but keeps the parameter object)
        self.lut_master._skm_copy = self.lut

    @property
    def out_features(self) -> int:
        return self.idx_packed.shape[0]

    def compute_tables(self):
        return self.lut if self.lut is not None else self.lut_master.detach()

    def refresh_copy(self) -> None:
        """Round the master into the compute copy (after changing the master outside the optimizers)."""
        if self.lut is not None:
            self.lut.copy_(self.lut_master.detach())

    def forward(self, X):
        self._link_copy()
        return sketch_matmul(X, self.lut_master, self.compute_tables(), self.idx_packed, self.b, self.gpr)


class GroupedSketchedLinear(torch.nn.Module):
    """Several sketched projections of the same input (q/k/v, gate/up) in one launch per pass.

    The projections' rows are stored back to back (indices and tables), so the forward, dX and dLUT
    each run as one launch over all rows; forward returns one view per projection.
    """

    def __init__(self, idx_list: Sequence, lut_list: Sequence, d: int, b: int, gpr: int,
                 compute_dtype=torch.float16):
        super().__init__()
        self.sizes = [int(i.shape[0]) for i in idx_list]
        self.inner = SketchedLinear(torch.cat([i.contiguous() for i in idx_list], 0),
                                    torch.cat([t.detach() for t in lut_list], 0), d, b, gpr, compute_dtype)

    @property
    def lut_master(self):
        return self.inner.lut_master

    def table_slices(self) -> List:
        """The master tables of each projection (views into the shared parameter)."""
        return list(torch.split(self.inner.lut_master, self.sizes, 0))

    def forward(self, X):
        Y = self.inner(X)
        return tuple(torch.split(Y, self.sizes, dim=1))


def _copy_of(p):
    return getattr(p, "_skm_copy", None)


class LutAdam(torch.optim.Optimizer):
    """Adam with decoupled weight decay on fp32 master tables, fused with the refresh of their compute copy.

    Parameters must be fp32 CUDA tensors; a master created by :class:`SketchedLinear` carries its copy.
    grad_scale multiplies every gradient (dLUT is a sum over tokens; e.g. 1/tokens gives a mean).
    """

    def __init__(self, params: Iterable, lr: float = 1e-5, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0, grad_scale: float = 1.0):
        super().__init__(params, dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay,
                                      grad_scale=grad_scale))

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        for group in self.param_groups:
            b1, b2 = group["betas"]
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                if not st:
                    st["step"] = 0
                    st["exp_avg"] = torch.zeros_like(p, memory_format=torch.contiguous_format)
                    st["exp_avg_sq"] = torch.zeros_like(p, memory_format=torch.contiguous_format)
                st["step"] += 1
                _lib.sketch_lut_adam_step(p, p.grad.contiguous(), st["exp_avg"], st["exp_avg_sq"], st["step"],
                                          group["lr"], b1, b2, group["eps"], group["weight_decay"],
                                          group["grad_scale"], lut=_copy_of(p))
        return loss


class LutSGD(torch.optim.Optimizer):
    """SGD (heavy-ball momentum, L2 weight decay) on fp32 master tables, fused with the copy refresh."""

    def __init__(self, params: Iterable, lr: float = 1e-3, momentum: float = 0.0, weight_decay: float = 0.0,
                 grad_scale: float = 1.0):
        super().__init__(params, dict(lr=lr, momentum=momentum, weight_decay=weight_decay, grad_scale=grad_scale))

    @torch.no_grad()
    def step(self, closure=None):
        loss = closure() if closure is not None else None
        for group in self.param_groups:
            for p in group["params"]:
                if p.grad is None:
                    continue
                st = self.state[p]
                buf: Optional[torch.Tensor] = None
                if group["momentum"] != 0.0:
                    if "momentum_buffer" not in st:
                        st["momentum_buffer"] = torch.zeros_like(p, memory_format=torch.contiguous_format)
                    buf = st["momentum_buffer"]
                _lib.sketch_lut_sgd_step(p, p.grad.contiguous(), group["lr"], group["momentum"],
                                         group["weight_decay"], group["grad_scale"], momentum_buf=buf,
                                         lut=_copy_of(p))
        return loss
