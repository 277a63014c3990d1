"""The synthetic LLaMA-shaped workloads the library is tested and measured on.

Each workload is a list of weight shapes (n rows = output features, d columns =
input features) sketched with b-bit indices and ``gpr`` groups per row, the
token counts m it runs at, the storage dtypes and the normal distributions its
tensors are drawn from. Shapes follow the public LLaMA-2-7B / 13B / LLaMA-3-70B
model configs (LLaMA-2-13B: hidden 5120, MLP 13824); every tensor is drawn by :mod:`lut_sketched_matmul_amd.synthetic`
under a name ``"<workload>/<shape>/<tensor>"``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

from . import synthetic as syn


@dataclass(frozen=True)
class Shape:
    name: str
    n: int
    d: int


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: Tuple[Shape, ...]
    bits: Tuple[int, ...]
    gpr: int
    lut_dtype: str
    lut_sigma: float
    x_dtype: str
    tokens: Tuple[int, ...]
    backward: bool
    dy_sigma: float = 1.0
    tol: float = 5e-3
    notes: str = ""

    def tensor_name(self, shape: Shape, b: int, tensor: str, m: int | None = None) -> str:
        tag = f"{self.name}/{shape.name}-b{b}"
        if m is not None:
            tag += f"-m{m}"
        return f"{tag}/{tensor}"

    def make(self, shape: Shape, b: int, m: int) -> Dict[str, object]:
        """Draw (idx_packed, lut, X[, dY]) for one shape, bit width and token count."""
        out: Dict[str, object] = {
            "n": shape.n, "d": shape.d, "b": b, "gpr": self.gpr, "m": m,
            "x_dtype": self.x_dtype, "lut_dtype": self.lut_dtype,
        }
        out["idx_packed"] = syn.random_packed_indices(self.tensor_name(shape, b, "idx"), shape.n, shape.d, b)
        out["lut"] = syn.random_lut(self.tensor_name(shape, b, "lut"), shape.n, self.gpr, b,
                                    self.lut_sigma, self.lut_dtype)
        out["X"] = syn.random_normal(self.tensor_name(shape, b, "X", m), (m, shape.d), 1.0, self.x_dtype)
        if self.backward:
            out["dY"] = syn.random_normal(self.tensor_name(shape, b, "dY", m), (m, shape.n),
                                          self.dy_sigma, self.x_dtype)
        return out


TINY = Workload(
    name="tiny-256x512",
    shapes=(Shape("w", 256, 512),),
    bits=(4,), gpr=1, lut_dtype="f32", lut_sigma=0.02, x_dtype="f32",
    tokens=(4,), backward=True, dy_sigma=1.0, tol=1e-5,
    notes="fp32 debug mode: forward and backward (dX, dLUT)",
)

LLAMA2_7B_ATTN = Workload(
    name="llama2-7b-attn-4096x4096",
    shapes=(Shape("qkvo", 4096, 4096),),
    bits=(4,), gpr=8, lut_dtype="f16", lut_sigma=0.02, x_dtype="f16",
    tokens=(1, 16), backward=False,
    notes="decode GEMV (m=1) and a 16-token forward",
)

LLAMA2_7B_MLP_LOWBIT = Workload(
    name="llama2-7b-mlp-lowbit",
    shapes=(Shape("gate_up", 11008, 4096), Shape("down", 4096, 11008)),
    bits=(2, 3), gpr=8, lut_dtype="f16", lut_sigma=0.02, x_dtype="f16",
    tokens=(1, 4, 16), backward=False,
    notes="2-bit and 3-bit (contiguous bitstream) indices",
)

LLAMA3_70B_MLP = Workload(
    name="llama3-70b-mlp",
    shapes=(Shape("up", 28672, 8192), Shape("down", 8192, 28672)),
    bits=(4,), gpr=4, lut_dtype="f16", lut_sigma=0.015, x_dtype="bf16",
    tokens=(1, 2048), backward=False,
    notes="decode at 1 token, prefill at 2048 tokens (MFMA path)",
)

LLAMA2_7B_FINETUNE = Workload(
    name="llama2-7b-layer-finetune",
    shapes=(Shape("q", 4096, 4096), Shape("k", 4096, 4096), Shape("v", 4096, 4096),
            Shape("o", 4096, 4096), Shape("gate", 11008, 4096), Shape("up", 11008, 4096),
            Shape("down", 4096, 11008)),
    bits=(4,), gpr=8, lut_dtype="f16", lut_sigma=0.02, x_dtype="bf16",
    tokens=(8192,), backward=True, dy_sigma=1e-2,
    notes="one decoder layer's seven projections: forward + dX + dLUT, fp32 gradients",
)

LLAMA2_13B_DECODE = Workload(
    name="llama2-13b-decode-gpr1",
    shapes=(Shape("qkvo", 5120, 5120), Shape("gate_up", 13824, 5120), Shape("down", 5120, 13824)),
    bits=(4,), gpr=1, lut_dtype="f16", lut_sigma=0.02, x_dtype="f16",
    tokens=(1, 16), backward=False,
    notes="the second model of the decode-efficiency comparison: 4-bit indices, one group per row",
)

LLAMA2_7B_FINETUNE_LOWBIT = Workload(
    name="llama2-7b-finetune-lowbit",
    shapes=(Shape("gate", 11008, 4096), Shape("down", 4096, 11008)),
    bits=(2, 3), gpr=8, lut_dtype="f16", lut_sigma=0.02, x_dtype="bf16",
    tokens=(8192,), backward=True, dy_sigma=1e-2,
    notes="forward, dX and dLUT at 2- and 3-bit indices (m = 8192)",
)

LLAMA2_7B_FINETUNE_GPR1 = Workload(
    name="llama2-7b-finetune-gpr1",
    shapes=(Shape("q", 4096, 4096), Shape("gate", 11008, 4096)),
    bits=(4,), gpr=1, lut_dtype="f16", lut_sigma=0.02, x_dtype="bf16",
    tokens=(8192,), backward=True, dy_sigma=1e-2,
    notes="dX and dLUT at one group per row (the 7B setting of the decode comparison): 32 and 86 row "
          "blocks, so the table gradient is split over column ranges of the group",
)

ALL: List[Workload] = [TINY, LLAMA2_7B_ATTN, LLAMA2_7B_MLP_LOWBIT, LLAMA3_70B_MLP, LLAMA2_7B_FINETUNE,
                       LLAMA2_13B_DECODE, LLAMA2_7B_FINETUNE_LOWBIT, LLAMA2_7B_FINETUNE_GPR1]
BY_NAME = {w.name: w for w in ALL}


def runs(w: Workload):
    """Every (shape, b, m) triple of a workload."""
    for s in w.shapes:
        for b in w.bits:
            for m in w.tokens:
                yield s, b, m


def algorithmic_bytes_fwd(n: int, d: int, b: int, gpr: int, m: int, lut_bytes: int, x_bytes: int) -> int:
    """Bytes a forward pass must move at least: indices + tables + X + Y."""
    return n * d * b // 8 + n * gpr * (1 << b) * lut_bytes + m * d * x_bytes + m * n * x_bytes


def flops_pass(n: int, d: int, m: int) -> int:
    """Multiply-add flops of one contraction pass (forward, dX or dY^T X)."""
    return 2 * m * n * d


DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
