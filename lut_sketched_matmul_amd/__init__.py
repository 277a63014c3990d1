"""Sketched-weight (LUT + one-hot mapping) matrix multiply for AMD MI355X.

The compute lives in the HIP library ``libsketchmm.so`` (C ABI:
``include/sketch_matmul.h``); this package holds its ctypes binding, the
build script and the synthetic workload generators.
"""
from ._lib import (  # noqa: F401
    SKM_BF16,
    SKM_F16,
    SKM_F32,
    SketchError,
    header_functions,
    lib,
    sketch_column_weights,
    sketch_dequant,
    sketch_hessian_factor,
    sketch_lloyd,
    sketch_lut_adam_step,
    sketch_lut_sgd_step,
    sketch_map,
    sketch_matmul_bwd,
    sketch_matmul_bwd_noalloc,
    sketch_matmul_bwd_workspace,
    sketch_matmul_fwd,
    sketch_matmul_fwd_workspace,
    sketch_matmul_fwd_multi,
    sketch_unpack_indices,
)

__version__ = "0.1.0"
