"""Host <-> device plumbing for the GPU tests (no arithmetic of the method)."""
import numpy as np

from lut_sketched_matmul_amd import synthetic as syn


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray, dtype: str):
    """numpy storage array (bf16 as uint16 bits) -> torch tensor on cuda:0."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to("cuda:0")
    if dtype == "u8":
        return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda:0")
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def to_f64(x) -> np.ndarray:
    """torch tensor (any float dtype) -> exact float64 numpy array."""
    t = torch()
    return x.detach().to("cpu", t.float32).numpy().astype(np.float64)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return syn.to_float64(a, dtype)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to a storage dtype and back (nearest-even)."""
    return syn.to_float64(syn.to_storage(x.astype(np.float32) if dtype != "f32" else x, dtype), dtype)
