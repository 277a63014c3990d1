"""GPU parity of sketch construction: column weights, weighted Lloyd tables, error-compensated mapping.

The kernels compute in fp32 and the oracle in float64, on the same fp32 inputs
(the factor U and the weights are rounded to fp32 before either side sees
them). Column weights and table values: |gpu - oracle| <= 1e-5 |oracle| +
1e-7 max|oracle| (fp32 tolerance). Indices are integers decided by fp32
comparisons: at the small sizes they must equal the oracle's; at full size a
decision may differ where two table entries are within rounding of equally
near, so sampled rows are checked along the GPU's own decisions (each chosen
entry is the nearest to the float64 compensated weight, within 1e-4 of the
table's scale) and at least 99.9 % of them must equal the oracle's. 16-bit
tables must be bit-exact the rounding of the same run's fp32 tables.
"""
import numpy as np
import pytest

import oracle
from lut_sketched_matmul_amd import synthetic as syn

from gpu_util import round_to, to_dev, to_f64

pytestmark = pytest.mark.gpu


def skm():
    import lut_sketched_matmul_amd as m
    return m


def torch():
    import torch as _t
    return _t


def close(got, ref, tol=1e-5, what=""):
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    bad = np.abs(got - ref) > tol * np.abs(ref) + 1e-7 * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} off, first {np.argwhere(bad)[:3].tolist()}"


def calib(tag, s, d):
    """Sample inputs with correlated columns: Z (I + 0.5 N / sqrt(d))."""
    Z = syn.random_normal(f"{tag}/Z", (s, d), 1.0, "f32").astype(np.float64)
    M = np.eye(d) + 0.5 * syn.random_normal(f"{tag}/M", (d, d), 1.0, "f32").astype(np.float64) / np.sqrt(d)
    return Z @ M


def factor32(tag, s, d):
    """The oracle's factor of the damped inverse Hessian, rounded to fp32 (the input both sides use)."""
    return oracle.hessian_factor(calib(tag, s, d), 0.01).astype(np.float32)


def weights(tag, n, d):
    return syn.random_normal(f"{tag}/W", (n, d), 0.02, "f32")


@pytest.mark.parametrize("d,s", [(1, 4), (5, 12), (63, 150), (64, 160), (65, 200), (200, 500), (1000, 2400)])
@pytest.mark.parametrize("damp", [0.01, 0.0])
def test_hessian_factor(d, s, damp):
    """U from the float64 Gram matrix (blocked Cholesky and triangular inverse in 64-column steps, padded to a
    multiple of 64) against the oracle's factor: float64 on both sides, so the fp32 result must equal the
    rounding of the oracle's within a few fp32 units of its scale; U is upper triangular with exact zeros below."""
    t = torch()
    X = calib(f"factor/{d}", s, d)
    H = to_dev(X.T @ X, "f64")
    U = to_f64(skm().sketch_hessian_factor(H, damp))
    want = oracle.hessian_factor(X, damp)
    assert np.all(np.tril(U, -1) == 0.0)
    assert float(np.max(np.abs(U - want))) <= 1e-6 * float(np.max(np.abs(want)))
    # and UᵀU inverts the damped H
    Hd = X.T @ X + damp * np.mean(np.diag(X.T @ X)) * np.eye(d)
    assert float(np.max(np.abs(U.T @ U @ Hd - np.eye(d)))) <= 1e-4
    # repeat calls are bit-identical (no atomics)
    assert np.array_equal(to_f64(skm().sketch_hessian_factor(H, damp)), U)
    del t


@pytest.mark.parametrize("d", [1, 37, 256, 1024])
def test_column_weights(d):
    U = factor32(f"cw/{d}", 2 * d + 8, d)
    h = to_f64(skm().sketch_column_weights(to_dev(U, "f32")))
    close(h, oracle.column_weights(U.astype(np.float64)), what="h")


@pytest.mark.parametrize("iters", [0, 1, 4, 60])
@pytest.mark.parametrize("b,gpr,n,d", [(4, 1, 9, 256), (3, 4, 17, 512), (2, 8, 5, 256), (4, 2, 33, 2048),
                                       (4, 8, 8, 4096)])
def test_lloyd(b, gpr, n, d, iters):
    tag = f"lloyd/{b}/{gpr}/{n}/{d}"
    W = weights(tag, n, d)
    h = np.exp(syn.random_normal(f"{tag}/h", (d,), 1.0, "f32")).astype(np.float32)
    got = to_f64(skm().sketch_lloyd(to_dev(W, "f32"), to_dev(h, "f32"), b, gpr, iters))
    want = oracle.weighted_lloyd(W.astype(np.float64), h.astype(np.float64), gpr, 1 << b, iters)
    close(got, want, what="tables")
    t = torch()
    for dt, name in ((t.float16, "f16"), (t.bfloat16, "bf16")):
        g16 = to_f64(skm().sketch_lloyd(to_dev(W, "f32"), to_dev(h, "f32"), b, gpr, iters, lut_dtype=dt))
        assert np.array_equal(g16, round_to(got, name)), name


def _map_case(tag, n, d, b, gpr, lut_dtype):
    U = factor32(tag, 2 * d, d)
    W = weights(tag, n, d)
    h = oracle.column_weights(U.astype(np.float64))
    lut = syn.to_storage(oracle.weighted_lloyd(W.astype(np.float64), h, gpr, 1 << b, 20), lut_dtype)
    return U, W, lut


@pytest.mark.parametrize("lut_dtype", ["f32", "f16"])
@pytest.mark.parametrize("b,gpr,n,d", [
    (4, 1, 7, 64), (4, 2, 33, 256), (3, 4, 20, 384), (2, 8, 65, 256),
    (4, 3, 9, 288),      # 96-column groups: a group boundary in the middle of a 64-column block
    (3, 7, 12, 224),     # 32-column groups, and a last block of 32 columns
    (4, 1, 70, 96),      # a last block of 32 columns
    (4, 2, 20, 1088),    # past one 512-column batch of errors: two batches and a 64-column rest
    (3, 3, 9, 1056),     # the same with a last block of 32 columns
])
def test_map_small(b, gpr, n, d, lut_dtype):
    U, W, lut = _map_case(f"map/{b}/{gpr}/{n}/{d}/{lut_dtype}", n, d, b, gpr, lut_dtype)
    work = to_dev(W, "f32")
    idx = skm().sketch_map(work, to_dev(U, "f32"), to_dev(lut, lut_dtype), b, gpr).cpu().numpy()
    got = oracle.unpack_indices(idx, d, b)
    want = oracle.map_error_compensated(W.astype(np.float64), U.astype(np.float64),
                                        syn.to_float64(lut, lut_dtype), gpr)
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} indices differ"


def _check_decisions(W, U, lut, idx, gpr):
    """Along the GPU's decisions (idx, for the rows of W and lut given): each chosen entry is the nearest
    to the float64 compensated weight; returns the largest excess distance."""
    w = W.astype(np.float64).copy()
    U = U.astype(np.float64)
    n, d = w.shape
    G = d // gpr
    r = np.arange(n)
    worst = 0.0
    for j in range(d):
        t = lut[:, j // G, :]
        a = idx[:, j]
        dist = np.abs(w[:, j:j + 1] - t)
        worst = max(worst, float(np.max(dist[r, a] - dist.min(axis=1))))
        err = (w[:, j] - t[r, a]) / U[j, j]
        w[:, j + 1:] -= err[:, None] * U[j, j + 1:][None, :]
    return worst


def test_construct_full_size():
    """A 4096 x 4096 layer, b = 4, 4 groups per row: sampled groups and rows against the oracle."""
    t = torch()
    n = d = 4096
    b, gpr, iters = 4, 4, 30
    Xs = calib("full", 2048, d)
    U = oracle.hessian_factor(Xs, 0.01).astype(np.float32)
    W = weights("full", n, d)
    from lut_sketched_matmul_amd import construct
    # the library's own factor (torch.linalg) agrees with the oracle's
    Ug = construct.hessian_factor(to_dev(Xs.astype(np.float32), "f32"))
    assert float(np.max(np.abs(to_f64(Ug) - U))) <= 1e-4 * float(np.max(np.abs(U)))
    gU, gW = to_dev(U, "f32"), to_dev(W, "f32")
    h = skm().sketch_column_weights(gU)
    lut32 = to_f64(skm().sketch_lloyd(gW, h, b, gpr, iters))
    lut = skm().sketch_lloyd(gW, h, b, gpr, iters, lut_dtype=t.float16)
    idx = skm().sketch_map(gW.clone(), gU, lut, b, gpr).cpu().numpy()
    lut64, h64 = to_f64(lut), to_f64(h)
    close(h64, oracle.column_weights(U.astype(np.float64)), what="h")
    assert np.array_equal(lut64, round_to(lut32, "f16"))
    rng = np.random.default_rng(5)
    groups = rng.choice(n * gpr, 96, replace=False)
    G = d // gpr
    for wg in groups:
        i, g = divmod(int(wg), gpr)
        c, _ = oracle.lloyd_group(W[i, g * G:(g + 1) * G].astype(np.float64), h64[g * G:(g + 1) * G], 16, iters)
        close(lut32[i, g], c, what=f"tables of row {i} group {g}")
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    got = oracle.unpack_indices(idx[rows], d, b)
    worst = _check_decisions(W[rows], U, lut64[rows], got, gpr)
    assert worst <= 1e-4 * float(np.max(np.abs(lut64))), worst
    want = oracle.map_error_compensated(W[rows].astype(np.float64), U.astype(np.float64), lut64[rows], gpr)
    assert np.mean(got == want) >= 0.999, float(np.mean(got == want))


def test_compensation_lowers_output_error():
    """The point of the mapping sweep: on the sample inputs, the layer output of the sketched weights is
    closer to the dense layer's than with plain nearest-entry rounding."""
    t = torch()
    from lut_sketched_matmul_amd import construct
    n, d, b, gpr = 256, 1024, 3, 4
    Xs = calib("gain", 1024, d).astype(np.float32)
    W = weights("gain", n, d)
    gX, gW = to_dev(Xs, "f32"), to_dev(W, "f32")
    idx, lut = construct.build_sketch(gW, b, gpr, Xs=gX, lut_dtype=t.float32)
    plain = skm().sketch_map(gW.clone(), t.eye(d, device="cuda:0"), lut, b, gpr)
    Wd = to_f64(skm().sketch_dequant(idx, lut, d, b, gpr))
    Wp = to_f64(skm().sketch_dequant(plain, lut, d, b, gpr))
    X64 = Xs.astype(np.float64)
    e_comp = np.linalg.norm(X64 @ (W - Wd).T)
    e_plain = np.linalg.norm(X64 @ (W - Wp).T)
    assert e_comp < 0.9 * e_plain, (e_comp, e_plain)
    assert np.array_equal(to_f64(gW), W.astype(np.float64))     # build_sketch leaves W alone
