"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: unpacked indices, dequantised W, selection inputs (one-hot rows of
X pick single weights), the identity example. Floating point: every output
tensor scored as max|gpu - oracle| / max|oracle| <= 5e-3 for 16-bit I/O with
fp32 accumulation and <= 1e-5 for the fp32 path.
"""
import numpy as np
import pytest

import oracle
from lut_sketched_matmul_amd import synthetic as syn
from lut_sketched_matmul_amd import workloads as wl

from gpu_util import round_to, to_dev, to_f64

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL32 = 1e-5


def skm():
    import lut_sketched_matmul_amd as m
    return m


def make_case(tag, n, d, b, gpr, m, x_dtype="f16", lut_dtype="f16", lut_sigma=0.02, dy_sigma=1.0):
    idx = syn.random_packed_indices(f"{tag}/idx", n, d, b)
    lut = syn.random_lut(f"{tag}/lut", n, gpr, b, lut_sigma, lut_dtype)
    X = syn.random_normal(f"{tag}/X", (m, d), 1.0, x_dtype)
    dY = syn.random_normal(f"{tag}/dY", (m, n), dy_sigma, x_dtype)
    return idx, lut, X, dY


# ---------------------------------------------------------------------------
# bit-exact checking aids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("n,d", [(5, 32), (37, 480), (64, 4096)])
def test_unpack_bit_exact(b, n, d):
    idx = syn.random_packed_indices(f"unpack/{b}/{n}/{d}", n, d, b)
    got = skm().sketch_unpack_indices(to_dev(idx, "u8"), d, b).cpu().numpy()
    assert np.array_equal(got.astype(np.int64), oracle.unpack_indices(idx, d, b))


@pytest.mark.parametrize("lut_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("b,gpr,n,d", [(2, 1, 16, 64), (3, 4, 33, 512), (4, 8, 40, 4096), (3, 8, 17, 11008)])
def test_dequant_bit_exact(lut_dtype, b, gpr, n, d):
    idx, lut, _, _ = make_case(f"deq/{lut_dtype}/{b}/{gpr}/{n}/{d}", n, d, b, gpr, 1, lut_dtype=lut_dtype)
    W = skm().sketch_dequant(to_dev(idx, "u8"), to_dev(lut, lut_dtype), d, b, gpr)
    want = oracle.dequantize(idx, syn.to_float64(lut, lut_dtype), d, b, gpr)
    assert np.array_equal(to_f64(W), want)


# ---------------------------------------------------------------------------
# fp32 path (tiny single layer, forward and backward)
# ---------------------------------------------------------------------------

def _check_fp32(idx, lut, X, dY, b, gpr, d):
    dev = dict(idx=to_dev(idx, "u8"), lut=to_dev(lut, "f32"), X=to_dev(X, "f32"), dY=to_dev(dY, "f32"))
    Y = skm().sketch_matmul_fwd(dev["X"], dev["idx"], dev["lut"], b, gpr)
    L64, X64, dY64 = lut.astype(np.float64), X.astype(np.float64), dY.astype(np.float64)
    assert oracle.rel_err(to_f64(Y), oracle.forward(X64, idx, L64, b, gpr)) <= TOL32
    dX, dL = skm().sketch_matmul_bwd(dev["dY"], dev["X"], dev["idx"], dev["lut"], b, gpr)
    assert oracle.rel_err(to_f64(dX), oracle.backward_dx(dY64, idx, L64, d, b, gpr)) <= TOL32
    assert oracle.rel_err(to_f64(dL), oracle.backward_dlut(dY64, X64, idx, b, gpr)) <= TOL32


def test_tiny_workload_fp32():
    w = wl.TINY
    s = w.shapes[0]
    t = w.make(s, 4, 4)
    _check_fp32(t["idx_packed"], t["lut"], t["X"], t["dY"], 4, w.gpr, s.d)


@pytest.mark.parametrize("b,gpr,n,d,m", [(2, 2, 19, 256, 3), (3, 1, 50, 96, 9), (4, 4, 7, 512, 1)])
def test_fp32_ragged(b, gpr, n, d, m):
    idx, lut, X, dY = make_case(f"f32r/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m, "f32", "f32")
    _check_fp32(idx, lut, X, dY, b, gpr, d)


# ---------------------------------------------------------------------------
# 16-bit forward
# ---------------------------------------------------------------------------

def _fwd16(idx, lut, X, b, gpr, x_dtype, lut_dtype, rows=None):
    Y = skm().sketch_matmul_fwd(to_dev(X, x_dtype), to_dev(idx, "u8"), to_dev(lut, lut_dtype), b, gpr)
    got = to_f64(Y)
    X64 = syn.to_float64(X, x_dtype)
    L64 = syn.to_float64(lut, lut_dtype)
    if rows is None:
        return got, oracle.forward(X64, idx, L64, b, gpr)
    return got[:, rows], oracle.forward(X64, idx[rows], L64[rows], b, gpr)


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 8, 4096, 4096, 1), (4, 1, 100, 160, 3), (2, 2, 257, 1024, 16), (3, 4, 77, 1536, 5),
    (2, 8, 300, 11008, 4), (3, 8, 48, 11008, 16), (4, 4, 64, 8192, 2), (4, 32, 70, 2048, 3),
    # decode rows of 48 and 80 128-column slots (several slot batches per
    # wave, the last one partial), and rows of one and of two slots
    (4, 4, 40, 6144, 2), (2, 2, 33, 10240, 1), (3, 2, 40, 10240, 16), (4, 1, 21, 128, 3), (2, 1, 18, 256, 5),
    # just over the activation staging limit (m * d > 32768: activations read
    # per slot), and a ragged row
    (4, 8, 40, 4096, 16), (2, 8, 50, 3072, 16), (3, 2, 17, 4096, 12), (4, 8, 70, 4096, 9), (4, 1, 24, 2080, 16),
])
def test_fwd16_small(x_dtype, lut_dtype, b, gpr, n, d, m):
    idx, lut, X, _ = make_case(f"fwd16/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m,
                               x_dtype, lut_dtype)
    got, want = _fwd16(idx, lut, X, b, gpr, x_dtype, lut_dtype)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 1, 8200, 1184, 3), (4, 4, 8200, 1152, 2), (3, 8, 9001, 2048, 1), (2, 8, 12000, 512, 16),
    (4, 1, 16400, 96, 7), (4, 8, 8400, 4096, 1),
])
def test_fwd16_large_n_decode(x_dtype, lut_dtype, b, gpr, n, d, m):
    """Decode with more 16-row blocks than the GPU holds at once (8-wave
    blocks); ragged rows and ragged 128-column slots included. Every row is
    checked."""
    idx, lut, X, _ = make_case(f"stream/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m,
                               x_dtype, lut_dtype)
    got, want = _fwd16(idx, lut, X, b, gpr, x_dtype, lut_dtype)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_large_n_decode_selection_bit_exact(dt):
    """One-hot activation rows through the decode at large n: exact weights."""
    b, gpr, n, d, m = 4, 4, 9000, 1024, 5
    idx, lut, _, _ = make_case(f"ssel/{dt}", n, d, b, gpr, 1, dt, dt)
    cols = np.random.default_rng(5).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    Y = skm().sketch_matmul_fwd(to_dev(syn.to_storage(X, dt), dt), to_dev(idx, "u8"), to_dev(lut, dt), b, gpr)
    W = oracle.dequantize(idx, syn.to_float64(lut, dt), d, b, gpr)
    assert np.array_equal(to_f64(Y), W[:, cols].T)


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 8, 200, 4096, 300), (4, 1, 64, 512, 17), (2, 8, 130, 11008, 40), (3, 4, 257, 1536, 513),
    (2, 2, 96, 1024, 256), (3, 8, 128, 11008, 33), (4, 4, 300, 8192, 260), (4, 1, 70, 64, 40),
    (3, 1, 33, 128, 19), (2, 2, 300, 128, 300), (4, 8, 150, 11008, 40), (4, 1, 96, 96, 33),
])
def test_fwd16_gemm(x_dtype, lut_dtype, b, gpr, n, d, m):
    """m > 16 runs the tiled matrix-core GEMM: ragged token and row tiles; one-
    and two-step K loops; 32- and 64-column K-steps (odd / even units per
    group), for every bit width (b = 4 with 43 and 3 units per group takes the
    32-column steps)."""
    idx, lut, X, _ = make_case(f"gemm16/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m,
                               x_dtype, lut_dtype)
    got, want = _fwd16(idx, lut, X, b, gpr, x_dtype, lut_dtype)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_gemm_selection_bit_exact(dt):
    """m > 16 one-hot rows through the GEMM: Y[t, i] = W[i, j_t] exactly."""
    b, gpr, n, d, m = 4, 8, 150, 4096, 70
    idx, lut, _, _ = make_case(f"gsel/{dt}", n, d, b, gpr, 1, dt, dt)
    cols = np.random.default_rng(7).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    Y = skm().sketch_matmul_fwd(to_dev(syn.to_storage(X, dt), dt), to_dev(idx, "u8"), to_dev(lut, dt), b, gpr)
    W = oracle.dequantize(idx, syn.to_float64(lut, dt), d, b, gpr)
    assert np.array_equal(to_f64(Y), W[:, cols].T)


def _workload_rows(n, seed):
    r = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(0, 32), np.arange(n - 32, n), r.choice(n, 448, replace=False)])
    return np.unique(rows)


@pytest.mark.parametrize("wname", [wl.LLAMA2_7B_ATTN.name, wl.LLAMA2_7B_MLP_LOWBIT.name, wl.LLAMA3_70B_MLP.name,
                                   wl.LLAMA2_13B_DECODE.name])
def test_fwd_workloads(wname):
    """Every (shape, b, m) of the forward workloads at full size; sampled rows."""
    w = wl.BY_NAME[wname]
    worst = 0.0
    for s, b, m in wl.runs(w):
        t = w.make(s, b, m)
        rows = _workload_rows(s.n, s.n + m + b)
        got, want = _fwd16(t["idx_packed"], t["lut"], t["X"], b, w.gpr, w.x_dtype, w.lut_dtype, rows)
        e = oracle.rel_err(got, want)
        worst = max(worst, e)
        assert e <= w.tol, (s.name, b, m, e)
    print(f"{wname}: worst rel err {worst:.3e}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [1, 7, 16])
def test_fwd_selection_bit_exact(dt, m):
    """X rows are one-hot: Y[t, i] = W[i, j_t] exactly (one non-zero product)."""
    b, gpr, n, d = 4, 8, 80, 4096
    idx, lut, _, _ = make_case(f"sel/{dt}/{m}", n, d, b, gpr, 1, dt, dt)
    cols = np.random.default_rng(m).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    Xs = syn.to_storage(X, dt)
    Y = skm().sketch_matmul_fwd(to_dev(Xs, dt), to_dev(idx, "u8"), to_dev(lut, dt), b, gpr)
    W = oracle.dequantize(idx, syn.to_float64(lut, dt), d, b, gpr)
    assert np.array_equal(to_f64(Y), W[:, cols].T)


# ---------------------------------------------------------------------------
# several table sets over one mapping, one set per token (SpaLLM section 2.3)
# ---------------------------------------------------------------------------

def _multi_case(tag, n, d, b, gpr, m, n_sets, x_dtype, lut_dtype):
    idx, _, X, _ = make_case(tag, n, d, b, gpr, m, x_dtype, lut_dtype)
    luts = np.stack([syn.random_lut(f"{tag}/lut{s}", n, gpr, b, 0.02, lut_dtype) for s in range(n_sets)])
    return idx, luts, X


def _fwd_multi(idx, luts, X, sets, b, gpr, x_dtype, lut_dtype):
    return skm().sketch_matmul_fwd_multi(to_dev(X, x_dtype), to_dev(idx, "u8"), to_dev(luts, lut_dtype),
                                         to_dev(np.asarray(sets, dtype=np.int32), "i32"), b, gpr)


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("b,gpr,n,d,sets,n_sets", [
    (4, 8, 64, 4096, [0, 1, 2, 3], 4),
    (4, 8, 70, 4096, [2, 0, 1, 1, 0, 2, 2, 2, 0, 1, 0, 2, 1, 1, 0, 0], 3),
    (2, 8, 40, 11008, [1, 1, 0], 2),       # 11008 columns: ragged 128-column slots
    (3, 4, 33, 1536, [4, 3, 2, 1, 0], 5),
    (4, 1, 20, 512, [1], 2),               # one token, using set 1 only
    (4, 4, 8200, 1152, [0, 1], 2),         # more blocks than the GPU holds at once
    # more tokens of one set than one pass stages (32768 // d of them): the set
    # takes several passes
    (4, 8, 64, 4096, [0] * 12 + [1] * 4, 2),
    (2, 8, 40, 11008, [0, 0, 0, 1, 0], 2),
    (4, 4, 33, 16384, [1, 0, 1, 1, 0, 0, 1], 2),
    (4, 8, 16, 32768, [0, 0, 1], 2),       # one token per pass
    (4, 8, 32, 36864, [1, 0, 1], 2),       # no activation staging (one row exceeds it)
    (3, 4, 24, 4096, [0] * 16, 1),         # one set: all 16 rows read from memory, one pass
])
def test_fwd_multi(x_dtype, lut_dtype, b, gpr, n, d, sets, n_sets):
    idx, luts, X = _multi_case(f"multi/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{n_sets}", n, d, b, gpr, len(sets),
                               n_sets, x_dtype, lut_dtype)
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, x_dtype, lut_dtype))
    want = oracle.forward_multi(syn.to_float64(X, x_dtype), idx, syn.to_float64(luts, lut_dtype), sets, b, gpr)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("seed", range(12))
def test_fwd_multi_random_patterns(seed):
    """Seeded random batches: token count, set count, set indices (some out of range, clamped), bit width,
    groups and column count (staging capacities of 32768 / d = 32, 8, 2 or 1 tokens per pass)."""
    r = np.random.default_rng(1000 + seed)
    b = int(r.choice([2, 3, 4]))
    d, gpr = [(1024, 4), (4096, 8), (11008, 8), (16384, 4), (32768, 8)][seed % 5]
    m = int(r.integers(1, 17))
    n_sets = int(r.integers(1, 7))
    sets = r.integers(-1, n_sets + 1, m).tolist()
    clamped = [min(max(v, 0), n_sets - 1) for v in sets]
    n = 24
    xdt, ldt = [("f16", "f16"), ("bf16", "f16"), ("bf16", "bf16")][seed % 3]
    idx, luts, X = _multi_case(f"multirand/{seed}", n, d, b, gpr, m, n_sets, xdt, ldt)
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, xdt, ldt))
    want = oracle.forward_multi(syn.to_float64(X, xdt), idx, syn.to_float64(luts, ldt), clamped, b, gpr)
    assert oracle.rel_err(got, want) <= TOL16, (b, d, gpr, m, n_sets, sets)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [5, 16])
def test_fwd_multi_one_set_is_fwd(dt, m):
    """All tokens on one set: the same numbers as the single-set forward (m = 16: the set takes two
    passes of 8 staged tokens, the single-set kernel reads all 16 from memory)."""
    b, gpr, n, d = 4, 8, 80, 4096
    idx, luts, X = _multi_case(f"multi1/{dt}/{m}", n, d, b, gpr, m, 3, dt, dt)
    got = _fwd_multi(idx, luts, X, [1] * m, b, gpr, dt, dt)
    ref = skm().sketch_matmul_fwd(to_dev(X, dt), to_dev(idx, "u8"), to_dev(luts[1], dt), b, gpr)
    assert bool((got == ref).all())


def test_fwd_multi_clamps_set_indices():
    b, gpr, n, d = 4, 4, 48, 1024
    sets, clamped = [-3, 0, 7, 1], [0, 0, 1, 1]
    idx, luts, X = _multi_case("multiclamp", n, d, b, gpr, len(sets), 2, "f16", "f16")
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, "f16", "f16"))
    want = oracle.forward_multi(syn.to_float64(X, "f16"), idx, syn.to_float64(luts, "f16"), clamped, b, gpr)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("b", [2, 3, 4])
def test_fwd_multi_selection_bit_exact(b):
    """One-hot activation rows: token t reads W_{s(t)}[i, j_t] exactly."""
    gpr, n, d, m, n_sets = 4, 96, 2048, 6, 3
    idx, luts, _ = _multi_case(f"multisel/{b}", n, d, b, gpr, 1, n_sets, "f16", "f16")
    cols = np.random.default_rng(b).choice(d, m, replace=False)
    sets = [2, 0, 1, 1, 2, 0]
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    got = to_f64(_fwd_multi(idx, luts, syn.to_storage(X, "f16"), sets, b, gpr, "f16", "f16"))
    L = syn.to_float64(luts, "f16")
    for t in range(m):
        W = oracle.dequantize(idx, L[sets[t]], d, b, gpr)
        assert np.array_equal(got[t], W[:, cols[t]]), t


@pytest.mark.parametrize("b", [2, 3, 4])
def test_fwd_identity_exact(b):
    """SpaLLM section 2.4: the identity sketched with the two values 0 and 1."""
    n, gpr, m = 256, 4, 5
    k = 1 << b
    lut = np.full((n, gpr, k), 0.5, dtype=np.float32)
    lut[:, :, 0] = 0.0
    lut[:, :, 1] = 1.0
    idx = oracle.pack_indices(np.eye(n, dtype=np.int64), b)
    X = syn.random_normal(f"ident/{b}", (m, n), 1.0, "f16")
    Y = skm().sketch_matmul_fwd(to_dev(X, "f16"), to_dev(idx, "u8"), to_dev(syn.to_storage(lut, "f16"), "f16"), b, gpr)
    assert np.array_equal(to_f64(Y), syn.to_float64(X, "f16"))


def test_fwd_deterministic():
    idx, lut, X, _ = make_case("det", 1000, 4096, 4, 8, 4)
    a = skm().sketch_matmul_fwd(to_dev(X, "f16"), to_dev(idx, "u8"), to_dev(lut, "f16"), 4, 8)
    b_ = skm().sketch_matmul_fwd(to_dev(X, "f16"), to_dev(idx, "u8"), to_dev(lut, "f16"), 4, 8)
    assert bool((a == b_).all())


# ---------------------------------------------------------------------------
# 16-bit backward (dX and dLUT on the matrix cores)
# ---------------------------------------------------------------------------

def _bwd16(idx, lut, X, dY, b, gpr, d, io, lut_dtype, accumulate=False, dlut_init=None):
    dl = None
    if dlut_init is not None:
        dl = to_dev(dlut_init.astype(np.float32), "f32")
    dX, dL = skm().sketch_matmul_bwd(to_dev(dY, io), to_dev(X, io), to_dev(idx, "u8"), to_dev(lut, lut_dtype), b,
                                     gpr, d=d, dlut_out=dl, accumulate=accumulate)
    return to_f64(dX), to_f64(dL)


@pytest.mark.parametrize("io,lut_dtype", [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 8, 200, 4096, 300), (2, 2, 130, 1024, 40), (3, 8, 96, 11008, 33), (4, 1, 257, 512, 17),
    (3, 4, 300, 1536, 260), (2, 32, 64, 1024, 64), (4, 4, 33, 8192, 5), (4, 1, 64, 256, 100),
    (2, 2, 129, 512, 70), (4, 8, 70, 11008, 40), (4, 8, 256, 11008, 64),
    # whole 32-token steps and rows a multiple of 8 (tiles copied into LDS by
    # DMA): one, two and several steps, partial row blocks, groups of 3 and 4
    # column chunks, columns clamped at the row end
    (2, 2, 64, 1024, 32), (4, 1, 128, 512, 64), (4, 8, 200, 4096, 96), (3, 4, 136, 1536, 64),
    (3, 8, 72, 11008, 96), (4, 4, 40, 8192, 160),
])
def test_bwd16(io, lut_dtype, b, gpr, n, d, m):
    idx, lut, X, dY = make_case(f"bwd16/{io}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m, io, lut_dtype)
    gdx, gdl = _bwd16(idx, lut, X, dY, b, gpr, d, io, lut_dtype)
    L64, X64, dY64 = syn.to_float64(lut, lut_dtype), syn.to_float64(X, io), syn.to_float64(dY, io)
    assert oracle.rel_err(gdx, oracle.backward_dx(dY64, idx, L64, d, b, gpr)) <= TOL16
    assert oracle.rel_err(gdl, oracle.backward_dlut(dY64, X64, idx, b, gpr)) <= TOL16


@pytest.mark.parametrize("b", [2, 3, 4])
def test_dlut_bins_exact(b):
    """Integer dY and one-hot X rows: every bin sum is an exact small integer."""
    n, gpr, d, m = 130, 4, 2048, 96
    idx, lut, _, _ = make_case(f"bins/{b}", n, d, b, gpr, 1, "bf16", "bf16")
    cols = np.random.default_rng(b).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    dY = syn.random_int_valued(f"bins/{b}/dY", (m, n), -3, 3, "bf16")
    Xs = syn.to_storage(X, "bf16")
    _, gdl = _bwd16(idx, lut, Xs, dY, b, gpr, d, "bf16", "bf16")
    want = oracle.backward_dlut(syn.to_float64(dY, "bf16"), X.astype(np.float64), idx, b, gpr)
    assert np.array_equal(gdl, want)


@pytest.mark.parametrize("m", [80, 96])
def test_bwd_accumulate_and_deterministic(m):
    b, gpr, n, d = 4, 8, 160, 4096
    idx, lut, X, dY = make_case(f"bwdacc/{m}", n, d, b, gpr, m, "bf16", "f16")
    a1 = _bwd16(idx, lut, X, dY, b, gpr, d, "bf16", "f16")
    a2 = _bwd16(idx, lut, X, dY, b, gpr, d, "bf16", "f16")
    assert np.array_equal(a1[0], a2[0]) and np.array_equal(a1[1], a2[1])
    base = np.random.default_rng(3).normal(size=(n, gpr, 16)).astype(np.float32)
    _, acc = _bwd16(idx, lut, X, dY, b, gpr, d, "bf16", "f16", accumulate=True, dlut_init=base)
    assert np.allclose(acc, base.astype(np.float64) + a1[1], rtol=0, atol=1e-6 * max(1.0, np.abs(a1[1]).max()))


@pytest.mark.parametrize("wname,b", [(wl.LLAMA2_7B_FINETUNE.name, 4), (wl.LLAMA2_7B_FINETUNE_LOWBIT.name, 2),
                                     (wl.LLAMA2_7B_FINETUNE_LOWBIT.name, 3)])
def test_finetune_workload_sampled(wname, b):
    """The 7B decoder layer's projections at full size (m = 8192): sampled outputs."""
    w = wl.BY_NAME[wname]
    r = np.random.default_rng(11 + b)
    shapes = (w.shapes[0], w.shapes[4], w.shapes[6]) if b == 4 else w.shapes   # q, gate, down
    for s in shapes:
        t = w.make(s, b, 8192)
        X64 = syn.to_float64(t["X"], w.x_dtype)
        dY64 = syn.to_float64(t["dY"], w.x_dtype)
        L64 = syn.to_float64(t["lut"], w.lut_dtype)
        gi, gl = to_dev(t["idx_packed"], "u8"), to_dev(t["lut"], w.lut_dtype)
        gx, gdy = to_dev(t["X"], w.x_dtype), to_dev(t["dY"], w.x_dtype)
        Y = to_f64(skm().sketch_matmul_fwd(gx, gi, gl, b, w.gpr))
        dX, dL = skm().sketch_matmul_bwd(gdy, gx, gi, gl, b, w.gpr)
        dX, dL = to_f64(dX), to_f64(dL)
        rows = np.unique(np.concatenate([[0, s.n - 1], r.choice(s.n, 256, replace=False)]))
        cols = np.unique(np.concatenate([[0, s.d - 1], r.choice(s.d, 256, replace=False)]))
        toks = np.unique(np.concatenate([[0, 8191], r.choice(8192, 512, replace=False)]))
        want_y = oracle.forward(X64[toks], t["idx_packed"][rows], L64[rows], b, w.gpr)
        assert oracle.rel_err(Y[np.ix_(toks, rows)], want_y) <= w.tol, s.name
        W = oracle.dequantize(t["idx_packed"], L64, s.d, b, w.gpr)
        assert oracle.rel_err(dX[np.ix_(toks, cols)], dY64[toks] @ W[:, cols]) <= w.tol, s.name
        want_dl = oracle.backward_dlut(dY64[:, rows], X64, t["idx_packed"][rows], b, w.gpr)
        assert oracle.rel_err(dL[rows], want_dl) <= w.tol, s.name
