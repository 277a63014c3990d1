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
    # up to 49152 activation elements staged when m < 8 and the grid is at most one block per CU (a ragged
    # row among them), and just past that
    (4, 1, 40, 8224, 5), (2, 8, 64, 11008, 4), (2, 8, 64, 11008, 5),
    # the LDS turn-around from its first token count on, with a ragged row
    (4, 1, 40, 4128, 8),
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
    # activations past the staging limit: from 8 tokens on turned around in LDS (one with a ragged
    # slot), below that loaded per lane
    (2, 8, 8200, 4096, 12), (4, 5, 8300, 2080, 16), (4, 4, 6400, 4736, 7),
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


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("gpr,d", [(8, 4096), (8, 11008)])
def test_gemm_selection_bit_exact(x_dtype, lut_dtype, b, gpr, d):
    """m > 16 one-hot rows through the GEMM: Y[t, i] = W[i, j_t] exactly. Groups of 16 units take the
    64-column K-steps, groups of 43 units (11008 / 8 columns) the 32-column K-steps."""
    n, m = 150, 70
    idx, lut, _, _ = make_case(f"gsel/{x_dtype}/{lut_dtype}/{b}/{d}", n, d, b, gpr, 1, x_dtype, lut_dtype)
    cols = np.random.default_rng(7 + b).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    Y = skm().sketch_matmul_fwd(to_dev(syn.to_storage(X, x_dtype), x_dtype), to_dev(idx, "u8"),
                                to_dev(lut, lut_dtype), b, gpr)
    W = oracle.dequantize(idx, syn.to_float64(lut, lut_dtype), d, b, gpr)
    want = round_to(W[:, cols].T, x_dtype)  # Y is stored in X's dtype
    assert np.array_equal(to_f64(Y), want)


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
    (4, 8, 32, 36864, [1], 2),             # the same with one token
    (3, 4, 24, 4096, [0] * 16, 1),         # one set: all 16 rows read from memory, one pass
])
def test_fwd_multi(x_dtype, lut_dtype, b, gpr, n, d, sets, n_sets):
    idx, luts, X = _multi_case(f"multi/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{n_sets}", n, d, b, gpr, len(sets),
                               n_sets, x_dtype, lut_dtype)
    if (x_dtype, lut_dtype) == ("bf16", "f16") and d > 32768 and len(sets) == 1:
        # one prescaled token takes the kernel that stages its row in LDS, which
        # holds at most 32768 columns (from two tokens on, the set-interleaved
        # kernel finds the row exponents without staging)
        with pytest.raises(skm().SketchError) as e:
            _fwd_multi(idx, luts, X, sets, b, gpr, x_dtype, lut_dtype)
        assert e.value.status == -2
        return
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


@pytest.mark.parametrize("seed", range(24))
def test_fwd_multi_set_cells_random(seed):
    """Seeded random batches for the set-interleaved lookups: 2-16 tokens over up to 20 sets (so 2-, 4- and
    8-set lookups and two cells per entry), random and out-of-range set indices, every dtype pair, row counts
    off the 16-row blocks and column counts off the 128-column slots."""
    r = np.random.default_rng(5000 + seed)
    b = int(r.choice([2, 3, 4]))
    d, gpr = [(1024, 4), (1376, 1), (2752, 2), (2048, 8), (4096, 8), (1536, 4)][seed % 6]
    if (gpr << b) > 128:
        gpr = max(1, 128 >> b)
        d = gpr * 32 * int(d // (gpr * 32))
    m = int(r.integers(2, 17))
    n_sets = int(r.integers(1, 21))
    sets = r.integers(-2, n_sets + 2, m).tolist()
    clamped = [min(max(v, 0), n_sets - 1) for v in sets]
    n = int(r.integers(17, 120))
    xdt, ldt = [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")][seed % 4]
    idx, luts, X = _multi_case(f"cellrand/{seed}", n, d, b, gpr, m, n_sets, xdt, ldt)
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, xdt, ldt))
    want = oracle.forward_multi(syn.to_float64(X, xdt), idx, syn.to_float64(luts, ldt), clamped, b, gpr)
    assert oracle.rel_err(got, want) <= TOL16, (b, d, gpr, m, n_sets, sets)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [5, 16])
def test_fwd_multi_one_set_is_fwd(dt, m):
    """All tokens on one set: the single-set forward's numbers up to the rounding of the outputs. The
    multi-set kernel with set-interleaved tables adds each token's products in MFMAs of 16 columns (its
    contraction runs over column and set-parity pairs), the single-set decode in MFMAs of 32, so the fp32
    sums round differently before the 16-bit output; both stay within the parity bound of the oracle."""
    b, gpr, n, d = 4, 8, 80, 4096
    idx, luts, X = _multi_case(f"multi1/{dt}/{m}", n, d, b, gpr, m, 3, dt, dt)
    got = to_f64(_fwd_multi(idx, luts, X, [1] * m, b, gpr, dt, dt))
    ref = to_f64(skm().sketch_matmul_fwd(to_dev(X, dt), to_dev(idx, "u8"), to_dev(luts[1], dt), b, gpr))
    want = oracle.forward(syn.to_float64(X, dt), idx, syn.to_float64(luts[1], dt), b, gpr)
    assert oracle.rel_err(got, want) <= TOL16 and oracle.rel_err(ref, want) <= TOL16
    # no output differs by more than one unit in the last place of the largest output
    assert oracle.rel_err(got, ref) <= 2.0 ** (-10 if dt == "f16" else -7), dt


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("bf16", "f16"), ("f16", "bf16"), ("bf16", "bf16")])
@pytest.mark.parametrize("setv,want_set", [(2, 2), (-1, 0), (7, 2)])
def test_fwd_multi_one_token_is_fwd(x_dtype, lut_dtype, setv, want_set):
    """One token uses one set: the multi-set call runs the single-set decode on the set it reads from lut_set
    on the device (clamped), so its output equals the single-set forward on that set bit for bit."""
    b, gpr, n, d = 4, 8, 80, 4096
    idx, luts, X = _multi_case(f"multi1tok/{x_dtype}/{lut_dtype}", n, d, b, gpr, 1, 3, x_dtype, lut_dtype)
    got = _fwd_multi(idx, luts, X, [setv], b, gpr, x_dtype, lut_dtype)
    ref = skm().sketch_matmul_fwd(to_dev(X, x_dtype), to_dev(idx, "u8"), to_dev(luts[want_set], lut_dtype), b, gpr)
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


@pytest.mark.parametrize("x_dtype,lut_dtype", [("f16", "f16"), ("f16", "bf16"), ("bf16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("b,gpr,n,d,sets,n_sets", [
    # eight sets in use: one 128-bit lookup per weight serves them all
    (4, 8, 48, 4096, [0, 1, 2, 3, 4, 5, 6, 7], 8),
    (2, 2, 40, 2752, [7, 6, 5, 4, 3, 2, 1, 0, 7, 6], 8),        # ragged 128-column slots
    (3, 4, 33, 1536, [3, 1, 4, 1, 5, 0, 2, 6, 5, 3, 5], 7),
    # more than eight sets: a second cell per (entry, row)
    (4, 8, 64, 4096, list(range(16)), 16),
    (4, 8, 70, 4096, [15 - t for t in range(16)], 16),
    (2, 2, 40, 2752, [(5 * t) % 13 for t in range(13)], 13),    # ragged slots
    (4, 1, 24, 1376, [(7 * t) % 16 for t in range(16)], 16),    # ragged slots, one group
    (3, 4, 37, 1536, [(3 * t + 1) % 11 for t in range(12)], 11),
    (4, 2, 16, 1024, [t % 9 for t in range(16)], 9),
    # capacity above the sets in use (the pairs past them are not kept)
    (4, 8, 32, 4096, [2, 2, 9, 9, 2, 9, 2, 2, 9, 9, 2, 9, 2, 9, 9, 2], 12),
    (4, 8, 32, 4096, [1, 1, 1, 1, 1, 0, 0, 0], 8),
    (2, 4, 24, 2048, [5, 3, 5, 3, 5, 3, 5, 3, 5, 3], 10),
    # entry limits: 224 per row with at most 8 sets, 128 with more; beyond
    # that, one round of lookups per set
    (4, 14, 32, 14336, [0, 1, 2, 3, 4, 5], 6),
    (3, 16, 32, 4096, list(range(12)), 12),
    (4, 14, 32, 14336, list(range(10)), 10),
    # out-of-range set indices (clamped) with two cells
    (4, 8, 40, 4096, [-5, 0, 20, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 17], 16),
    # more than 384 row blocks: 8-wave blocks, two per CU
    (4, 4, 6160, 512, [3, 1, 2, 0, 3, 1], 4),
    (2, 1, 6176, 1024, [(5 * t + 2) % 16 for t in range(16)], 16),
    (3, 2, 6150, 512, [4, 0, 1, 2, 3, 4, 0, 1, 2, 3], 5),
])
def test_fwd_multi_set_cells(x_dtype, lut_dtype, b, gpr, n, d, sets, n_sets):
    """Set-interleaved tables (SpaLLM section 2.3, several adapters over one mapping): up to eight sets per
    lookup and sixteen with two cells per (entry, row), activations turned around in LDS in one, two or four
    groups of token rows; the oracle takes the clamped set indices."""
    clamped = [min(max(v, 0), n_sets - 1) for v in sets]
    idx, luts, X = _multi_case(f"multicell/{x_dtype}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{n_sets}/{len(sets)}", n, d, b,
                               gpr, len(sets), n_sets, x_dtype, lut_dtype)
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, x_dtype, lut_dtype))
    want = oracle.forward_multi(syn.to_float64(X, x_dtype), idx, syn.to_float64(luts, lut_dtype), clamped, b, gpr)
    assert oracle.rel_err(got, want) <= TOL16


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("m,n_sets", [(8, 8), (16, 16), (12, 16)])
def test_fwd_multi_set_cells_selection_exact(b, m, n_sets):
    """One-hot activation rows through the set-interleaved lookups (one cell, two cells): token t reads
    W_{s(t)}[i, j_t] exactly, for every set slot and parity."""
    gpr, n, d = 4, 40, 2048
    idx, luts, _ = _multi_case(f"multicellsel/{b}/{m}/{n_sets}", n, d, b, gpr, 1, n_sets, "f16", "f16")
    cols = np.random.default_rng(10 * b + m).choice(d, m, replace=False)
    sets = [(5 * t + 3) % n_sets for t in range(m)]
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


@pytest.mark.parametrize("b", [2, 3, 4])
def test_dlut_bins_exact_dma(b):
    """As above with whole 32-token steps and rows a multiple of 8, which take the kernel that copies its
    operand tiles into LDS (swizzled chunks): exact integer bin sums."""
    n, gpr, d, m = 128, 4, 2048, 96
    idx, lut, _, _ = make_case(f"binsdma/{b}", n, d, b, gpr, 1, "bf16", "bf16")
    cols = np.random.default_rng(20 + b).choice(d, m, replace=False)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    dY = syn.random_int_valued(f"binsdma/{b}/dY", (m, n), -3, 3, "bf16")
    _, gdl = _bwd16(idx, lut, syn.to_storage(X, "bf16"), dY, b, gpr, d, "bf16", "bf16")
    want = oracle.backward_dlut(syn.to_float64(dY, "bf16"), X.astype(np.float64), idx, b, gpr)
    assert np.array_equal(gdl, want)


@pytest.mark.parametrize("io,lut_dtype", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("gpr,d", [(8, 4096), (32, 4096)])
def test_dx_selection_bit_exact(io, lut_dtype, b, gpr, d):
    """One-hot dY rows: dX[t, :] = W[i_t, :] exactly (one non-zero product per output). Groups of 512
    columns take the 64-row dX steps, groups of 128 columns the 32-row steps."""
    n, m = 200, 40
    idx, lut, X, _ = make_case(f"dxsel/{io}/{lut_dtype}/{b}/{gpr}", n, d, b, gpr, m, io, lut_dtype)
    rows = np.random.default_rng(30 + b).choice(n, m, replace=False)
    dY = np.zeros((m, n), dtype=np.float32)
    dY[np.arange(m), rows] = 1.0
    gdx, _ = _bwd16(idx, lut, X, syn.to_storage(dY, io), b, gpr, d, io, lut_dtype)
    W = oracle.dequantize(idx, syn.to_float64(lut, lut_dtype), d, b, gpr)
    assert np.array_equal(gdx, W[rows])


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
    """The 7B decoder layer at full size (m = 8192), forward + dX + dLUT on sampled outputs: the q, gate
    and down projections at b = 4 (k, v and o have q's shape and up has gate's, so they run the same kernel
    instances on the same grids) and gate and down at b = 2 and 3."""
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


# ---------------------------------------------------------------------------
# bf16 activations with f16 tables: the matrix cores take f16 operands, so the
# activations (forward) and output gradients (dX) are prescaled per token row
# by a power of two before the conversion. These inputs lie outside f16's
# range (entries above 65504, rows of gradients far below 2^-14).
# ---------------------------------------------------------------------------

def _scaled_rows(tag, shape, scales):
    """bf16 N(0, 1) rows, row t multiplied by scales[t % len(scales)] (bits)."""
    z = syn.random_normal(tag, shape, 1.0, "f32").astype(np.float64)
    s = np.asarray([scales[t % len(scales)] for t in range(shape[0])], dtype=np.float64)[:, None]
    return syn.to_storage((z * s).astype(np.float32), "bf16")


def _row_errs(got, want):
    return [oracle.rel_err(got[t], want[t]) for t in range(want.shape[0])]


@pytest.mark.parametrize("b,gpr,d", [(4, 8, 4096), (4, 32, 4096), (2, 8, 4096), (3, 4, 1536)])
@pytest.mark.parametrize("sigma", [1e-6, 1e-8, 1e-20, 1e-33, 1e4])
def test_dx_gradient_scales_bf16_f16(b, gpr, d, sigma):
    """dY ~ N(0, sigma) in bf16: dX within the 16-bit tolerance at gradient scales far below f16's normal
    range (and up to f16's largest value). The scales take each conversion of a block: none (1e4),
    exponent-field add (1e-6 .. 1e-20), multiply (1e-33, rows below 2^-87). Groups of 512 and 384 columns take the 64-row dX steps, groups of
    128 columns the 32-row steps."""
    n, m = 256, 96
    idx, lut, X, _ = make_case(f"dxscale/{b}/{gpr}/{d}", n, d, b, gpr, m, "bf16", "f16")
    dY = syn.random_normal(f"dxscale/{b}/{gpr}/{d}/{sigma}", (m, n), sigma, "bf16")
    gdx, gdl = _bwd16(idx, lut, X, dY, b, gpr, d, "bf16", "f16")
    dY64, L64 = syn.to_float64(dY, "bf16"), syn.to_float64(lut, "f16")
    want = oracle.backward_dx(dY64, idx, L64, d, b, gpr)
    assert oracle.rel_err(gdx, want) <= TOL16
    assert max(_row_errs(gdx, want)) <= TOL16
    assert oracle.rel_err(gdl, oracle.backward_dlut(dY64, syn.to_float64(X, "bf16"), idx, b, gpr)) <= TOL16


def test_dx_rows_of_different_scales_bf16_f16():
    """Each token row of dY at its own scale (2^-60 .. 2^40): every row of dX within the tolerance."""
    b, gpr, n, d, m = 4, 8, 300, 4096, 70
    idx, lut, X, _ = make_case("dxrows", n, d, b, gpr, m, "bf16", "f16")
    dY = _scaled_rows("dxrows/dY", (m, n), [2.0 ** k for k in range(-60, 41, 10)])
    gdx, _ = _bwd16(idx, lut, X, dY, b, gpr, d, "bf16", "f16")
    want = oracle.backward_dx(syn.to_float64(dY, "bf16"), idx, syn.to_float64(lut, "f16"), d, b, gpr)
    assert max(_row_errs(gdx, want)) <= TOL16


@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 8, 256, 4096, 1), (4, 4, 64, 8192, 4),       # decode, activations staged in LDS
    (3, 4, 40, 16384, 3),                            # decode, 96 KB of activations staged (few tokens, few rows)
    (4, 8, 64, 4096, 16), (3, 4, 40, 16384, 5),      # decode, activations read per slot (row exponents from the workspace)
    (4, 8, 200, 4096, 300), (2, 8, 130, 11008, 40),  # GEMM, 64- and 32-column K-steps
    (3, 1, 33, 96, 19),
])
@pytest.mark.parametrize("scale", [3e4, 1e-6, 1e-32])
def test_fwd_activation_scales_bf16_f16(b, gpr, n, d, m, scale):
    """X ~ N(0, scale) in bf16: entries up to ~1e5 (beyond f16's largest) or rows far below f16's normal
    range, through every forward path; every output row within the tolerance. The GEMM blocks take the
    multiply (3e4 with 1e5 entries; 1e-32, rows below 2^-87) and exponent-add (1e-6) conversions."""
    idx, lut, _, _ = make_case(f"fwdscale/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, 1, "bf16", "f16")
    X = syn.random_normal(f"fwdscale/{b}/{gpr}/{n}/{d}/{m}/{scale}", (m, d), scale, "bf16")
    if scale > 1:
        X[0, :4] = syn.to_storage(np.array([1e5, -1e5, 7e4, -9e4], dtype=np.float32), "bf16")
    got, want = _fwd16(idx, lut, X, b, gpr, "bf16", "f16")
    assert np.all(np.isfinite(got))
    assert max(_row_errs(got, want)) <= TOL16


@pytest.mark.parametrize("m,d", [(1, 4096), (16, 2048), (16, 4096), (300, 4096)])
def test_fwd_rows_of_different_scales_bf16_f16(m, d):
    """Each token row at its own scale (2^-70 .. 2^60): every output row within the tolerance."""
    b, gpr, n = 4, 8, 96
    idx, lut, _, _ = make_case(f"fwdrows/{m}/{d}", n, d, b, gpr, 1, "bf16", "f16")
    X = _scaled_rows(f"fwdrows/{m}/{d}/X", (m, d), [2.0 ** k for k in range(-70, 61, 10)])
    got, want = _fwd16(idx, lut, X, b, gpr, "bf16", "f16")
    assert max(_row_errs(got, want)) <= TOL16


# bf16 row maxima at the edges of [2^-2, 2^16), the window of rows converted without a prescale:
# 2^-2 and 65280 (the largest bf16 below 2^16) lie inside it, 2^-2 - 2^-10 and 2^16 outside
_WINDOW_EDGES = [0.25, 0.25 - 2.0 ** -10, 65280.0, 65536.0]


@pytest.mark.parametrize("peak", _WINDOW_EDGES)
@pytest.mark.parametrize("d", [4096, 28672, 40960])
def test_decode_window_edge_rows_bf16_f16(peak, d):
    """One token whose largest magnitude sits at an edge of the unscaled window (the staging decode checks
    the window and, outside it, re-stages the activations prescaled): the output within the tolerance."""
    b, gpr, n = 4, 4, 80
    idx, lut, _, _ = make_case(f"window/{d}", n, d, b, gpr, 1, "bf16", "f16")
    z = syn.random_normal(f"window/{d}/{peak}", (1, d), 1.0, "f32").astype(np.float64)
    x = np.clip(z / 4.0, -0.999, 0.999) * peak
    x[0, d // 3] = -peak
    X = syn.to_storage(x.astype(np.float32), "bf16")
    assert np.max(np.abs(syn.to_float64(X, "bf16"))) == peak
    got, want = _fwd16(idx, lut, X, b, gpr, "bf16", "f16")
    assert np.all(np.isfinite(got))
    assert max(_row_errs(got, want)) <= TOL16


@pytest.mark.parametrize("zero_row", [False, True])
def test_decode_window_mixed_rows_bf16_f16(zero_row):
    """Staged rows at every window edge together (one row outside it sends the whole block to the exact
    path), and optionally a row of zeros (whose outputs must be exactly 0): every output row within the
    tolerance."""
    b, gpr, n, d = 4, 8, 96, 4096
    m = len(_WINDOW_EDGES) + 2
    idx, lut, _, _ = make_case("windowmix", n, d, b, gpr, 1, "bf16", "f16")
    z = syn.random_normal("windowmix/X", (m, d), 1.0, "f32").astype(np.float64)
    peaks = _WINDOW_EDGES + [1.0, 0.0 if zero_row else 3.0]
    x = np.clip(z / 4.0, -0.999, 0.999) * np.asarray(peaks)[:, None]
    x[np.arange(m), (np.arange(m) * 37) % d] = peaks
    X = syn.to_storage(x.astype(np.float32), "bf16")
    got, want = _fwd16(idx, lut, X, b, gpr, "bf16", "f16")
    if zero_row:
        assert np.all(got[-1] == 0.0)
        got, want = got[:-1], want[:-1]
    assert max(_row_errs(got, want)) <= TOL16


@pytest.mark.parametrize("sets,d,n_sets", [
    ([0, 1, 2, 1], 4096, 3), ([1] * 12 + [0] * 4, 4096, 3), ([0, 1, 0], 16384, 3),
    # rows longer than the staging holds, 8 and 16 set slots, one table set
    ([2, 0, 1, 2, 1], 36864, 3), (list(range(8)), 2048, 8), ([15 - t for t in range(16)], 2048, 16),
    ([0, 0, 0, 0, 0, 0], 4096, 1)])
def test_fwd_multi_scales_bf16_f16(sets, d, n_sets):
    """Several table sets: token rows at their own scales (2^-66 .. 2^30, prescaled per row by powers of two:
    the row exponents come from the staged rows in the one-pass-per-set kernel and from a scan of each token
    row in the set-interleaved one); every row within the tolerance."""
    b, gpr, n = 4, 8, 64
    m = len(sets)
    idx, luts, _ = _multi_case(f"multiscale/{m}/{d}/{n_sets}", n, d, b, gpr, 1, n_sets, "bf16", "f16")
    X = _scaled_rows(f"multiscale/{m}/{d}/X", (m, d), [2.0 ** k for k in (-40, 17, -3, 30, -66, 8)])
    got = to_f64(_fwd_multi(idx, luts, X, sets, b, gpr, "bf16", "f16"))
    want = oracle.forward_multi(syn.to_float64(X, "bf16"), idx, syn.to_float64(luts, "f16"), sets, b, gpr)
    assert max(_row_errs(got, want)) <= TOL16


# ---------------------------------------------------------------------------
# table gradient split over column and token ranges (small (row block, group) grids)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("io", ["f16", "bf16"])
@pytest.mark.parametrize("b,gpr,n,d,m", [
    (4, 1, 256, 512, 640),     # 2 row blocks in one group: token ranges, whole 32-token steps (DMA kernel)
    (2, 1, 130, 1024, 1000),   # 2 column and 8 token ranges, ragged rows, ragged last token range (register-staged)
    (3, 2, 64, 1536, 4096),    # 2 blocks, 3-bit
    (4, 1, 96, 256, 200),      # too few tokens to split (fewer than 8 steps)
    (3, 1, 8100, 2560, 256),   # 64 row blocks, ragged rows: column ranges of 2, 2 and 1 chunks
])
def test_dlut_split(io, b, gpr, n, d, m):
    idx, lut, X, dY = make_case(f"dlsplit/{io}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m, io, io)
    gdx, gdl = _bwd16(idx, lut, X, dY, b, gpr, d, io, io)
    L64, X64, dY64 = syn.to_float64(lut, io), syn.to_float64(X, io), syn.to_float64(dY, io)
    assert oracle.rel_err(gdl, oracle.backward_dlut(dY64, X64, idx, b, gpr)) <= TOL16
    assert oracle.rel_err(gdx, oracle.backward_dx(dY64, idx, L64, d, b, gpr)) <= TOL16
    # deterministic, and accumulate adds to the given table
    _, gdl2 = _bwd16(idx, lut, X, dY, b, gpr, d, io, io)
    assert np.array_equal(gdl, gdl2)
    base = np.random.default_rng(5).normal(size=gdl.shape).astype(np.float32)
    _, acc = _bwd16(idx, lut, X, dY, b, gpr, d, io, io, accumulate=True, dlut_init=base)
    assert np.allclose(acc, base.astype(np.float64) + gdl, rtol=0, atol=1e-6 * max(1.0, np.abs(gdl).max()))


def test_dlut_split_bins_exact():
    """Integer dY, one-hot X, split over 4 column and 8 token ranges: every bin sum is the exact integer."""
    b, gpr, n, d, m = 4, 1, 256, 2048, 1024
    idx, lut, _, _ = make_case("dlsplitbins", n, d, b, gpr, 1, "bf16", "bf16")
    cols = np.random.default_rng(77).choice(d, m, replace=True)
    X = np.zeros((m, d), dtype=np.float32)
    X[np.arange(m), cols] = 1.0
    dY = syn.random_int_valued("dlsplitbins/dY", (m, n), -3, 3, "bf16")
    _, gdl = _bwd16(idx, lut, syn.to_storage(X, "bf16"), dY, b, gpr, d, "bf16", "bf16")
    want = oracle.backward_dlut(syn.to_float64(dY, "bf16"), X.astype(np.float64), idx, b, gpr)
    assert np.array_equal(gdl, want)


def test_dlut_split_7b_gpr1_sampled():
    """4096 x 4096 at one group per row (32 row blocks) and 8192 tokens: the gradient split over 8 column
    ranges of 512 columns, checked on sampled rows against the oracle."""
    b, gpr, n, d, m = 4, 1, 4096, 4096, 8192
    idx, lut, X, dY = make_case("dlsplit7b", n, d, b, gpr, m, "bf16", "f16", dy_sigma=1e-2)
    ws = skm().sketch_matmul_bwd_workspace(m, n, d, b, gpr, skm().SKM_BF16, skm().SKM_F16)
    assert ws >= 8 * n * 16 * 4     # the partial tables of the column ranges
    _, dL = skm().sketch_matmul_bwd(to_dev(dY, "bf16"), to_dev(X, "bf16"), to_dev(idx, "u8"), to_dev(lut, "f16"),
                                    b, gpr, need_dx=False)
    dL = to_f64(dL)
    rows = _workload_rows(n, 99)
    want = oracle.backward_dlut(syn.to_float64(dY, "bf16")[:, rows], syn.to_float64(X, "bf16"), idx[rows], b, gpr)
    assert oracle.rel_err(dL[rows], want) <= TOL16
