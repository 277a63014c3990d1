"""Host-side checks of the C ABI: the library loads, exports every declared
function, and rejects bad arguments before launching anything (no GPU needed:
every call below fails its argument checks on the host)."""
import ctypes

import pytest

import lut_sketched_matmul_amd as skm
from lut_sketched_matmul_amd import _lib

EINVAL, EUNSUP, EALIGN, EWS, EALIAS = -1, -2, -3, -4, -6
A = 0x10000          # fake, 16-byte aligned "device" addresses; never dereferenced
B_ = 0x20000000
C = 0x40000000
Dp = 0x60000000


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert {"sketch_matmul_fwd", "sketch_matmul_fwd_multi", "sketch_matmul_bwd", "sketch_matmul_bwd_workspace", "sketch_dequant",
            "sketch_unpack_indices", "sketch_status_str", "sketch_version", "sketch_lut_adam_step",
            "sketch_lut_sgd_step", "sketch_column_weights", "sketch_lloyd", "sketch_map",
            "sketch_map_workspace"} <= set(names)
    for nme in names:
        assert hasattr(lib, nme), nme


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, 12345):
        assert lib.sketch_status_str(code)
    assert lib.sketch_version() >= 100


def fwd(lib, X=A, xdt=1, idx=B_, lut=C, ldt=1, m=4, n=64, d=512, b=4, gpr=1, Y=Dp):
    return lib.sketch_matmul_fwd(X, xdt, idx, lut, ldt, m, n, d, b, gpr, Y, None, 0, None)


def test_fwd_rejects_bad_shapes(lib):
    assert fwd(lib, b=1) == EINVAL
    assert fwd(lib, b=5) == EINVAL
    assert fwd(lib, gpr=0) == EINVAL
    assert fwd(lib, d=512, gpr=3) == EINVAL            # d % gpr != 0
    assert fwd(lib, d=512, gpr=32) == EINVAL           # group of 16 columns
    assert fwd(lib, d=48) == EINVAL
    assert fwd(lib, m=-1) == EINVAL
    assert fwd(lib, n=0) == EINVAL


def test_fwd_workspace_follows_activation_staging(lib):
    """(BF16, F16): the decode needs the row-exponent workspace exactly when it reads its activations per
    slot; it stages them up to 32768 elements, and below 8 tokens up to 49152 on at most 4096 rows when the
    block's LDS holds them."""
    BF16, F16 = 2, 1
    ws = lambda m, n, d, b, gpr, x=BF16: lib.sketch_matmul_fwd_workspace(m, n, d, b, gpr, x, F16)
    assert ws(8, 64, 4096, 4, 8) == 0                  # 32768 elements
    assert ws(9, 64, 4096, 4, 8) == 256                # more, and 8 tokens or more: per slot
    assert ws(4, 64, 11008, 2, 8) == 0                 # 44032 elements, few rows
    assert ws(4, 4096, 11008, 2, 8) == 0
    assert ws(4, 4112, 11008, 2, 8) == 256             # more than one 16-row block per CU
    assert ws(3, 40, 16384, 3, 4) == 0                 # 49152 elements
    assert ws(5, 40, 16384, 3, 4) == 256
    assert ws(4, 64, 12096, 4, 14) == 256              # 224-entry tables: 168 KB of LDS would not fit
    assert ws(4, 64, 11008, 2, 8, x=F16) == 0          # no prescale for the (F16, F16) pair


def test_fwd_rejects_bad_pointers_and_dtypes(lib):
    assert fwd(lib, idx=0) == EINVAL
    assert fwd(lib, lut=0) == EINVAL
    assert fwd(lib, X=0) == EINVAL
    assert fwd(lib, Y=0) == EINVAL
    assert fwd(lib, X=A + 2) == EALIGN
    assert fwd(lib, idx=B_ + 8) == EALIGN
    assert fwd(lib, xdt=0, ldt=1) == EUNSUP           # fp32 activations need fp32 tables
    assert fwd(lib, xdt=1, ldt=0) == EUNSUP
    assert fwd(lib, xdt=7) == EUNSUP
    assert fwd(lib, Y=A) == EALIAS                    # output over the input
    assert fwd(lib, Y=C + 16) == EALIAS


def test_fwd_empty_is_noop(lib):
    assert fwd(lib, m=0, X=0, Y=0) == 0


def fwd_multi(lib, X=A, xdt=1, idx=B_, luts=C, ldt=1, sets=0x50000000, ns=2, m=4, n=64, d=512, b=4, gpr=1, Y=Dp):
    return lib.sketch_matmul_fwd_multi(X, xdt, idx, luts, ldt, sets, ns, m, n, d, b, gpr, Y, None)


def test_fwd_multi_rejects_bad_arguments(lib):
    assert fwd_multi(lib, ns=0) == EINVAL
    assert fwd_multi(lib, sets=0) == EINVAL
    assert fwd_multi(lib, b=5) == EINVAL
    assert fwd_multi(lib, sets=0x50000002) == EALIGN
    assert fwd_multi(lib, m=17) == EUNSUP               # decode-sized batches only
    assert fwd_multi(lib, xdt=0, ldt=0) == EUNSUP       # no fp32 path
    # (BF16, F16) rows over 32768 columns: one token stages its row (at most 32768
    # columns), and more than 8 tokens take two cells per entry (at most 128 entries)
    assert fwd_multi(lib, xdt=2, ldt=1, m=1, d=36864) == EUNSUP
    assert fwd_multi(lib, xdt=2, ldt=1, m=9, d=36864, gpr=9) == EUNSUP
    assert fwd_multi(lib, Y=0x50000000) == EALIAS       # output over the set array
    assert fwd_multi(lib, Y=C + 2048) == EALIAS         # output over the second table set
    assert fwd_multi(lib, m=0, X=0, Y=0, sets=0) == 0


def bwd(lib, dY=A, X=Dp, dt=1, idx=B_, lut=C, ldt=1, m=4, n=64, d=512, b=4, gpr=1, dX=0x70000000,
        dL=0x78000000, acc=0, ws=0, wsb=0):
    return lib.sketch_matmul_bwd(dY, X, dt, idx, lut, ldt, m, n, d, b, gpr, dX, dL, acc, ws, wsb, None)


def test_bwd_rejects_bad_arguments(lib):
    assert bwd(lib, b=6) == EINVAL
    assert bwd(lib, acc=2) == EINVAL
    assert bwd(lib, dY=0) == EINVAL
    assert bwd(lib, X=0) == EINVAL                    # dLUT needs X
    assert bwd(lib, dX=0x70000004) == EALIGN
    assert bwd(lib, dt=0) == EUNSUP
    assert bwd(lib, dX=A) == EALIAS
    assert bwd(lib, dL=0x70000000) == EALIAS          # dX and dLUT overlap


def adam(lib, p=A, lut=B_, ldt=1, g=C, m1=Dp, m2=0x70000000, count=1000, step=1, lr=1e-3, b1=0.9, b2=0.999,
         eps=1e-8, wd=0.0, gs=1.0):
    return lib.sketch_lut_adam_step(p, lut, ldt, g, m1, m2, count, step, lr, b1, b2, eps, wd, gs, None)


def sgd(lib, p=A, lut=B_, ldt=1, g=C, buf=Dp, count=1000, lr=1e-2, mom=0.9, wd=0.0, gs=1.0):
    return lib.sketch_lut_sgd_step(p, lut, ldt, g, buf, count, lr, mom, wd, gs, None)


def test_adam_step_rejects_bad_arguments(lib):
    assert adam(lib, count=-1) == EINVAL
    assert adam(lib, step=0) == EINVAL
    assert adam(lib, lr=-1.0) == EINVAL
    assert adam(lib, lr=float("nan")) == EINVAL
    assert adam(lib, b1=1.0) == EINVAL
    assert adam(lib, b2=-0.1) == EINVAL
    assert adam(lib, eps=float("inf")) == EINVAL
    assert adam(lib, gs=float("nan")) == EINVAL
    assert adam(lib, ldt=0) == EUNSUP                  # the compute copy is 16-bit
    assert adam(lib, m1=0) == EINVAL
    assert adam(lib, g=0) == EINVAL
    assert adam(lib, m2=0x70000008) == EALIGN
    assert adam(lib, lut=B_ + 2) == EALIGN
    assert adam(lib, m1=A + 3984) == EALIAS            # first moment over the master's last entries
    assert adam(lib, lut=C) == EALIAS                  # copy over the gradient
    assert adam(lib, count=0, p=0, g=0, m1=0, m2=0) == 0
    assert adam(lib, b1=0.0, b2=0.0, count=0) == 0


def test_sgd_step_rejects_bad_arguments(lib):
    assert sgd(lib, count=-1) == EINVAL
    assert sgd(lib, mom=-0.5) == EINVAL
    assert sgd(lib, wd=float("nan")) == EINVAL
    assert sgd(lib, buf=0) == EINVAL                   # momentum needs its buffer
    assert sgd(lib, ldt=2, lut=B_ + 8) == EALIGN
    assert sgd(lib, ldt=7) == EUNSUP
    assert sgd(lib, buf=A) == EALIAS
    assert sgd(lib, g=A + 16) == EALIAS
    assert sgd(lib, count=0, p=0, g=0) == 0


def test_construction_rejects_bad_arguments(lib):
    assert lib.sketch_column_weights(A, 0, B_, None) == EINVAL
    assert lib.sketch_column_weights(0, 64, B_, None) == EINVAL
    assert lib.sketch_column_weights(A, 64, A + 4096, None) == EALIAS      # h inside U (64 x 64 floats)
    assert lib.sketch_column_weights(A, 64, B_ + 4, None) == EALIGN
    lloyd = lambda W=A, h=B_, n=64, d=512, b=4, gpr=4, it=10, lut=C, ldt=1: lib.sketch_lloyd(
        W, h, n, d, b, gpr, it, lut, ldt, None)
    assert lloyd(b=5) == EINVAL
    assert lloyd(gpr=3) == EINVAL
    assert lloyd(it=-1) == EINVAL
    assert lloyd(ldt=9) == EUNSUP
    assert lloyd(lut=0) == EINVAL
    assert lloyd(h=B_ + 8) == EALIGN
    assert lloyd(lut=A + 1024) == EALIAS
    ws = lib.sketch_map_workspace(64)
    assert ws >= 64 * 64 * 4 and lib.sketch_map_workspace(0) == 0
    mp = lambda W=A, U=B_, lut=C, ldt=1, n=64, d=512, b=4, gpr=4, idx=Dp, w=0x70000000, wsb=ws: lib.sketch_map(
        W, U, lut, ldt, n, d, b, gpr, idx, w, wsb, None)
    assert mp(d=48) == EINVAL
    assert mp(w=0) == EINVAL
    assert mp(wsb=ws - 1) == EWS
    assert mp(idx=Dp + 2) == EALIGN
    assert mp(idx=A + 16) == EALIAS                     # indices over the weights
    assert mp(w=B_) == EALIAS                           # workspace over U
    assert mp(ldt=5) == EUNSUP


def test_hessian_factor_rejects_bad_arguments(lib):
    ws = lib.sketch_hessian_factor_workspace(100)
    # D = 128: 8 (128^2 + 128 * 64 + 32) bytes
    assert ws == 8 * (128 * 128 + 128 * 64 + 32)
    assert lib.sketch_hessian_factor_workspace(0) == 0 and lib.sketch_hessian_factor_workspace(1 << 17) == 0
    hf = lambda H=A, d=100, damp=0.01, U=B_, w=C, wsb=ws: lib.sketch_hessian_factor(H, d, damp, U, w, wsb, None)
    assert hf(d=0) == EINVAL
    assert hf(d=(1 << 16) + 1) == EINVAL
    assert hf(damp=-0.1) == EINVAL
    assert hf(damp=float("nan")) == EINVAL
    assert hf(damp=float("inf")) == EINVAL
    assert hf(H=0) == EINVAL
    assert hf(w=0) == EINVAL
    assert hf(wsb=ws - 1) == EWS
    assert hf(U=B_ + 4) == EALIGN
    assert hf(U=A + 8 * 100 * 100 - 16) == EALIAS       # U over the end of H
    assert hf(w=B_ + 16) == EALIAS                      # workspace over U


def test_dequant_and_unpack_reject(lib):
    assert lib.sketch_dequant(B_, C, 1, 64, 512, 7, 1, A, None) == EINVAL
    assert lib.sketch_dequant(B_, C, 9, 64, 512, 4, 1, A, None) == EUNSUP
    assert lib.sketch_unpack_indices(B_, 64, 40, 4, A, None) == EINVAL
    assert lib.sketch_unpack_indices(B_, 64, 512, 4, B_, None) == EALIAS


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setenv("SKETCHMM_LIB", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        _lib.lib()


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    # bf16 dY with f16 tables at 3 million tokens: 12 MB of row exponents > 8 MiB of scratch (no GPU call)
    assert lib.sketch_matmul_bwd_noalloc(A, B_, 2, C, Dp, 1, 3_000_000, 256, 1024, 4, 1, A, None, 0, None) == EWS
    assert lib.sketch_matmul_bwd_noalloc(A, B_, 2, C, Dp, 1, 64, 256, 1024, 5, 1, A, None, 0, None) == EINVAL
