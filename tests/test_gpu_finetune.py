"""GPU parity of the fine-tuning glue: fused table optimizer steps, autograd and grouped layers.

Optimizer steps run in fp32 on the GPU and in float64 in the oracle; master
tables and moments are scored elementwise, |gpu - oracle| <= 1e-5 |oracle| +
1e-7 max|oracle| (fp32 tolerance). The 16-bit compute copy must be bit-exact
the nearest-even rounding of the GPU's own fp32 master (the rounding decision
is taken from the same fp32 value on both sides). Forward outputs and
gradients use the parity tests' scoring (max-norm relative error, 5e-3 for
16-bit I/O, 1e-5 for the fp32 path).
"""
import numpy as np
import pytest

import oracle
from lut_sketched_matmul_amd import synthetic as syn

from gpu_util import round_to, to_dev, to_f64

pytestmark = pytest.mark.gpu

TOL16 = 5e-3
TOL32 = 1e-5


def skm():
    import lut_sketched_matmul_amd as m
    return m


def ft():
    from lut_sketched_matmul_amd import finetune
    return finetune


def torch():
    import torch as _t
    return _t


def tdtype(name):
    t = torch()
    return {"f32": t.float32, "f16": t.float16, "bf16": t.bfloat16}[name]


def assert_close_elementwise(got, ref, tol=1e-5, what=""):
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
    bad = np.abs(got - ref) > tol * np.abs(ref) + 1e-7 * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} entries off, first at {np.argwhere(bad)[:3].ravel()}"


def assert_rel(got, ref, tol, what=""):
    err = float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30)
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol}"


def f32(v):
    """A hyperparameter as the library receives it (the C ABI takes fp32 values): the oracle is given the
    same value, so 1 - beta2 is compared for beta2 = 0.999f on both sides."""
    if isinstance(v, tuple):
        return tuple(f32(x) for x in v)
    return float(np.float32(v))


def check_copy(copy, master_dev, dtype):
    if copy is None:
        return
    src = to_f64(master_dev)
    want, got = round_to(src, dtype), to_f64(copy)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"16-bit copy is not the rounding of the fp32 master at {bad.size} entries: "
                           + "; ".join(f"[{i}] master {src[i]!r} copy {got[i]!r} want {want[i]!r}" for i in bad[:6]))


# ---------------------------------------------------------------------------
# fused optimizer steps
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("copy", [None, "f16", "bf16"])
@pytest.mark.parametrize("count", [8, 13, 4101, (1 << 20) + 3])
def test_adam_step(count, copy):
    t = torch()
    tag = f"adam/{count}/{copy}"
    master = to_dev(syn.random_normal(f"{tag}/p", (count,), 0.02, "f32"), "f32")
    m1 = t.zeros(count, dtype=t.float32, device="cuda:0")
    m2 = t.zeros(count, dtype=t.float32, device="cuda:0")
    lut = t.empty(count, dtype=tdtype(copy), device="cuda:0") if copy else None
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, grad_scale=0.5)
    for step in range(1, 4):
        g = syn.random_normal(f"{tag}/g{step}", (count,), 1.0, "f32")
        g[::7] *= np.float32(1e-4)      # gradients near eps in some entries
        prev = [to_f64(x) for x in (master, m1, m2)]
        skm().sketch_lut_adam_step(master, to_dev(g, "f32"), m1, m2, step, hp["lr"], hp["beta1"], hp["beta2"],
                                   hp["eps"], hp["weight_decay"], hp["grad_scale"], lut=lut)
        ref = oracle.adam_step(prev[0], g.astype(np.float64), prev[1], prev[2], step,
                               **{k: f32(v) for k, v in hp.items()})
        for got, want, what in zip((master, m1, m2), ref, ("master", "exp_avg", "exp_avg_sq")):
            assert_close_elementwise(to_f64(got), want, what=f"step {step} {what}")
        check_copy(lut, master, copy)


@pytest.mark.parametrize("copy", [None, "f16", "bf16"])
@pytest.mark.parametrize("momentum,wd", [(0.0, 0.0), (0.9, 0.0), (0.9, 0.02)])
@pytest.mark.parametrize("count", [13, 65541])
def test_sgd_step(count, momentum, wd, copy):
    t = torch()
    tag = f"sgd/{count}/{momentum}/{wd}/{copy}"
    master = to_dev(syn.random_normal(f"{tag}/p", (count,), 0.02, "f32"), "f32")
    buf = t.zeros(count, dtype=t.float32, device="cuda:0") if momentum else None
    lut = t.empty(count, dtype=tdtype(copy), device="cuda:0") if copy else None
    ref_buf = None
    for step in range(1, 4):
        g = syn.random_normal(f"{tag}/g{step}", (count,), 1e-2, "f32")
        prev = to_f64(master)
        prev_buf = to_f64(buf) if buf is not None else None
        skm().sketch_lut_sgd_step(master, to_dev(g, "f32"), 0.05, momentum, wd, 2.0, momentum_buf=buf, lut=lut)
        ref, ref_buf = oracle.sgd_step(prev, g.astype(np.float64), f32(0.05), f32(momentum), f32(wd), 2.0, prev_buf)
        assert_close_elementwise(to_f64(master), ref, what=f"step {step} master")
        if buf is not None:
            assert_close_elementwise(to_f64(buf), ref_buf, what=f"step {step} momentum")
        check_copy(lut, master, copy)


def test_optimizer_steps_reject_mismatched_buffers():
    t = torch()
    a = t.zeros(64, dtype=t.float32, device="cuda:0")
    with pytest.raises(ValueError):
        skm().sketch_lut_adam_step(a, t.zeros(32, dtype=t.float32, device="cuda:0"), t.zeros_like(a),
                                   t.zeros_like(a), 1, 1e-3)
    with pytest.raises(skm().SketchError):
        skm().sketch_lut_adam_step(a, t.zeros_like(a), t.zeros_like(a), t.zeros_like(a), 0, 1e-3)
    with pytest.raises(skm().SketchError):
        skm().sketch_lut_sgd_step(a, a, 1e-3)       # master over the gradient


# ---------------------------------------------------------------------------
# autograd
# ---------------------------------------------------------------------------

def make_layer_case(tag, n, d, b, gpr, m, io, lut_dtype):
    idx = syn.random_packed_indices(f"{tag}/idx", n, d, b)
    lut = syn.random_lut(f"{tag}/lut", n, gpr, b, 0.02, lut_dtype)
    X = syn.random_normal(f"{tag}/X", (m, d), 1.0, io)
    R = syn.random_normal(f"{tag}/R", (m, n), 1.0, io)
    return idx, lut, X, R


@pytest.mark.parametrize("io,lut_dtype,b,gpr,n,d,m", [
    ("bf16", "f16", 4, 8, 96, 1024, 8),      # decode-sized forward
    ("f16", "f16", 4, 4, 64, 512, 40),       # matrix-core forward
    ("bf16", "bf16", 3, 2, 80, 1024, 64),
    ("f16", "bf16", 2, 1, 50, 256, 3),
    ("f32", "f32", 4, 1, 48, 256, 4),        # fp32 path
])
def test_autograd_matches_oracle(io, lut_dtype, b, gpr, n, d, m):
    t = torch()
    tol = TOL32 if io == "f32" else TOL16
    idx, lut, X, R = make_layer_case(f"ag/{io}/{lut_dtype}/{b}/{gpr}/{n}/{d}/{m}", n, d, b, gpr, m, io, lut_dtype)
    layer = ft().SketchedLinear(to_dev(idx, "u8"), to_dev(lut, lut_dtype), d, b, gpr, compute_dtype=tdtype(lut_dtype))
    Xt = to_dev(X, io).requires_grad_(True)
    Y = layer(Xt)
    Y.backward(to_dev(R, io))
    X64, R64, L64 = syn.to_float64(X, io), syn.to_float64(R, io), syn.to_float64(lut, lut_dtype)
    assert Y.dtype == tdtype(io) and Xt.grad.dtype == tdtype(io)
    assert layer.lut_master.grad.dtype == t.float32
    assert_rel(to_f64(Y), oracle.forward(X64, idx, L64, b, gpr), tol, "Y")
    assert_rel(to_f64(Xt.grad), oracle.backward_dx(R64, idx, L64, d, b, gpr), tol, "dX")
    assert_rel(to_f64(layer.lut_master.grad), oracle.backward_dlut(R64, X64, idx, b, gpr), tol, "dLUT")


def test_autograd_only_table_gradient():
    idx, lut, X, R = make_layer_case("ag-frozen-x", 64, 512, 4, 4, 24, "bf16", "f16")
    layer = ft().SketchedLinear(to_dev(idx, "u8"), to_dev(lut, "f16"), 512, 4, 4)
    Y = layer(to_dev(X, "bf16"))            # X does not require a gradient: dX is skipped
    Y.backward(to_dev(R, "bf16"))
    want = oracle.backward_dlut(syn.to_float64(R, "bf16"), syn.to_float64(X, "bf16"), idx, 4, 4)
    assert_rel(to_f64(layer.lut_master.grad), want, TOL16, "dLUT")


@pytest.mark.parametrize("m", [4, 40])
def test_grouped_layer_matches_oracle(m):
    sizes, d, b, gpr = (64, 32, 96), 512, 4, 4
    cases = [make_layer_case(f"grp/{m}/{k}", nk, d, b, gpr, m, "bf16", "f16") for k, nk in enumerate(sizes)]
    X = cases[0][2]
    layer = ft().GroupedSketchedLinear([to_dev(c[0], "u8") for c in cases], [to_dev(c[1], "f16") for c in cases],
                                       d, b, gpr)
    Xt = to_dev(X, "bf16").requires_grad_(True)
    outs = layer(Xt)
    loss = sum((o.float() * to_dev(c[3], "bf16").float()).sum() for o, c in zip(outs, cases))
    loss.backward()
    X64 = syn.to_float64(X, "bf16")
    dx_ref = np.zeros_like(X64)
    for o, g, c in zip(outs, layer.table_slices(), cases):
        idx, L64, R64 = c[0], syn.to_float64(c[1], "f16"), syn.to_float64(c[3], "bf16")
        assert_rel(to_f64(o), oracle.forward(X64, idx, L64, b, gpr), TOL16, "Y")
        dx_ref += oracle.backward_dx(R64, idx, L64, d, b, gpr)
    grads = list(layer.lut_master.grad.split(list(sizes), 0))
    for gr, c in zip(grads, cases):
        want = oracle.backward_dlut(syn.to_float64(c[3], "bf16"), X64, c[0], b, gpr)
        assert_rel(to_f64(gr), want, TOL16, "dLUT")
    assert_rel(to_f64(Xt.grad), dx_ref, TOL16, "dX")


# ---------------------------------------------------------------------------
# training steps in lockstep with the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("opt", ["adam", "sgd"])
def test_training_steps_lockstep(opt):
    """Each step: forward from the current 16-bit copy, backward, fused update; every piece against the oracle
    applied to the GPU's state at the start of that step."""
    t = torch()
    n, d, b, gpr, m = 64, 512, 4, 4, 32
    idx, lut, _, _ = make_layer_case(f"train/{opt}", n, d, b, gpr, m, "bf16", "f16")
    layer = ft().SketchedLinear(to_dev(idx, "u8"), to_dev(lut, "f16"), d, b, gpr)
    if opt == "adam":
        hp = dict(lr=2e-3, betas=(0.9, 0.99), eps=1e-8, weight_decay=0.01, grad_scale=1.0 / m)
        optim = ft().LutAdam([layer.lut_master], **hp)
    else:
        hp = dict(lr=0.05, momentum=0.9, weight_decay=0.0, grad_scale=1.0 / m)
        optim = ft().LutSGD([layer.lut_master], **hp)
    moved = 0.0
    start = to_f64(layer.lut_master)
    for step in range(1, 4):
        X = syn.random_normal(f"train/{opt}/X{step}", (m, d), 1.0, "bf16")
        R = syn.random_normal(f"train/{opt}/R{step}", (m, n), 1.0, "bf16")
        X64, R64 = syn.to_float64(X, "bf16"), syn.to_float64(R, "bf16")
        copy0, master0 = to_f64(layer.lut), to_f64(layer.lut_master)
        st = optim.state.get(layer.lut_master, {})
        optim.zero_grad()
        Y = layer(to_dev(X, "bf16"))
        Y.backward(to_dev(R, "bf16"))
        g_gpu = to_f64(layer.lut_master.grad)
        assert_rel(to_f64(Y), oracle.forward(X64, idx, copy0, b, gpr), TOL16, f"step {step} Y")
        assert_rel(g_gpu, oracle.backward_dlut(R64, X64, idx, b, gpr), TOL16, f"step {step} dLUT")
        if opt == "adam":
            m0 = to_f64(st["exp_avg"]) if st else np.zeros_like(master0)
            v0 = to_f64(st["exp_avg_sq"]) if st else np.zeros_like(master0)
            optim.step()
            want, _, _ = oracle.adam_step(master0, g_gpu, m0, v0, step, f32(hp["lr"]), f32(hp["betas"][0]),
                                          f32(hp["betas"][1]), f32(hp["eps"]), f32(hp["weight_decay"]),
                                          f32(hp["grad_scale"]))
        else:
            b0 = to_f64(st["momentum_buffer"]) if st else None
            optim.step()
            want, _ = oracle.sgd_step(master0, g_gpu, f32(hp["lr"]), f32(hp["momentum"]), f32(hp["weight_decay"]),
                                      f32(hp["grad_scale"]), b0)
        assert_close_elementwise(to_f64(layer.lut_master), want, what=f"step {step} master")
        check_copy(layer.lut, layer.lut_master, "f16")
        moved = float(np.max(np.abs(to_f64(layer.lut_master) - start)))
    assert moved > 0.0
    assert t.equal(layer.idx_packed.cpu(), t.from_numpy(idx))      # the mapping stays frozen


def test_training_recovers_tables():
    """Fine-tuning end to end: the target layer uses the same frozen mapping with other tables, so the
    tables can be recovered exactly; SGD through the autograd function and the fused optimizer step must
    bring the loss on fresh random batches down by three orders of magnitude (60 steps, f16)."""
    t = torch()
    n, d, b, gpr, m = 128, 512, 4, 4, 32
    idx = syn.random_packed_indices("recover/idx", n, d, b)
    target = syn.random_lut("recover/target", n, gpr, b, 0.02, "f16")
    noise = syn.random_normal("recover/noise", (n, gpr, 1 << b), 0.01, "f32").astype(np.float64)
    start = syn.to_storage(syn.to_float64(target, "f16") + noise, "f16")
    gi = to_dev(idx, "u8")
    layer = ft().SketchedLinear(gi, to_dev(start, "f16"), d, b, gpr)
    goal = to_dev(target, "f16")
    opt = ft().LutSGD([layer.lut_master], lr=2.0, grad_scale=1.0 / (m * n))
    losses = []
    for step in range(60):
        X = to_dev(syn.random_normal(f"recover/X{step}", (m, d), 1.0, "f16"), "f16")
        with t.no_grad():
            Ystar = skm().sketch_matmul_fwd(X, gi, goal, b, gpr).float()
        opt.zero_grad()
        loss = ((layer(X).float() - Ystar) ** 2).sum()
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    assert losses[-1] < 1e-3 * losses[0], (losses[0], losses[-1])
    # entries that some columns map to approach the target; an entry no column
    # maps to gets a zero gradient and keeps its starting value exactly
    u = oracle.unpack_indices(idx, d, b)
    uses = np.zeros((n, gpr, 1 << b), dtype=np.int64)
    np.add.at(uses, (np.arange(n)[:, None], (np.arange(d) // (d // gpr))[None, :], u), 1)
    got, tgt, st = to_f64(layer.lut_master), syn.to_float64(target, "f16"), syn.to_float64(start, "f16")
    well = uses >= 4
    err0 = np.abs(st - tgt)[well].max()
    err = np.abs(got - tgt)[well].max()
    assert err < 0.05 * err0, (err0, err)
    assert np.array_equal(got[uses == 0], st[uses == 0])
