#!/usr/bin/env python3
"""Benchmark of the sketched-weight matmul on one MI355X.

Headline: decode GEMV (m = 1 token) on the LLaMA-2-7B-shaped 4096 x 4096
projection (b = 4, 8 groups per row, fp16 tables and activations), in GB/s of
algorithmic traffic (indices + tables + X + Y) and as a fraction of the 8 TB/s
HBM peak. Every timed launch reads a different copy of the indices and tables
(>= 1 GiB in rotation) so the 256 MB last-level cache cannot serve repeats.

The same JSON line carries the other measured parts of the hot path (16-token
forward, the 7B MLP at 2 and 3 bits, decode with one table set per token over
one index stream, 70B-shaped decode and prefill GEMM, the 7B decoder-layer
fine-tuning step, the fused table optimizer steps and a grouped q/k/v decode,
LLaMA-2-13B decode at one group per row, the backward at 2 and 3 bits and at
one group per row, sketch construction of a 4096 x 4096 layer, a rotated
read-only stream of the decode calls' sizes) and the CPU oracle timed on this
host as a baseline. The CPU leg also scores each part's outputs (sampled rows,
tokens and columns) against the oracle: ``parity_err`` = max |gpu - oracle| /
max |oracle| on the sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "LUT-GEMV GB/s (% HBM peak) at 7B shapes; LUT-GEMM + bwd TFLOP/s (% MFMA)"
ROTATE_BYTES = 1 << 30
SPIN_MIN_MS = 0.5  # shortest hold of the stream before the timed launches
# rocprofv3 summary of the headline kernel (FETCH_SIZE / WRITE_SIZE counters)
DECODE_PROFILE = os.path.join(ROOT, "profiles", "k_decode_llama2_7b_attn_4096x4096_b4_m1.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--parts", default="all",
                    help="comma list of decode,fwd16,lowbit,multilut,decode70b,prefill,finetune,glue,13b,bwdlowbit,"
                         "bwdgpr1,construct,dense,copy,readref "
                         "(default all; decode always runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def dev(torch, a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


class Rotation:
    """Distinct device copies of (idx, lut) whose total size is >= ROTATE_BYTES."""

    def __init__(self, torch, idx, lut):
        per = idx.numel() * idx.element_size() + lut.numel() * lut.element_size()
        self.count = max(2, -(-ROTATE_BYTES // per))
        self.idx = [idx.clone() for _ in range(self.count)]
        self.lut = [lut.clone() for _ in range(self.count)]
        self.i = 0

    def next(self):
        k = self.i % self.count
        self.i += 1
        return self.idx[k], self.lut[k]


_SPIN_RATE = []  # cycles of torch.cuda._sleep per millisecond, measured once


def spin_cycles_per_ms(torch):
    if not _SPIN_RATE:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_RATE.append(2_000_000 / max(e0.elapsed_time(e1), 1e-3))
    return _SPIN_RATE[0]


def time_launches(torch, launch, steps, warmup, launches_per_step=1):
    """GPU time (ms) of `steps` back-to-back launches, from HIP events on the launch stream.

    The stream is held by a spin kernel while the host enqueues every timed
    launch, so the GPU then runs them back to back: the events measure the
    kernels and the dispatch gaps between them, not the host's submission time.
    The spin is sized from the host's own submission time per launch (twice
    the warm-up's median, measured here) at the spin kernel's measured rate; when the
    timed submissions still outlast it, the run is repeated with a spin sized
    from them.
    """
    del launches_per_step  # the spin is sized from measured host time
    stream = torch.cuda.current_stream()
    rate = spin_cycles_per_ms(torch)
    per = []
    for _ in range(max(1, warmup)):
        t0 = time.perf_counter()
        launch()
        per.append((time.perf_counter() - t0) * 1e3)
    host_ms = float(np.median(per))  # (the first calls may load code objects)
    torch.cuda.synchronize()
    for attempt in range(2):
        spin_ms = SPIN_MIN_MS + 2.0 * host_ms * steps
        first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(rate * spin_ms))
        t0 = time.perf_counter()
        first.record(stream)
        for _ in range(steps):
            launch()
        last.record(stream)
        submit_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        if submit_ms < spin_ms:
            break
        host_ms = submit_ms / max(1, steps)
    else:
        print(f"time_launches: host submission ({submit_ms:.2f} ms) outlasted the spin ({spin_ms:.2f} ms); "
              "the time may include host gaps", file=sys.stderr)
    return first.elapsed_time(last)


def sample_ids(count, k, seed):
    """Sorted sample of indices in [0, count): the first and last 16 and k random ones."""
    r = np.random.default_rng(seed)
    ids = np.concatenate([np.arange(min(16, count)), np.arange(max(0, count - 16), count),
                          r.choice(count, min(k, count), replace=False)])
    return np.unique(ids)


def fwd_workspace(torch, skm, X, lut, n, d, b, gpr):
    nb = skm.sketch_matmul_fwd_workspace(X.shape[0], n, d, b, gpr, skm._lib.dtype_code(X), skm._lib.dtype_code(lut))
    return torch.empty(nb, dtype=torch.uint8, device="cuda:0") if nb else None


def bwd_workspace(torch, skm, dY, lut, n, d, b, gpr):
    nb = skm.sketch_matmul_bwd_workspace(dY.shape[0], n, d, b, gpr, skm._lib.dtype_code(dY),
                                         skm._lib.dtype_code(lut))
    return torch.empty(nb, dtype=torch.uint8, device="cuda:0") if nb else None


def fwd_check(name, t, Y, b, gpr, x_dtype, lut_dtype, seed):
    """A parity sample of a forward output (scored by the CPU leg): sampled tokens x sampled rows."""
    m, n = Y.shape
    toks = sample_ids(m, 96, seed) if m > 128 else np.arange(m)
    rows = sample_ids(n, 224, seed + 1)
    got = Y.float().cpu().numpy()[np.ix_(toks, rows)].astype(np.float64)
    return {"name": name, "kind": "fwd", "X": t["X"][toks], "idx": t["idx_packed"][rows], "lut": t["lut"][rows],
            "b": b, "gpr": gpr, "x_dtype": x_dtype, "lut_dtype": lut_dtype, "got": got}


def bwd_checks(name, t, dX, dL, b, gpr, x_dtype, lut_dtype, seed):
    """Parity samples of dX (sampled tokens x sampled columns) and dLUT (sampled rows)."""
    out = []
    if dX is not None:
        m, d = dX.shape
        toks, cols = sample_ids(m, 96, seed), sample_ids(d, 224, seed + 1)
        out.append({"name": name + ".dx", "kind": "dx", "dY": t["dY"][toks], "idx": t["idx_packed"],
                    "lut": t["lut"], "cols": cols, "b": b, "gpr": gpr, "x_dtype": x_dtype, "lut_dtype": lut_dtype,
                    "got": dX.cpu().numpy()[np.ix_(toks, cols)].astype(np.float64)})
    if dL is not None:
        rows = sample_ids(dL.shape[0], 96, seed + 2)
        out.append({"name": name + ".dlut", "kind": "dlut", "dY": t["dY"][:, rows], "X": t["X"],
                    "idx": t["idx_packed"][rows], "b": b, "gpr": gpr, "x_dtype": x_dtype, "lut_dtype": lut_dtype,
                    "got": dL.cpu().numpy()[rows].astype(np.float64)})
    return out


CHECKS = []   # parity samples of the parts, scored against the oracle by the CPU leg


def bench_fwd(torch, skm, w, shape, b, m, steps, warmup, rotate=True, check=None):
    from lut_sketched_matmul_amd import workloads as wl
    t = w.make(shape, b, m)
    X = dev(torch, t["X"], w.x_dtype)
    idx = dev(torch, t["idx_packed"], "u8")
    lut = dev(torch, t["lut"], w.lut_dtype)
    Y = torch.empty((m, shape.n), dtype=X.dtype, device="cuda:0")
    ws = fwd_workspace(torch, skm, X, lut, shape.n, shape.d, b, w.gpr)
    rot = Rotation(torch, idx, lut) if rotate else None

    def launch():
        i, l = rot.next() if rot else (idx, lut)
        skm.sketch_matmul_fwd(X, i, l, b, w.gpr, out=Y, workspace=ws)

    total = time_launches(torch, launch, steps, warmup)
    if check:
        skm.sketch_matmul_fwd(X, idx, lut, b, w.gpr, out=Y, workspace=ws)
        CHECKS.append(fwd_check(check, t, Y, b, w.gpr, w.x_dtype, w.lut_dtype, shape.n + m + b))
    xb = wl.DTYPE_BYTES[w.x_dtype]
    lb = wl.DTYPE_BYTES[w.lut_dtype]
    nbytes = wl.algorithmic_bytes_fwd(shape.n, shape.d, b, w.gpr, m, lb, xb)
    flops = wl.flops_pass(shape.n, shape.d, m)
    ms = total / steps
    return {
        "shape": f"{shape.name} {shape.n}x{shape.d}", "b": b, "gpr": w.gpr, "m": m,
        "ms_per_launch": ms, "bytes": nbytes, "flops": flops,
        "GBps": nbytes / (ms * 1e-3) / 1e9, "TFLOPs": flops / (ms * 1e-3) / 1e12,
        "rotation_copies": rot.count if rot else 1,
    }


def bench_multi(torch, skm, steps, warmup):
    """Decode with one table set per token over one shared index stream (b=4):
    one multi-set launch against one single-set launch per set on that set's
    tokens. The 7B attention projection (f16) and the 70B up projection (bf16
    activations with f16 tables: the prescaled pair)."""
    from lut_sketched_matmul_amd import synthetic as syn
    from lut_sketched_matmul_amd import workloads as wl
    b = 4
    out = {}
    cases = [(wl.LLAMA2_7B_ATTN, 0, m, ns, "") for m, ns in ((4, 4), (16, 4), (16, 16))]
    cases += [(wl.LLAMA3_70B_MLP, 0, m, ns, "70b_up_") for m, ns in ((4, 4), (16, 16))]
    for w, si, m, n_sets, tag in cases:
        shape = w.shapes[si]
        t = w.make(shape, b, m)
        X = dev(torch, t["X"], w.x_dtype)
        idx = dev(torch, t["idx_packed"], "u8")
        luts_np = np.stack([syn.random_lut(f"bench-multi/{tag}{m}/{n_sets}/{s}", shape.n, w.gpr, b, w.lut_sigma,
                                           w.lut_dtype) for s in range(n_sets)])
        luts = dev(torch, luts_np, w.lut_dtype)
        sets = [tt % n_sets for tt in range(m)]
        lut_set = torch.tensor(sets, dtype=torch.int32, device="cuda:0")
        Y = torch.empty((m, shape.n), dtype=X.dtype, device="cuda:0")
        rot = Rotation(torch, idx, luts)
        total = time_launches(torch, lambda: skm.sketch_matmul_fwd_multi(X, *rot.next(), lut_set, b, w.gpr, out=Y),
                              steps, warmup)
        # parity sample: every token on sampled rows (the rotated copies hold the same values)
        rows = sample_ids(shape.n, 224, 70 + m + n_sets)
        CHECKS.append({"name": f"decode_multi_lut.{tag}m{m}_sets{n_sets}", "kind": "fwdmulti", "X": t["X"],
                       "idx": t["idx_packed"][rows], "lut": luts_np[:, rows], "sets": sets, "b": b, "gpr": w.gpr,
                       "x_dtype": w.x_dtype, "lut_dtype": w.lut_dtype,
                       "got": Y.float().cpu().numpy()[:, rows].astype(np.float64)})
        # one single-set launch per set, on that set's tokens
        Xs = [X[[tt for tt in range(m) if sets[tt] == s]].contiguous() for s in range(n_sets)]
        Ys = [torch.empty((x.shape[0], shape.n), dtype=X.dtype, device="cuda:0") for x in Xs]

        def per_set():
            i, l = rot.next()
            for s in range(n_sets):
                skm.sketch_matmul_fwd(Xs[s], i, l[s], b, w.gpr, out=Ys[s])

        total_sep = time_launches(torch, per_set, steps, warmup, launches_per_step=n_sets)
        nbytes = (shape.n * shape.d * b // 8 + n_sets * shape.n * w.gpr * (1 << b) * 2 + m * shape.d * 2
                  + m * shape.n * 2)
        ms, ms_sep = total / steps, total_sep / steps
        out[f"{tag}m{m}_sets{n_sets}"] = {
            "shape": f"{shape.name} {shape.n}x{shape.d}", "b": b, "m": m, "n_sets": n_sets,
            "ms_per_launch": ms, "bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_one_launch_per_set": ms_sep, "speedup_vs_one_launch_per_set": ms_sep / ms,
            "rotation_copies": rot.count,
        }
    return out


def bench_glue(torch, skm, steps, warmup):
    """Fine-tuning glue: the fused table optimizer steps over a 7B decoder layer's tables, and the
    q/k/v decode as one grouped launch against three launches."""
    from lut_sketched_matmul_amd import synthetic as syn
    from lut_sketched_matmul_amd import workloads as wl
    out = {}
    wf = wl.LLAMA2_7B_FINETUNE
    count = sum(s.n for s in wf.shapes) * wf.gpr * 16
    per_set = count * (4 * 4 + 2)
    sets = max(2, -(-ROTATE_BYTES // per_set))
    g0 = torch.from_numpy(syn.random_normal("bench-glue/grad", (count,), 1e-3, "f32")).to("cuda:0")
    p0 = torch.from_numpy(syn.random_normal("bench-glue/master", (count,), 0.02, "f32")).to("cuda:0")
    bufs = [dict(p=p0.clone(), g=g0.clone(), m=torch.zeros_like(p0), v=torch.zeros_like(p0),
                 c=torch.empty(count, dtype=torch.float16, device="cuda:0")) for _ in range(sets)]
    it = [0]

    def adam():
        b_ = bufs[it[0] % sets]
        it[0] += 1
        skm.sketch_lut_adam_step(b_["p"], b_["g"], b_["m"], b_["v"], 1 + it[0] // sets, 1e-5, lut=b_["c"])

    def sgd():
        b_ = bufs[it[0] % sets]
        it[0] += 1
        skm.sketch_lut_sgd_step(b_["p"], b_["g"], 1e-5, lut=b_["c"])

    for name, fn, bpe in (("adam", adam, 30), ("sgd", sgd, 14)):
        ms = time_launches(torch, fn, steps, warmup) / steps
        gbs = count * bpe / (ms * 1e-3) / 1e9
        out[f"optimizer_{name}_7b_layer_tables"] = {
            "entries": count, "bytes_per_entry": bpe, "ms_per_step": ms, "GBps": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "rotation_copies": sets}
    del bufs
    # q, k, v of the 7B attention at m = 1: three launches against one over the 12288 stacked rows
    w = wl.LLAMA2_7B_ATTN
    shape = w.shapes[0]
    t = w.make(shape, 4, 1)
    X = dev(torch, t["X"], w.x_dtype)
    idx = dev(torch, t["idx_packed"], "u8")
    lut = dev(torch, t["lut"], w.lut_dtype)
    idx3, lut3 = torch.cat([idx] * 3, 0), torch.cat([lut] * 3, 0)
    rot1, rot3 = Rotation(torch, idx, lut), Rotation(torch, idx3, lut3)
    Y1 = torch.empty((1, shape.n), dtype=X.dtype, device="cuda:0")
    Y3 = torch.empty((1, 3 * shape.n), dtype=X.dtype, device="cuda:0")

    def three():
        for _ in range(3):
            i, l = rot1.next()
            skm.sketch_matmul_fwd(X, i, l, 4, w.gpr, out=Y1)

    def grouped():
        i, l = rot3.next()
        skm.sketch_matmul_fwd(X, i, l, 4, w.gpr, out=Y3)

    ms3 = time_launches(torch, three, steps, warmup, launches_per_step=3) / steps
    msg = time_launches(torch, grouped, steps, warmup) / steps
    nbytes = 3 * wl.algorithmic_bytes_fwd(shape.n, shape.d, 4, w.gpr, 1, 2, 2)
    out["decode_qkv_7b_m1"] = {"ms_three_launches": ms3, "ms_grouped": msg, "speedup": ms3 / msg,
                               "GBps_grouped": nbytes / (msg * 1e-3) / 1e9, "bytes": nbytes}
    return out


def bench_finetune(torch, skm, steps, warmup):
    """One fine-tuning step of a 7B decoder layer: forward, dX and dLUT of all seven projections, then the
    fused Adam step on their fp32 master tables (which also writes the f16 copies the kernels read)."""
    from lut_sketched_matmul_amd import workloads as wl
    w = wl.LLAMA2_7B_FINETUNE
    m = w.tokens[0]
    projs = []
    for s in w.shapes:
        t = w.make(s, 4, m)
        projs.append(dict(
            s=s, X=dev(torch, t["X"], w.x_dtype), dY=dev(torch, t["dY"], w.x_dtype),
            idx=dev(torch, t["idx_packed"], "u8"), lut=dev(torch, t["lut"], w.lut_dtype),
            Y=torch.empty((m, s.n), dtype=torch.bfloat16, device="cuda:0"),
            dL=torch.empty((s.n, w.gpr, 16), dtype=torch.float32, device="cuda:0")))
        p = projs[-1]
        p["wsf"] = fwd_workspace(torch, skm, p["X"], p["lut"], s.n, s.d, 4, w.gpr)
        p["wsb"] = bwd_workspace(torch, skm, p["dY"], p["lut"], s.n, s.d, 4, w.gpr)
        if s.name == "gate":
            p["host"] = {k: t[k] for k in ("X", "dY", "idx_packed", "lut")}
        # fp32 master tables and Adam moments; the step refreshes the f16 copy the kernels read
        p["master"] = p["lut"].float()
        p["m1"], p["m2"] = torch.zeros_like(p["master"]), torch.zeros_like(p["master"])
        del t
    it = [0]

    def step():
        it[0] += 1
        for p in projs:
            skm.sketch_matmul_fwd(p["X"], p["idx"], p["lut"], 4, w.gpr, out=p["Y"], workspace=p["wsf"])
            skm.sketch_matmul_bwd(p["dY"], p["X"], p["idx"], p["lut"], 4, w.gpr, dlut_out=p["dL"],
                                  workspace=p["wsb"])
        for p in projs:
            skm.sketch_lut_adam_step(p["master"], p["dL"], p["m1"], p["m2"], it[0], 1e-5, grad_scale=1.0 / m,
                                     lut=p["lut"])

    total = time_launches(torch, step, steps, warmup, launches_per_step=3 * len(projs))
    flops = sum(3 * wl.flops_pass(p["s"].n, p["s"].d, m) for p in projs)
    ms = total / steps
    # per-pass split, timed the same way on the largest projection (gate)
    g = projs[4]
    t_fwd = time_launches(torch, lambda: skm.sketch_matmul_fwd(g["X"], g["idx"], g["lut"], 4, w.gpr, out=g["Y"],
                                                               workspace=g["wsf"]), steps, warmup) / steps
    t_dx = time_launches(torch, lambda: skm.sketch_matmul_bwd(g["dY"], g["X"], g["idx"], g["lut"], 4, w.gpr,
                                                               need_dlut=False, workspace=g["wsb"]),
                         steps, warmup) / steps
    t_dl = time_launches(torch, lambda: skm.sketch_matmul_bwd(g["dY"], g["X"], g["idx"], g["lut"], 4, w.gpr,
                                                               need_dx=False, dlut_out=g["dL"], workspace=g["wsb"]),
                         steps, warmup) / steps
    fg = wl.flops_pass(g["s"].n, g["s"].d, m)
    # parity samples of the gate projection (forward, dX, dLUT), on its original tables (the timed Adam
    # steps have moved the device copy)
    g["lut"].copy_(dev(torch, g["host"]["lut"], w.lut_dtype))
    skm.sketch_matmul_fwd(g["X"], g["idx"], g["lut"], 4, w.gpr, out=g["Y"], workspace=g["wsf"])
    gdx, _ = skm.sketch_matmul_bwd(g["dY"], g["X"], g["idx"], g["lut"], 4, w.gpr, dlut_out=g["dL"],
                                   workspace=g["wsb"])
    CHECKS.append(fwd_check("finetune_7b_layer.gate.y", g["host"], g["Y"], 4, w.gpr, w.x_dtype, w.lut_dtype, 41))
    CHECKS.extend(bwd_checks("finetune_7b_layer.gate", g["host"], gdx, g["dL"], 4, w.gpr, w.x_dtype, w.lut_dtype, 43))
    return {
        "workload": w.name, "m": m, "ms_per_step": ms, "flops": flops, "TFLOPs": flops / (ms * 1e-3) / 1e12,
        "frac_mfma_peak": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "gate_11008x4096": {"fwd_TFLOPs": fg / (t_fwd * 1e-3) / 1e12, "dx_TFLOPs": fg / (t_dx * 1e-3) / 1e12,
                            "dlut_TFLOPs": fg / (t_dl * 1e-3) / 1e12, "fwd_ms": t_fwd, "dx_ms": t_dx,
                            "dlut_ms": t_dl},
    }


def bench_13b(torch, skm, steps, warmup):
    """LLaMA-2-13B decode at 4-bit indices and one group per row (the decode-efficiency comparison's second
    model): each projection shape at m = 1, and one token through the sketched projections of all 40
    layers (distinct weights per layer; q/k/v and gate/up as grouped launches)."""
    from lut_sketched_matmul_amd import workloads as wl
    w = wl.LLAMA2_13B_DECODE
    out = {}
    for s_ in w.shapes:
        r = bench_fwd(torch, skm, w, s_, 4, 1, steps, warmup)
        r["frac_hbm_peak"] = r["GBps"] / HBM_PEAK_GBS
        out[f"{s_.name}_m1"] = r
    layers = 40
    sh = {s_.name: s_ for s_ in w.shapes}
    t_attn, t_up, t_down = (w.make(sh[k], 4, 1) for k in ("qkvo", "gate_up", "down"))
    X = dev(torch, t_attn["X"], w.x_dtype)
    Xm = torch.empty((1, sh["gate_up"].n), dtype=X.dtype, device="cuda:0")   # input of the down projection
    Xm.copy_(dev(torch, t_down["X"], w.x_dtype))
    base = {
        "qkv": (dev(torch, t_attn["idx_packed"], "u8").repeat(3, 1), dev(torch, t_attn["lut"], w.lut_dtype).repeat(3, 1, 1)),
        "o": (dev(torch, t_attn["idx_packed"], "u8"), dev(torch, t_attn["lut"], w.lut_dtype)),
        "gate_up": (dev(torch, t_up["idx_packed"], "u8").repeat(2, 1), dev(torch, t_up["lut"], w.lut_dtype).repeat(2, 1, 1)),
        "down": (dev(torch, t_down["idx_packed"], "u8"), dev(torch, t_down["lut"], w.lut_dtype)),
    }
    mats = [{k: (i.clone(), l.clone()) for k, (i, l) in base.items()} for _ in range(layers)]
    outs = {k: torch.empty((1, i.shape[0]), dtype=X.dtype, device="cuda:0") for k, (i, _) in base.items()}
    ins = {"qkv": X, "o": X, "gate_up": X, "down": Xm}

    def token():
        for L in mats:
            for k, (i, l) in L.items():
                skm.sketch_matmul_fwd(ins[k], i, l, 4, w.gpr, out=outs[k])

    tok_steps = max(3, steps // 20)
    ms = time_launches(torch, token, tok_steps, max(1, warmup // 10), launches_per_step=4 * layers) / tok_steps
    nbytes = sum(wl.algorithmic_bytes_fwd(i.shape[0], ins[k].shape[1], 4, w.gpr, 1, 2, 2)
                 for k, (i, _) in base.items()) * layers
    out["token_all_40_layers"] = {"launches": 4 * layers, "ms_per_token": ms, "bytes": nbytes,
                                  "GBps": nbytes / (ms * 1e-3) / 1e9,
                                  "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del mats
    return out


def bench_bwd_lowbit(torch, skm, steps, warmup):
    """Forward, dX and dLUT at 2- and 3-bit indices on the 7B gate and down projections (m = 8192)."""
    from lut_sketched_matmul_amd import workloads as wl
    w = wl.LLAMA2_7B_FINETUNE_LOWBIT
    m = w.tokens[0]
    out = {}
    for s_ in w.shapes:
        for b in w.bits:
            t = w.make(s_, b, m)
            X, dY = dev(torch, t["X"], w.x_dtype), dev(torch, t["dY"], w.x_dtype)
            idx, lut = dev(torch, t["idx_packed"], "u8"), dev(torch, t["lut"], w.lut_dtype)
            Y = torch.empty((m, s_.n), dtype=X.dtype, device="cuda:0")
            dL = torch.empty((s_.n, w.gpr, 1 << b), dtype=torch.float32, device="cuda:0")
            wf = fwd_workspace(torch, skm, X, lut, s_.n, s_.d, b, w.gpr)
            wb = bwd_workspace(torch, skm, dY, lut, s_.n, s_.d, b, w.gpr)
            t_fwd = time_launches(torch, lambda: skm.sketch_matmul_fwd(X, idx, lut, b, w.gpr, out=Y, workspace=wf),
                                  steps, warmup) / steps
            t_dx = time_launches(torch, lambda: skm.sketch_matmul_bwd(dY, X, idx, lut, b, w.gpr, need_dlut=False,
                                                                       workspace=wb), steps, warmup) / steps
            t_dl = time_launches(torch, lambda: skm.sketch_matmul_bwd(dY, X, idx, lut, b, w.gpr, need_dx=False,
                                                                       dlut_out=dL, workspace=wb),
                                 steps, warmup) / steps
            if s_.name == "down":
                gdx, _ = skm.sketch_matmul_bwd(dY, X, idx, lut, b, w.gpr, dlut_out=dL, workspace=wb)
                CHECKS.extend(bwd_checks(f"finetune_lowbit_7b_m8192.down_b{b}", t, gdx, dL, b, w.gpr, w.x_dtype,
                                         w.lut_dtype, 50 + b))
            del t
            f = wl.flops_pass(s_.n, s_.d, m)
            out[f"{s_.name}_{s_.n}x{s_.d}_b{b}"] = {
                "fwd_ms": t_fwd, "dx_ms": t_dx, "dlut_ms": t_dl,
                "fwd_TFLOPs": f / (t_fwd * 1e-3) / 1e12, "dx_TFLOPs": f / (t_dx * 1e-3) / 1e12,
                "dlut_TFLOPs": f / (t_dl * 1e-3) / 1e12}
    return out


def bench_bwd_gpr1(torch, skm, steps, warmup):
    """dX and dLUT at one group per row on the 7B q and gate projections (m = 8192): the (128-row block,
    group) grid alone has 32 / 86 blocks, so the table gradient is split over token ranges into the
    workspace and the partial tables are added in range order."""
    from lut_sketched_matmul_amd import workloads as wl
    w = wl.LLAMA2_7B_FINETUNE_GPR1
    m = w.tokens[0]
    out = {}
    for s_ in w.shapes:
        t = w.make(s_, 4, m)
        X, dY = dev(torch, t["X"], w.x_dtype), dev(torch, t["dY"], w.x_dtype)
        idx, lut = dev(torch, t["idx_packed"], "u8"), dev(torch, t["lut"], w.lut_dtype)
        dL = torch.empty((s_.n, 1, 16), dtype=torch.float32, device="cuda:0")
        wb = bwd_workspace(torch, skm, dY, lut, s_.n, s_.d, 4, 1)
        t_dx = time_launches(torch, lambda: skm.sketch_matmul_bwd(dY, X, idx, lut, 4, 1, need_dlut=False,
                                                                   workspace=wb), steps, warmup) / steps
        t_dl = time_launches(torch, lambda: skm.sketch_matmul_bwd(dY, X, idx, lut, 4, 1, need_dx=False,
                                                                   dlut_out=dL, workspace=wb), steps, warmup) / steps
        f = wl.flops_pass(s_.n, s_.d, m)
        rb = (s_.n + 127) // 128
        # the workspace holds the row exponents of dY (bf16 with f16 tables), then one partial table per
        # (column range, token range) of the split
        rexp_bytes = -(-m * 4 // 256) * 256
        ranges = (wb.numel() - rexp_bytes) // (s_.n * 16 * 4)
        out[f"{s_.name}_{s_.n}x{s_.d}_gpr1"] = {
            "dx_ms": t_dx, "dlut_ms": t_dl, "dx_TFLOPs": f / (t_dx * 1e-3) / 1e12,
            "dlut_TFLOPs": f / (t_dl * 1e-3) / 1e12, "dlut_row_blocks": rb, "dlut_partial_tables": int(ranges),
            "dlut_blocks": int(rb * ranges)}
        if s_.name == "q":
            gdx, _ = skm.sketch_matmul_bwd(dY, X, idx, lut, 4, 1, dlut_out=dL, workspace=wb)
            CHECKS.extend(bwd_checks("finetune_7b_gpr1.q", t, gdx, dL, 4, 1, w.x_dtype, w.lut_dtype, 61))
        del t
    return out


def bench_read_reference(torch, steps, warmup):
    """A rotated read-only stream of the headline decode's and the 70B up decode's byte counts per call
    (the vendor reduction torch.sum over fp16 buffers, >= 1 GiB in rotation): the per-call cost of reading
    that many bytes once from HBM, launch and ramp included. Context for the decode rates, not a roof."""
    from lut_sketched_matmul_amd import workloads as wl
    out = {}
    for name, nbytes in (("7b_attn_decode_9.45MB", wl.algorithmic_bytes_fwd(4096, 4096, 4, 8, 1, 2, 2)),
                         ("70b_up_decode_121MB", wl.algorithmic_bytes_fwd(28672, 8192, 4, 4, 1, 2, 2))):
        elems = nbytes // 2
        count = max(2, -(-ROTATE_BYTES // nbytes))
        bufs = [torch.ones(elems, dtype=torch.float16, device="cuda:0") for _ in range(count)]
        it = [0]

        def launch():
            torch.sum(bufs[it[0] % count])
            it[0] += 1

        ms = time_launches(torch, launch, steps, warmup) / steps
        out[name] = {"bytes": int(elems * 2), "ms_per_call": ms, "GBps": elems * 2 / (ms * 1e-3) / 1e9,
                     "rotation_copies": count}
        del bufs
    return out


def bench_construct(torch, skm):
    """Sketching one 4096 x 4096 layer at 4-bit indices and 4 groups per row (the configuration whose
    sketching time the pages report): factor of the damped inverse Hessian from 2048 sample inputs
    (torch.linalg), column weights, 30 weighted Lloyd iterations, the mapping sweep."""
    from lut_sketched_matmul_amd import construct
    from lut_sketched_matmul_amd import synthetic as syn
    n = d = 4096
    b, gpr, iters = 4, 4, 30
    W = torch.from_numpy(syn.random_normal("bench-construct/W", (n, d), 0.02, "f32")).to("cuda:0")
    Xs = torch.from_numpy(syn.random_normal("bench-construct/X", (2048, d), 1.0, "f32")).to("cuda:0")
    Wk = torch.empty_like(W)
    out = {}

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            r = fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps, r

    out["factor_ms"], U = timed(lambda: construct.hessian_factor(Xs))
    out["column_weights_ms"], h = timed(lambda: skm.sketch_column_weights(U))
    out["lloyd_ms"], lut = timed(lambda: skm.sketch_lloyd(W, h, b, gpr, iters, lut_dtype=torch.float16))

    def mapping():
        Wk.copy_(W)
        return skm.sketch_map(Wk, U, lut, b, gpr)

    out["map_ms"], _ = timed(mapping)
    out["total_ms"] = out["factor_ms"] + out["column_weights_ms"] + out["lloyd_ms"] + out["map_ms"]
    # the mapping's arithmetic: n d^2 multiply-adds of the error spreading (fp32)
    out["map_TFLOPs"] = 2.0 * n * d * d / 2 / (out["map_ms"] * 1e-3) / 1e12
    out.update({"n": n, "d": d, "b": b, "gpr": gpr, "lloyd_iters": iters, "samples": 2048})
    return out


def bench_dense_reference(torch, steps, warmup):
    """The vendor dense GEMM (torch.matmul -> hipBLASLt) at the prefill shapes,
    with an already dequantised 16-bit weight: context for the sketched GEMM,
    which does the dequantisation inside the kernel."""
    out = {}
    for name, (m, n, d) in {"70b_up_m2048": (2048, 28672, 8192), "70b_down_m2048": (2048, 8192, 28672),
                            "7b_gate_m8192": (8192, 11008, 4096)}.items():
        a = torch.randn(m, d, device="cuda:0", dtype=torch.float16)
        w = torch.randn(n, d, device="cuda:0", dtype=torch.float16)
        c = torch.empty(m, n, device="cuda:0", dtype=torch.float16)
        total = time_launches(torch, lambda: torch.matmul(a, w.t(), out=c), steps, warmup)
        ms = total / steps
        out[name] = {"ms": ms, "TFLOPs": 2.0 * m * n * d / (ms * 1e-3) / 1e12}
        del a, w, c
    return out


COPY_BYTES = 1 << 30


def bench_copy(torch, steps, warmup):
    """A plain streaming kernel (dst = src + 1, fp32, 1 GiB each way): the
    practical HBM ceiling, and the known-size kernel that scales the FETCH_SIZE
    / WRITE_SIZE counters."""
    n = COPY_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    total = time_launches(torch, lambda: torch.add(src, 1.0, out=dst), steps, warmup)
    ms = total / steps
    return {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES, "ms_per_launch": ms,
            "GBps_read_plus_write": 2 * COPY_BYTES / (ms * 1e-3) / 1e9}


def cpu_baseline(w, shape, b, m, checks, budget_s=12.0):
    """The CPU oracle (float64 numpy) on the same decode workload, and on the backward (dX, dW and the
    binning into dLUT) of one fine-tuning projection; then the parity samples of the parts scored against
    it."""
    import oracle
    from lut_sketched_matmul_amd import synthetic as syn
    from lut_sketched_matmul_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t = w.make(shape, b, m)
    X64 = syn.to_float64(t["X"], w.x_dtype)
    L64 = syn.to_float64(t["lut"], w.lut_dtype)
    times = []
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        oracle.forward(X64, t["idx_packed"], L64, b, w.gpr)
        times.append(time.perf_counter() - t0)
    nbytes = wl.algorithmic_bytes_fwd(shape.n, shape.d, b, w.gpr, m, wl.DTYPE_BYTES[w.lut_dtype],
                                      wl.DTYPE_BYTES[w.x_dtype])
    med = float(np.median(times))
    out = {
        "value": nbytes / med / 1e9, "unit": "GB/s",
        "cores": int(blas_threads), "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{len(times)} oracle forward calls (unpack + float64 dequant + matvec) on the full "
                  f"{shape.n}x{shape.d} b={b} m={m} layer, median {med * 1e3:.1f} ms",
    }
    # backward of the 7B fine-tuning q projection (4096 x 4096, 8192 tokens): dX = dY W, then dW = dY^T X
    # binned into dLUT, in float64; one run (about 2 x 0.27 TFLOP)
    wf = wl.LLAMA2_7B_FINETUNE
    sq = wf.shapes[0]
    tq = wf.make(sq, 4, wf.tokens[0])
    dY64, X64 = syn.to_float64(tq["dY"], wf.x_dtype), syn.to_float64(tq["X"], wf.x_dtype)
    L64 = syn.to_float64(tq["lut"], wf.lut_dtype)
    t0 = time.perf_counter()
    oracle.backward_dx(dY64, tq["idx_packed"], L64, sq.d, 4, wf.gpr)
    oracle.backward_dlut(dY64, X64, tq["idx_packed"], 4, wf.gpr)
    tb = time.perf_counter() - t0
    fb = 2 * wl.flops_pass(sq.n, sq.d, wf.tokens[0])
    out["backward"] = {"value": fb / tb / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
                       "seconds": tb,
                       "sample": f"one oracle backward (dX, dW, binning) of the {sq.n}x{sq.d} b=4 gpr={wf.gpr} "
                                 f"q projection at {wf.tokens[0]} tokens"}
    del tq, dY64, X64
    return out, _score_checks(oracle, syn, checks)


def _score_checks(oracle, syn, checks):
    """max |gpu - oracle| / max |oracle| of each part's parity sample (part of the CPU leg)."""
    errs = {}
    for c in checks:
        L64 = syn.to_float64(c["lut"], c["lut_dtype"]) if "lut" in c else None
        if c["kind"] == "fwd":
            want = oracle.forward(syn.to_float64(c["X"], c["x_dtype"]), c["idx"], L64, c["b"], c["gpr"])
        elif c["kind"] == "fwdmulti":
            want = oracle.forward_multi(syn.to_float64(c["X"], c["x_dtype"]), c["idx"], L64, c["sets"], c["b"],
                                        c["gpr"])
        elif c["kind"] == "dx":
            d = c["idx"].shape[1] * 8 // c["b"]
            W = oracle.dequantize(c["idx"], L64, d, c["b"], c["gpr"])
            want = syn.to_float64(c["dY"], c["x_dtype"]) @ W[:, c["cols"]]
        else:
            want = oracle.backward_dlut(syn.to_float64(c["dY"], c["x_dtype"]), syn.to_float64(c["X"], c["x_dtype"]),
                                        c["idx"], c["b"], c["gpr"])
        errs[c["name"]] = oracle.rel_err(c["got"], want)
    return errs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU runs are not part "
              f"of this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    import lut_sketched_matmul_amd as skm
    from lut_sketched_matmul_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    skm.lib()
    want = set(args.parts.split(",")) if args.parts != "all" else {"decode", "fwd16", "lowbit", "multilut",
                                                                   "decode70b", "prefill", "finetune", "glue",
                                                                   "13b", "bwdlowbit", "bwdgpr1", "construct",
                                                                   "dense", "copy", "readref"}
    w = wl.LLAMA2_7B_ATTN
    shape = w.shapes[0]
    parts = {}
    log = lambda msg: print("# " + msg, file=sys.stderr, flush=True)

    dec = bench_fwd(torch, skm, w, shape, 4, 1, args.steps, args.warmup, check="decode_m1")
    parts["decode_m1"] = dec
    log(f"decode 4096x4096 b=4 m=1: {dec['ms_per_launch'] * 1e3:.2f} us/launch, {dec['GBps']:.0f} GB/s")
    if "fwd16" in want:
        f16 = bench_fwd(torch, skm, w, shape, 4, 16, args.steps, args.warmup, check="fwd_m16")
        parts["fwd_m16"] = f16
        log(f"forward 4096x4096 b=4 m=16: {f16['ms_per_launch'] * 1e3:.2f} us/launch, {f16['GBps']:.0f} GB/s")
    if "lowbit" in want:
        # the 7B MLP at 2- and 3-bit indices, 1 / 4 / 16 tokens (decode kernel)
        wlb = wl.LLAMA2_7B_MLP_LOWBIT
        lb = {}
        for s_, b_, m_ in wl.runs(wlb):
            key = f"{s_.name}_b{b_}_m{m_}"
            r = bench_fwd(torch, skm, wlb, s_, b_, m_, args.steps, args.warmup,
                          check=f"decode_lowbit_7b_mlp.{key}")
            r["frac_hbm_peak"] = r["GBps"] / HBM_PEAK_GBS
            lb[key] = r
        parts["decode_lowbit_7b_mlp"] = lb
        log("7B MLP b=2/3 decode: " + ", ".join(f"{k} {v['GBps']:.0f} GB/s" for k, v in lb.items()))
    if "multilut" in want:
        ml = bench_multi(torch, skm, args.steps, args.warmup)
        parts["decode_multi_lut"] = ml
        log("multi-LUT decode (4096x4096 f16; 70b_up: 28672x8192 bf16/f16): " + ", ".join(
            f"{k} {v['ms_per_launch'] * 1e3:.2f} us ({v['speedup_vs_one_launch_per_set']:.2f}x vs one launch per set)"
            for k, v in ml.items()))
    if "decode70b" in want:
        w7 = wl.LLAMA3_70B_MLP
        d7 = {}
        for s_ in w7.shapes:
            r = bench_fwd(torch, skm, w7, s_, 4, 1, max(20, args.steps // 4), max(2, args.warmup // 4),
                          check=f"decode_70b_mlp_m1.{s_.name}")
            r["frac_hbm_peak"] = r["GBps"] / HBM_PEAK_GBS
            d7[s_.name] = r
        parts["decode_70b_mlp_m1"] = d7
        log("70B MLP decode m=1: " + ", ".join(f"{k} {v['ms_per_launch'] * 1e3:.1f} us {v['GBps']:.0f} GB/s"
                                                for k, v in d7.items()))
    big_steps = max(2, min(args.steps, 10))
    big_warm = max(1, min(args.warmup, 2))
    if "prefill" in want:
        w4 = wl.LLAMA3_70B_MLP
        for s4 in w4.shapes:
            r = bench_fwd(torch, skm, w4, s4, 4, 2048, big_steps, big_warm, rotate=False,
                          check=f"prefill_70b_{s4.name}_m2048")
            r["frac_mfma_peak"] = r["TFLOPs"] / MFMA_F16_PEAK_TFLOPS
            parts[f"prefill_70b_{s4.name}_m2048"] = r
            log(f"prefill 70B {s4.name} m=2048: {r['ms_per_launch']:.3f} ms, {r['TFLOPs']:.0f} TFLOP/s")
    if "finetune" in want:
        ft = bench_finetune(torch, skm, big_steps, big_warm)
        parts["finetune_7b_layer"] = ft
        log(f"fine-tune step 7B layer m=8192: {ft['ms_per_step']:.2f} ms, {ft['TFLOPs']:.0f} TFLOP/s")
    if "13b" in want:
        r13 = bench_13b(torch, skm, args.steps, args.warmup)
        parts["decode_13b_gpr1"] = r13
        tk = r13["token_all_40_layers"]
        log("13B decode gpr=1 m=1: " + ", ".join(f"{k} {v['ms_per_launch'] * 1e3:.1f} us {v['GBps']:.0f} GB/s"
                                                 for k, v in r13.items() if k != "token_all_40_layers")
            + f"; one token through 40 layers: {tk['ms_per_token']:.3f} ms, {tk['GBps']:.0f} GB/s")
    if "bwdlowbit" in want:
        rb = bench_bwd_lowbit(torch, skm, big_steps, big_warm)
        parts["finetune_lowbit_7b_m8192"] = rb
        log("7B b=2/3 m=8192 fwd/dX/dLUT TFLOP/s: " + ", ".join(
            f"{k} {v['fwd_TFLOPs']:.0f}/{v['dx_TFLOPs']:.0f}/{v['dlut_TFLOPs']:.0f}" for k, v in rb.items()))
    if "bwdgpr1" in want:
        rg = bench_bwd_gpr1(torch, skm, big_steps, big_warm)
        parts["finetune_7b_gpr1_m8192"] = rg
        log("7B gpr=1 m=8192 dX/dLUT TFLOP/s: " + ", ".join(
            f"{k} {v['dx_TFLOPs']:.0f}/{v['dlut_TFLOPs']:.0f} ({v['dlut_blocks']} dLUT blocks)" for k, v in rg.items()))
    if "readref" in want:
        rr = bench_read_reference(torch, max(20, args.steps // 2), max(2, args.warmup // 2))
        rr["decode_m1_over_read_ref"] = dec["ms_per_launch"] / rr["7b_attn_decode_9.45MB"]["ms_per_call"]
        parts["read_reference_torch_sum"] = rr
        log("read-only reference (torch.sum, rotated): " + ", ".join(
            f"{k} {v['ms_per_call'] * 1e3:.2f} us {v['GBps']:.0f} GB/s" for k, v in rr.items() if isinstance(v, dict)))
    if "construct" in want:
        cs = bench_construct(torch, skm)
        parts["sketch_construction_4096x4096_b4_gpr4"] = cs
        log(f"sketch construction 4096x4096 b=4 gpr=4: factor {cs['factor_ms']:.1f} ms, column weights "
            f"{cs['column_weights_ms']:.2f} ms, Lloyd {cs['lloyd_ms']:.2f} ms, mapping {cs['map_ms']:.2f} ms, "
            f"total {cs['total_ms']:.1f} ms")
    if "glue" in want:
        gl = bench_glue(torch, skm, args.steps, args.warmup)
        parts["finetune_glue"] = gl
        q = gl["decode_qkv_7b_m1"]
        log("optimizer steps over a 7B layer's tables: " + ", ".join(
            f"{k} {v['ms_per_step'] * 1e3:.1f} us {v['GBps']:.0f} GB/s" for k, v in gl.items() if "optimizer" in k)
            + f"; q/k/v decode m=1: three launches {q['ms_three_launches'] * 1e3:.2f} us, grouped "
              f"{q['ms_grouped'] * 1e3:.2f} us")

    if "dense" in want:
        dr = bench_dense_reference(torch, big_steps, big_warm)
        parts["dense_f16_gemm_reference"] = dr
        log("dense f16 GEMM reference: " + ", ".join(f"{k} {v['TFLOPs']:.0f} TFLOP/s" for k, v in dr.items()))
    if "copy" in want:
        cp = bench_copy(torch, big_steps, big_warm)
        parts["copy_1GiB"] = cp
        log(f"device copy 1 GiB: {cp['ms_per_launch']:.3f} ms, {cp['GBps_read_plus_write']:.0f} GB/s read+write")

    cpu = None
    if not args.no_cpu:
        cpu, errs = cpu_baseline(w, shape, 4, 1, CHECKS)
        parts["parity_err"] = errs
        log("parity (max|gpu - oracle| / max|oracle| on sampled outputs): " + ", ".join(
            f"{k} {v:.2e}" for k, v in errs.items()))
    value = dec["GBps"]
    from lut_sketched_matmul_amd import profiling
    # measured HBM bytes per launch (scaled counters); None once the kernel sources changed
    traffic = profiling.measured_bytes(DECODE_PROFILE, "k_decode<4,")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_launch"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama2-7b-attn-4096x4096 decode GEMV", "n": 4096, "d": 4096, "b": 4, "gpr": 8,
                   "m": 1, "x_dtype": "f16", "lut_dtype": "f16"},
        "roofline": {
            "bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "parts": parts,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
