"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an object ``o`` exposing the oracle API (the real oracle
module, or a copy with a planted mistake) and raises ``AssertionError`` when
``o`` disagrees with the fact it checks. The facts are:

* hand-worked bitstreams (``tests/golden/bitstream_*.txt``) and an
  independent big-integer field extractor for the index layout;
* the identity example of SpaLLM section 2.4 (``tests/golden/identity_two_values.txt``);
* a dense special case (group width == k and idx[i, j] = j mod k), where the
  sketch reproduces an arbitrary matrix and the forward pass must equal the
  textbook product ``X @ W.T`` and each table entry's gradient must equal the
  single virtual parameter's gradient;
* a second formulation of the forward pass (bin the inputs, then multiply by
  the table: sum_{g,c} LUT[i,g,c] * sum_{j in g, idx=c} x_j);
* central finite differences of L = <dY, Y(X, LUT)> (exact up to rounding,
  since Y is linear in X and in LUT);
* invariants: bins partition a group (sum over c of dLUT equals the group's sum
  of dW), adjointness <dY, X W^T> = <dY W, X>, entry-permutation invariance;
* exact integer histograms for selection inputs;
* several table sets over one mapping (SpaLLM section 2.3, multiple
  adapters): the identity mapping with per-set values 1, 2, -1 scales each
  token by its set's value; per-set dense cases give the textbook product with
  the token's own matrix; a token's output ignores the sets it does not use;
* the table optimizer steps: torch.optim.AdamW and torch.optim.SGD (float64
  on the CPU, an independent implementation of the same textbook rules) over
  several steps; Adam's closed form under a constant gradient (bias correction
  makes every step move by lr * g / (|g| + eps)); Adam's invariance when the
  gradient and eps are scaled together;
* sketch construction: scikit-learn's KMeans (Lloyd, with sample weights and
  the same starting centroids) for the weighted Lloyd step; hand-worked
  groups (the starting centroids, a weighted two-cluster case, an empty
  cluster); the objective never increasing; the factor of the damped inverse
  Hessian checked by multiplication; the column weights against the
  diagonal of an explicitly inverted Hessian; the mapping with U = I (plain
  nearest rounding), with tables that hold every weight exactly, and against
  the closed-form optimal compensation (the free weights that minimise the
  quadratic loss given the columns already mapped, solved from H directly);
* the parity score, max |got - ref| / max |ref| (the stated acceptance
  measure: largest absolute error over the largest absolute reference value):
  hand-worked arrays whose largest error is negative and whose largest
  reference value is negative, the vector infinity norm of numpy.linalg as a
  second definition, scale invariance, an all-zero reference, empty arrays
  and a shape mismatch.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def _ints(s):
    return [int(t, 0) for t in s.split()]


def _rng(seed):
    return np.random.default_rng(seed)


def _bigint_fields(row_bytes, d, b):
    """Independent extractor: read the row as one little-endian integer."""
    s = 0
    for q, byte in enumerate(row_bytes):
        s |= int(byte) << (8 * q)
    mask = (1 << b) - 1
    return [(s >> (b * j)) & mask for j in range(d)]


def _random_case(seed, n, d, b, gpr, m):
    r = _rng(seed)
    k = 1 << b
    idx = r.integers(0, k, size=(n, d))
    lut = np.sort(r.normal(0.0, 0.02, size=(n, gpr, k)), axis=-1)
    X = r.normal(size=(m, d))
    dY = r.normal(size=(m, n))
    return idx, lut, X, dY


# ---------------------------------------------------------------------------
# index layout
# ---------------------------------------------------------------------------

def pin_bitstream_golden(o):
    g3 = _read_golden("bitstream_b3_0to7.txt")
    packed = np.array([_ints(g3["bytes"])], dtype=np.uint8)
    want = _ints(g3["indices"])
    assert list(o.unpack_indices(packed, int(g3["d"]), int(g3["b"]))[0]) == want
    assert list(o.pack_indices(np.array([want]), 3)[0]) == _ints(g3["bytes"])
    g = _read_golden("bitstream_b4_b2.txt")
    for b, ik, bk in ((4, "b4_indices", "b4_bytes"), (2, "b2_indices", "b2_bytes")):
        ind, byt = _ints(g[ik]), _ints(g[bk])
        assert list(o.unpack_indices(np.array([byt], dtype=np.uint8), len(ind), b)[0]) == ind
        assert list(o.pack_indices(np.array([ind]), b)[0]) == byt


def pin_unpack_bigint(o):
    r = _rng(1)
    for b in (2, 3, 4):
        for d in (8, 16, 24, 64, 96):
            if (d * b) % 8:
                continue
            packed = r.integers(0, 256, size=(3, d * b // 8), dtype=np.uint8)
            got = o.unpack_indices(packed, d, b)
            for i in range(3):
                assert list(got[i]) == _bigint_fields(packed[i], d, b), (b, d, i)


def pin_unpack_exhaustive_b3(o):
    # every value 0..7 at every field position modulo 8 (fields that straddle bytes)
    d = 64
    for v in range(8):
        for start in range(8):
            idx = np.zeros((1, d), dtype=np.int64)
            idx[0, start::8] = v
            packed = o.pack_indices(idx, 3)
            assert _bigint_fields(packed[0], d, 3) == list(idx[0])
            assert np.array_equal(o.unpack_indices(packed, d, 3), idx)


# ---------------------------------------------------------------------------
# dequantisation
# ---------------------------------------------------------------------------

def pin_identity(o):
    """SpaLLM section 2.4: the identity is exact with two shared values."""
    _read_golden("identity_two_values.txt")
    for b, gpr, n in ((2, 1, 32), (3, 2, 64), (4, 4, 64)):
        k = 1 << b
        lut = np.full((n, gpr, k), 7.25)
        lut[:, :, 0] = 0.0
        lut[:, :, 1] = 1.0
        idx = np.eye(n, dtype=np.int64)
        packed = o.pack_indices(idx, b)
        W = o.dequantize(packed, lut, n, b, gpr)
        assert np.array_equal(W, np.eye(n))
        X = _rng(2).normal(size=(5, n))
        dY = _rng(3).normal(size=(5, n))
        assert np.array_equal(o.forward(X, packed, lut, b, gpr), X)
        assert np.array_equal(o.backward_dx(dY, packed, lut, n, b, gpr), dY)
        dl = o.backward_dlut(dY, X, packed, b, gpr)
        want = np.zeros_like(dl)
        G = n // gpr
        for i in range(n):
            for j in range(n):
                # the diagonal maps to slot 1, every other column to the shared 0 in slot 0
                want[i, j // G, 1 if i == j else 0] += float(np.dot(dY[:, i], X[:, j]))
        assert np.allclose(dl, want, rtol=1e-12, atol=1e-12)


def pin_dense_special_case(o):
    """Group width == k and idx = j mod k: every W is representable."""
    r = _rng(4)
    for b in (2, 3, 4):
        k = 1 << b
        n, gpr, m = 6, 4, 3
        d = gpr * k
        W = r.normal(size=(n, d))
        lut = W.reshape(n, gpr, k).copy()
        idx = np.tile(np.arange(d) % k, (n, 1))
        packed = o.pack_indices(idx, b)
        assert np.array_equal(o.dequantize(packed, lut, d, b, gpr), W)
        X = r.normal(size=(m, d))
        dY = r.normal(size=(m, n))
        assert np.allclose(o.forward(X, packed, lut, b, gpr), X @ W.T, rtol=1e-12, atol=1e-12)
        assert np.allclose(o.backward_dx(dY, packed, lut, d, b, gpr), dY @ W, rtol=1e-12, atol=1e-12)
        dW = dY.T @ X
        assert np.allclose(o.backward_dlut(dY, X, packed, b, gpr), dW.reshape(n, gpr, k), rtol=1e-12, atol=1e-12)
        assert np.allclose(o.backward_dlut_loop(dY, X, packed, b, gpr), dW.reshape(n, gpr, k),
                           rtol=1e-12, atol=1e-12)


def pin_dequant_elementwise(o):
    """Direct element-by-element read of the definition on a tiny case."""
    b, gpr, n, d = 3, 2, 3, 16
    idx, lut, _, _ = _random_case(5, n, d, b, gpr, 1)
    W = o.dequantize(o.pack_indices(idx, b), lut, d, b, gpr)
    G = d // gpr
    for i in range(n):
        for j in range(d):
            assert W[i, j] == lut[i, j // G, idx[i, j]]


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def pin_forward_binned(o):
    """Bin the inputs first, then multiply by the table entries."""
    for b, gpr in ((2, 1), (3, 2), (4, 4)):
        n, d, m = 5, 32, 3
        k = 1 << b
        idx, lut, X, _ = _random_case(6 + b, n, d, b, gpr, m)
        G = d // gpr
        want = np.zeros((m, n))
        for t in range(m):
            for i in range(n):
                S = np.zeros((gpr, k))
                for j in range(d):
                    S[j // G, idx[i, j]] += X[t, j]
                want[t, i] = float(np.sum(lut[i] * S))
        got = o.forward(X, o.pack_indices(idx, b), lut, b, gpr)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def pin_permutation_invariance(o):
    b, gpr, n, d, m = 4, 2, 4, 32, 2
    k = 1 << b
    idx, lut, X, _ = _random_case(9, n, d, b, gpr, m)
    perm = _rng(10).permutation(k)
    inv = np.argsort(perm)
    lut_p = lut[:, :, perm]             # new slot s holds old entry perm[s]
    idx_p = inv[idx]                    # old entry c now lives at slot inv[c]
    y0 = o.forward(X, o.pack_indices(idx, b), lut, b, gpr)
    y1 = o.forward(X, o.pack_indices(idx_p, b), lut_p, b, gpr)
    assert np.allclose(y0, y1, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(o, X, packed, lut, dY, b, gpr):
    return float(np.sum(dY * o.forward(X, packed, lut, b, gpr)))


def pin_finite_difference(o):
    for b, gpr in ((2, 2), (3, 1), (4, 2)):
        n, d, m = 4, 32, 3
        idx, lut, X, dY = _random_case(11 + b, n, d, b, gpr, m)
        packed = o.pack_indices(idx, b)
        h = 0.5  # L is linear in X and in LUT: the central difference is exact
        dX = o.backward_dx(dY, packed, lut, d, b, gpr)
        for (t, j) in ((0, 0), (1, 17), (2, 31), (0, 9)):
            Xp, Xm = X.copy(), X.copy()
            Xp[t, j] += h
            Xm[t, j] -= h
            fd = (_loss(o, Xp, packed, lut, dY, b, gpr) - _loss(o, Xm, packed, lut, dY, b, gpr)) / (2 * h)
            assert abs(fd - dX[t, j]) <= 1e-10 * max(1.0, abs(fd)), (b, t, j, fd, dX[t, j])
        dl = o.backward_dlut(dY, X, packed, b, gpr)
        k = 1 << b
        for (i, g, c) in ((0, 0, 0), (1, gpr - 1, k - 1), (3, 0, k // 2), (2, gpr - 1, 1)):
            Lp, Lm = lut.copy(), lut.copy()
            Lp[i, g, c] += h
            Lm[i, g, c] -= h
            fd = (_loss(o, X, packed, Lp, dY, b, gpr) - _loss(o, X, packed, Lm, dY, b, gpr)) / (2 * h)
            assert abs(fd - dl[i, g, c]) <= 1e-10 * max(1.0, abs(fd)), (b, i, g, c, fd, dl[i, g, c])


def pin_bins_partition_group(o):
    b, gpr, n, d, m = 4, 4, 6, 64, 5
    idx, lut, X, dY = _random_case(20, n, d, b, gpr, m)
    packed = o.pack_indices(idx, b)
    dl = o.backward_dlut(dY, X, packed, b, gpr)
    dW = dY.T @ X
    G = d // gpr
    for i in range(n):
        for g in range(gpr):
            assert np.isclose(dl[i, g].sum(), dW[i, g * G:(g + 1) * G].sum(), rtol=1e-12, atol=1e-12)


def pin_adjoint(o):
    b, gpr, n, d, m = 3, 2, 7, 64, 4
    idx, lut, X, dY = _random_case(21, n, d, b, gpr, m)
    packed = o.pack_indices(idx, b)
    lhs = float(np.sum(dY * o.forward(X, packed, lut, b, gpr)))
    rhs = float(np.sum(o.backward_dx(dY, packed, lut, d, b, gpr) * X))
    assert np.isclose(lhs, rhs, rtol=1e-12, atol=1e-13)


def pin_histogram(o):
    """X = identity (m = d), dY = 1: dLUT counts each (row, group) bin exactly."""
    for b, gpr in ((2, 2), (3, 4), (4, 1)):
        n, d = 5, 32
        k = 1 << b
        idx = _rng(30 + b).integers(0, k, size=(n, d))
        packed = o.pack_indices(idx, b)
        X = np.eye(d)
        dY = np.ones((d, n))
        dl = o.backward_dlut(dY, X, packed, b, gpr)
        G = d // gpr
        for i in range(n):
            for g in range(gpr):
                counts = np.zeros(k)
                for j in range(g * G, (g + 1) * G):
                    counts[idx[i, j]] += 1
                assert np.array_equal(dl[i, g], counts)


def pin_loop_vs_bincount(o):
    b, gpr, n, d, m = 3, 2, 4, 32, 3
    idx, lut, X, dY = _random_case(40, n, d, b, gpr, m)
    packed = o.pack_indices(idx, b)
    assert np.allclose(o.backward_dlut_loop(dY, X, packed, b, gpr),
                       o.backward_dlut(dY, X, packed, b, gpr), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# several table sets over one mapping
# ---------------------------------------------------------------------------

def pin_multi_identity_sets(o):
    """Identity mapping, set 0 = {0, 1}, set 1 = {0, 2}, set 2 = {0, -1}: token
    t's output is X[t] times its set's value."""
    for b, gpr, n in ((2, 1, 32), (4, 2, 64)):
        k = 1 << b
        luts = np.full((3, n, gpr, k), 5.5)
        luts[:, :, :, 0] = 0.0
        luts[0, :, :, 1], luts[1, :, :, 1], luts[2, :, :, 1] = 1.0, 2.0, -1.0
        packed = o.pack_indices(np.eye(n, dtype=np.int64), b)
        X = _rng(11).normal(size=(6, n))
        sets = [0, 2, 1, 1, 0, 2]
        scale = np.array([1.0, -1.0, 2.0, 2.0, 1.0, -1.0])[:, None]
        assert np.array_equal(o.forward_multi(X, packed, luts, sets, b, gpr), X * scale)


def pin_multi_dense(o):
    """Per-set dense special case: Y[t] = W_{s(t)} X[t]."""
    r = _rng(12)
    for b in (2, 3, 4):
        k = 1 << b
        n, gpr, m = 5, 3, 6
        d = gpr * k
        Ws = r.normal(size=(3, n, d))
        luts = Ws.reshape(3, n, gpr, k).copy()
        packed = o.pack_indices(np.tile(np.arange(d) % k, (n, 1)), b)
        X = r.normal(size=(m, d))
        sets = [2, 0, 1, 2, 0, 1]
        Y = o.forward_multi(X, packed, luts, sets, b, gpr)
        for t in range(m):
            assert np.allclose(Y[t], Ws[sets[t]] @ X[t], rtol=1e-12, atol=1e-12), (b, t)


def pin_multi_unused_sets(o):
    """A token's output does not depend on table sets it does not use."""
    b, gpr, n, d, m = 4, 2, 9, 64, 3
    idx, lut, X, _ = _random_case(13, n, d, b, gpr, m)
    packed = o.pack_indices(idx, b)
    luts = np.stack([lut, lut[::-1], lut * 3.0])
    sets = [0, 0, 2]
    Y = o.forward_multi(X, packed, luts, sets, b, gpr)
    luts2 = luts.copy()
    luts2[1] = _rng(14).normal(size=lut.shape)
    assert np.array_equal(o.forward_multi(X, packed, luts2, sets, b, gpr), Y)
    luts2[2] = -luts2[2]
    Y2 = o.forward_multi(X, packed, luts2, sets, b, gpr)
    assert np.array_equal(Y2[:2], Y[:2]) and not np.allclose(Y2[2], Y[2])


def _opt_inputs(seed, count=257):
    rng = np.random.default_rng(seed)
    p0 = rng.normal(0.0, 0.02, count)
    grads = [rng.normal(0.0, 1.0, count) * 10.0 ** rng.uniform(-3, 1, count) for _ in range(6)]
    return p0, grads


def pin_adam_vs_torch(o):
    import torch
    for wd, scale in ((0.0, 1.0), (0.05, 1.0), (0.01, 0.125)):
        p0, grads = _opt_inputs(11)
        prm = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
        opt = torch.optim.AdamW([prm], lr=3e-3, betas=(0.8, 0.95), eps=1e-6, weight_decay=wd, foreach=False)
        p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
        for t, g in enumerate(grads, start=1):
            prm.grad = torch.tensor(g * scale, dtype=torch.float64)
            opt.step()
            p, m, v = o.adam_step(p, g, m, v, t, 3e-3, 0.8, 0.95, 1e-6, wd, scale)
            ref = prm.detach().numpy()
            assert np.allclose(p, ref, rtol=1e-12, atol=1e-15), (wd, scale, t)
            st = opt.state[prm]
            assert np.allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=0)
            assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=0)


def pin_adam_constant_gradient(o):
    # with zero initial moments and a constant gradient the bias-corrected
    # moments are exactly g and g^2, so every step is lr * g / (|g| + eps)
    g = np.array([3.0, -0.5, 1e-3, 0.0, -2e2])
    lr, eps = 1e-2, 1e-4
    p, m, v = np.zeros_like(g), np.zeros_like(g), np.zeros_like(g)
    for t in range(1, 8):
        p, m, v = o.adam_step(p, g, m, v, t, lr, 0.9, 0.999, eps)
        assert np.allclose(p, -t * lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-15), t


def pin_adam_scale_invariance(o):
    # scaling the gradient and eps by s scales both moments' square roots by s
    # and leaves the step unchanged
    p0, grads = _opt_inputs(12, 64)
    s = 1024.0
    a = (p0.copy(), np.zeros_like(p0), np.zeros_like(p0))
    b = (p0.copy(), np.zeros_like(p0), np.zeros_like(p0))
    for t, g in enumerate(grads, start=1):
        a = o.adam_step(*a[:1], g, a[1], a[2], t, 1e-3, 0.9, 0.99, 1e-3)
        b = o.adam_step(*b[:1], g * s, b[1], b[2], t, 1e-3, 0.9, 0.99, 1e-3 * s)
        assert np.allclose(a[0], b[0], rtol=1e-10, atol=1e-15), t


def pin_sgd_vs_torch(o):
    import torch
    for mom, wd, scale in ((0.0, 0.0, 1.0), (0.9, 0.0, 1.0), (0.9, 0.01, 0.5), (0.0, 0.02, 2.0)):
        p0, grads = _opt_inputs(13)
        prm = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
        opt = torch.optim.SGD([prm], lr=0.05, momentum=mom, weight_decay=wd, foreach=False)
        p, buf = p0.copy(), None
        for g in grads:
            prm.grad = torch.tensor(g * scale, dtype=torch.float64)
            opt.step()
            p, buf = o.sgd_step(p, g, 0.05, mom, wd, scale, buf)
            assert np.allclose(p, prm.detach().numpy(), rtol=1e-12, atol=1e-15), (mom, wd)


def _own_init(x, k):
    # written here independently of the oracle: cell midpoints of k equal cells over [min, max]
    lo, hi = float(np.min(x)), float(np.max(x))
    step = (hi - lo) / k
    return np.array([lo + step * (r + 0.5) for r in range(k)])


def pin_lloyd_worked(o):
    # starting centroids: [0, 8] in 4 cells -> 1, 3, 5, 7
    assert np.allclose(o.lloyd_init(np.array([8.0, 0.0, 3.0]), 4), [1.0, 3.0, 5.0, 7.0], rtol=0, atol=1e-12)
    # weighted two clusters: start 3, 9 -> {0, 1} and {10, 12}; weighted means 0.75 and 11
    x4, w4 = np.array([0.0, 1.0, 10.0, 12.0]), np.array([1.0, 3.0, 1.0, 1.0])
    for iters, want in ((0, [3.0, 9.0]), (1, [0.75, 11.0]), (20, [0.75, 11.0])):
        c, _ = o.lloyd_group(x4, w4, 2, iters)
        assert np.allclose(c, want, rtol=0, atol=1e-12), (iters, c)
    # an empty cluster keeps its centroid: start 5/3, 5, 25/3; the middle one gets no value
    c, _ = o.lloyd_group(np.array([0.0, 0.1, 9.9, 10.0]), np.ones(4), 3, 20)
    assert np.allclose(c, [0.05, 5.0, 9.95], rtol=0, atol=1e-12), c


def pin_lloyd_vs_sklearn(o):
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(21)
    for k, G in ((4, 64), (8, 256), (16, 512)):
        for trial in range(3):
            x = rng.standard_normal(G) * 0.02
            wt = np.exp(rng.uniform(-3, 3, G))
            init = _own_init(x, k)
            km = KMeans(n_clusters=k, init=init.reshape(-1, 1), n_init=1, max_iter=300, tol=0.0,
                        algorithm="lloyd").fit(x.reshape(-1, 1), sample_weight=wt)
            if len(np.unique(km.labels_)) < k:
                continue          # scikit-learn moves empty clusters; the pin uses inputs without any
            c, _ = o.lloyd_group(x, wt, k, 300)
            assert np.allclose(np.sort(c), np.sort(km.cluster_centers_.ravel()), rtol=1e-9, atol=1e-12), (k, trial)
            for it in (1, 2, 3):       # the same number of iterations
                km = KMeans(n_clusters=k, init=init.reshape(-1, 1), n_init=1, max_iter=it, tol=0.0,
                            algorithm="lloyd").fit(x.reshape(-1, 1), sample_weight=wt)
                c, _ = o.lloyd_group(x, wt, k, it)
                assert np.allclose(c, km.cluster_centers_.ravel(), rtol=1e-9, atol=1e-12), (k, trial, it)


def pin_lloyd_monotone(o):
    rng = np.random.default_rng(22)
    x, wt = rng.standard_normal(300), np.exp(rng.uniform(-2, 2, 300))
    prev = np.inf
    for it in range(12):
        c, _ = o.lloyd_group(x, wt, 8, it)
        obj = float(np.sum(wt * np.min((x[:, None] - c[None, :]) ** 2, axis=1)))
        assert obj <= prev * (1 + 1e-12), (it, obj, prev)
        prev = obj


def _calib(seed, s, d):
    rng = np.random.default_rng(seed)
    mix = rng.standard_normal((d, d)) / np.sqrt(d) + np.eye(d)
    return rng.standard_normal((s, d)) @ mix          # correlated columns


def pin_hessian_factor(o):
    Xs = _calib(23, 64, 24)
    U = o.hessian_factor(Xs, 0.01)
    H = Xs.T @ Xs
    H = H + 0.01 * np.mean(np.diag(H)) * np.eye(24)
    assert np.allclose(np.tril(U, -1), 0.0)
    assert np.allclose(U.T @ U @ H, np.eye(24), atol=1e-9)
    assert np.allclose(o.column_weights(U), 1.0 / np.diag(np.linalg.inv(H)), rtol=1e-9)


def pin_map_identity_factor(o):
    rng = np.random.default_rng(24)
    n, d, gpr, k = 6, 64, 2, 8
    W = rng.standard_normal((n, d))
    lut = np.sort(rng.standard_normal((n, gpr, k)), axis=2)
    idx = o.map_error_compensated(W, np.eye(d), lut, gpr)
    G = d // gpr
    for i in range(n):
        for j in range(d):
            t = lut[i, j // G]
            assert idx[i, j] == int(np.argmin(np.abs(W[i, j] - t)))


def pin_map_exact_tables(o):
    rng = np.random.default_rng(25)
    n, d, gpr, k = 5, 48, 3, 4
    lut = rng.standard_normal((n, gpr, k))
    want = rng.integers(0, k, (n, d))
    W = lut[np.arange(n)[:, None], (np.arange(d) // (d // gpr))[None, :], want]
    U = o.hessian_factor(_calib(26, 80, d), 0.01)
    assert np.array_equal(o.map_error_compensated(W, U, lut, gpr), want)


def pin_map_closed_form(o):
    """After columns 0..j-1 are fixed at their table values, the compensated weights are the minimisers of
    (w - w0)^T H (w - w0) over the free columns; column j's entry must be the one nearest that optimum."""
    rng = np.random.default_rng(27)
    n, d, gpr, k = 4, 8, 2, 4
    Xs = _calib(28, 40, d)
    U = o.hessian_factor(Xs, 0.01)
    H = np.linalg.inv(U.T @ U)
    W = rng.standard_normal((n, d))
    lut = rng.standard_normal((n, gpr, k))
    idx = o.map_error_compensated(W, U, lut, gpr)
    G = d // gpr
    for i in range(n):
        q = lut[i, np.arange(d) // G, idx[i]]
        for j in range(d):
            Q, F = np.arange(j), np.arange(j, d)
            wf = W[i, F] - np.linalg.solve(H[np.ix_(F, F)], H[np.ix_(F, Q)] @ (q[Q] - W[i, Q]))
            assert idx[i, j] == int(np.argmin(np.abs(wf[0] - lut[i, j // G]))), (i, j)


def pin_rel_err_worked(o):
    # errors 0, -0.5, -1, 0.009 -> largest |error| 1, from a negative error;
    # largest |reference| 4, from a negative reference value; 1 / 4 = 0.25.
    # (The small entry's own relative error is 9: a per-element score differs.)
    got = np.array([[1.0, 2.0], [-5.0, 0.01]])
    ref = np.array([[1.0, 2.5], [-4.0, 0.001]])
    assert o.rel_err(got, ref) == 0.25
    # the score is not symmetric: the reference alone sets the scale (max |got| = 5)
    assert o.rel_err(ref, got) == 1.0 / 5.0
    # an exact result scores 0; a result of all zeros scores 1
    assert o.rel_err(ref.copy(), ref) == 0.0
    assert o.rel_err(np.zeros_like(ref), ref) == 1.0


def pin_rel_err_inf_norm(o):
    rng = _rng(4242)
    for shape in ((7,), (5, 9), (3, 4, 6)):
        ref = rng.standard_normal(shape) * 10.0 ** rng.integers(-3, 3, size=shape)
        got = ref + rng.standard_normal(shape) * 1e-3
        want = np.linalg.norm((got - ref).ravel(), np.inf) / np.linalg.norm(ref.ravel(), np.inf)
        assert abs(o.rel_err(got, ref) - want) <= 1e-15 * want
        # invariant under a common scale of both arguments (powers of two: exact)
        assert o.rel_err(got * 2.0 ** -20, ref * 2.0 ** -20) == o.rel_err(got, ref)


def pin_rel_err_degenerate(o):
    z = np.zeros((3, 2))
    assert o.rel_err(z, z) == 0.0
    assert o.rel_err(z + 1e-30, z) == float("inf")
    assert o.rel_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    try:
        o.rel_err(np.zeros((2, 3)), np.zeros((3, 2)))
    except ValueError:
        pass
    else:
        raise AssertionError("shape mismatch accepted")
    try:
        o.rel_err(np.zeros((1, 3)), np.zeros((3,)))  # broadcastable, still a mismatch
    except ValueError:
        pass
    else:
        raise AssertionError("broadcastable shape mismatch accepted")


ALL_PINS = [
    pin_bitstream_golden, pin_unpack_bigint, pin_unpack_exhaustive_b3,
    pin_identity, pin_dense_special_case, pin_dequant_elementwise,
    pin_forward_binned, pin_permutation_invariance,
    pin_finite_difference, pin_bins_partition_group, pin_adjoint, pin_histogram,
    pin_loop_vs_bincount, pin_multi_identity_sets, pin_multi_dense, pin_multi_unused_sets,
    pin_adam_vs_torch, pin_adam_constant_gradient, pin_adam_scale_invariance, pin_sgd_vs_torch,
    pin_lloyd_worked, pin_lloyd_vs_sklearn, pin_lloyd_monotone, pin_hessian_factor, pin_map_identity_factor,
    pin_map_exact_tables, pin_map_closed_form, pin_rel_err_worked, pin_rel_err_inf_norm, pin_rel_err_degenerate,
]
