"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` takes the oracle module (``oracle.fp64``) and raises
AssertionError on a violation, so the same pins can be run against planted
mutants of the oracle (tests/test_oracle_mutants.py).

The pages (Flash-KMeans paper page, abstract; the Hacker News article,
sections 論文の要点 / Flash-KMeans が変える点) print no worked example and no
numbers for k-means itself, so every pin comes from the mathematics of the
Lloyd iteration: exact rational brute force, closed forms, planted mixtures,
invariants and textbook library routines.
"""

from __future__ import annotations

from fractions import Fraction as F

import numpy as np
import torch

import datagen

# ---------------------------------------------------------------- rounding


_SPECS = {"fp32": (24, -126, 127), "fp16": (11, -14, 15), "bf16": (8, -126, 127)}


def frac_round(q: F, fmt: str) -> F:
    """Exact round-to-nearest-even of a rational into a binary format,
    written independently of the oracle (integer arithmetic on Fractions)."""
    if fmt == "fp64":
        return q
    p, emin, emax = _SPECS[fmt]
    if q == 0:
        return F(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    qe = max(e, emin) - p + 1
    scaled = a / (F(2) ** qe)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * F(2) ** qe
    big = (2 - F(2) ** (1 - p)) * F(2) ** emax
    if r > big:
        raise OverflowError
    return s * r


def pin_rounding(L):
    rng = np.random.default_rng(7)
    # log-uniform magnitudes over the normal and subnormal ranges of each format
    for fmt, lo, hi in (("fp32", -140, 120), ("fp16", -24, 15), ("bf16", -133, 120)):
        x = np.ldexp(rng.uniform(1, 2, 20000), rng.integers(lo, hi, 20000)) * rng.choice([-1, 1], 20000)
        # exact half-way points between neighbours (the tie rule decides them)
        p = _SPECS[fmt][0]
        e = rng.integers(max(lo, -14 if fmt == "fp16" else -126), hi - 1, 4000)
        m = rng.integers(1 << (p - 1), 1 << p, 4000)
        half = np.ldexp(m.astype(np.float64) + 0.5, e - p + 1)
        x = np.concatenate([x, half, -half, [0.0, -0.0]])
        got = L.round_to_format(x, fmt)
        if fmt == "fp32":
            ref = x.astype(np.float32).astype(np.float64)
        elif fmt == "fp16":
            ref = x.astype(np.float16).astype(np.float64)
        else:
            # bf16 reference: torch's float32 -> bfloat16 conversion (round to
            # nearest even) on values that are exact in fp32
            x32 = x.astype(np.float32)
            x = x32.astype(np.float64)
            got = L.round_to_format(x, fmt)
            ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
        assert np.array_equal(got, ref), (fmt, x[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])
    # exact rational rounding of a few awkward fp64 values
    for v in (1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, 255.5, 1.0 / 3.0, -2.0 ** -130, 3.3895e38):
        for fmt in ("bf16", "fp16", "fp32"):
            try:
                want = float(frac_round(F(v), fmt))
            except OverflowError:
                want = float("inf") if v > 0 else float("-inf")
            got = float(L.round_to_format(np.array([v]), fmt)[0])
            assert got == want, (v, fmt, got, want)


def pin_decode(L):
    rng = np.random.default_rng(3)
    v = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 50).to(torch.bfloat16)
    bits = v.view(torch.int16).numpy().view(np.uint16)
    got = L.decode(bits, "bf16")
    assert np.array_equal(got, v.to(torch.float32).numpy().astype(np.float64))
    h = (rng.standard_normal(4096) * 50).astype(np.float16)
    assert np.array_equal(L.decode(h.view(np.uint16), "fp16"), h.astype(np.float64))
    assert np.array_equal(L.decode(h, "fp16"), h.astype(np.float64))


# ------------------------------------------------- exact rational brute force


def bf_lloyd(X, C0, iters, fmt):
    """Lloyd's iteration in exact rational arithmetic (Fractions)."""
    X = [[F(float(v)) for v in row] for row in X]
    C = [[F(float(v)) for v in row] for row in C0]
    K = len(C)
    hist = []
    for _ in range(iters):
        Ch = [[frac_round(c, fmt) for c in row] for row in C]
        labels, J = [], F(0)
        for x in X:
            ds = [sum((a - b) ** 2 for a, b in zip(x, c)) for c in Ch]
            m = min(ds)
            labels.append(ds.index(m))  # first minimum: lowest index wins ties
            J += m
        hist.append(J)
        counts = [0] * K
        sums = [[F(0)] * len(X[0]) for _ in range(K)]
        for x, lab in zip(X, labels):
            counts[lab] += 1
            sums[lab] = [s + a for s, a in zip(sums[lab], x)]
        C = [[s / counts[k] for s in sums[k]] if counts[k] else C[k] for k in range(K)]
    return labels, C, hist, counts


def _dyadic_problem(rng, n, k, d, fmt):
    X = rng.integers(-16, 17, size=(n, d)).astype(np.float64) / 4.0
    C0 = X[rng.choice(n, size=k, replace=False)].copy()
    if k >= 3:
        C0[k - 1] = C0[1]            # duplicate centroid: the higher index must stay empty
    if fmt == "fp32":
        X = X.astype(np.float32).astype(np.float64)
    return X, C0


def pin_bruteforce(L):
    rng = np.random.default_rng(11)
    cases = [("fp64", 1), ("bf16", 4), ("fp16", 4), ("fp32", 3), ("bf16", 1)]
    for ci, (fmt, iters) in enumerate(cases):
        for rep in range(3):
            n = int(rng.integers(8, 64))
            k = int(rng.integers(1, 8))
            d = int(rng.integers(1, 4))
            X, C0 = _dyadic_problem(rng, n, k, d, fmt)
            # plant exact ties: points midway between two distinct centroids
            if k >= 2 and n >= 4:
                X[0] = (C0[0] + C0[1]) / 2
                X[1] = C0[0]
            labels, C, hist, counts = bf_lloyd(X, C0, iters, fmt)
            out = L.lloyd(X, fmt, C0, iters)
            assert np.array_equal(out["labels"], np.array(labels)), (fmt, rep, out["labels"], labels)
            assert np.array_equal(out["counts"], np.array(counts)), (fmt, rep)
            Cx = np.array([[float(v) for v in row] for row in C])
            assert np.allclose(out["C"], Cx, rtol=4e-16, atol=1e-300), (fmt, rep)
            for hj, bj in zip(out["history"], hist):
                assert abs(hj - float(bj)) <= 1e-14 * max(1.0, float(bj)), (fmt, rep, hj, float(bj))


# ------------------------------------------------------------- closed forms


def pin_closed_forms(L):
    rng = np.random.default_rng(5)
    X = rng.standard_normal((500, 6)) * 3 + 1
    # K = 1: the centroid is the column mean and the second inertia is
    # sum ||x||^2 - N ||mean||^2
    C0 = X[:1].copy()
    out = L.lloyd(X, "fp64", C0, 2)
    mean = X.mean(axis=0)
    assert np.allclose(out["C"][0], mean, rtol=1e-13, atol=1e-13)
    J1 = float((X * X).sum() - X.shape[0] * (mean @ mean))
    assert abs(out["history"][1] - J1) <= 1e-10 * J1
    assert abs(out["history"][0] - float(((X - X[0]) ** 2).sum())) <= 1e-12 * out["history"][0]
    # K = N, C0 = X with distinct rows: identity labels and zero inertia
    Xs = X[:40]
    out = L.lloyd(Xs, "fp64", Xs.copy(), 2)
    assert np.array_equal(out["labels"], np.arange(40))
    assert out["inertia"] == 0.0 and np.array_equal(out["C"], Xs)
    # all rows identical and all centroids equal to them: every label is 0,
    # the other clusters are empty and keep their previous value
    Xi = np.tile(np.array([[1.5, -2.0, 0.25]]), (30, 1))
    Ci = np.tile(Xi[:1], (4, 1))
    out = L.lloyd(Xi, "bf16", Ci, 2)
    assert np.array_equal(out["labels"], np.zeros(30)) and list(out["counts"]) == [30, 0, 0, 0]
    assert np.array_equal(out["C"], Ci) and out["inertia"] == 0.0
    # duplicate centroid: the higher index is never chosen and keeps its value
    C2 = X[[3, 7, 7, 9]].copy()
    labels, _ = L.assign(X, C2)
    assert not np.any(labels == 2) and np.any(labels == 1)
    Cn, cnt = L.update(X, labels, C2, 4)
    assert cnt[2] == 0 and np.array_equal(Cn[2], C2[2])
    # D = 1 with sorted centroids: labels are non-decreasing in x
    x1 = np.sort(rng.standard_normal((300, 1)) * 4, axis=0)
    c1 = np.sort(rng.standard_normal((7, 1)) * 4, axis=0)
    lab, _ = L.assign(x1, c1)
    assert np.all(np.diff(lab) >= 0)
    # known nearest centroid in 1-D by hand
    lab, dmin = L.assign(np.array([[0.0], [0.9], [2.0], [-5.0]]), np.array([[-1.0], [1.0], [3.0]]))
    assert list(lab) == [0, 1, 1, 0] and np.allclose(dmin, [1.0, 0.01, 1.0, 16.0])


# -------------------------------------------------------- planted mixtures


def pin_planted(L):
    for fmt, seed in (("bf16", 1), ("fp16", 2), ("fp32", 3)):
        M = 24
        X, _, comp, _ = datagen.mixture(3000, 16, M, dtype=fmt, center_dist="normal", center_scale=40.0,
                                        sigma=1.0, weights=None, workload_code=99, seed=seed)
        X = X[0]
        comp = comp[0]
        if fmt == "bf16":
            Xd = L.decode(X.view(torch.int16).numpy().view(np.uint16), fmt)
        else:
            Xd = L.decode(X.numpy(), fmt)
        rng = np.random.default_rng(seed)
        order = rng.permutation(M)                 # centroid j starts at a point of component order[j]
        first = np.array([np.nonzero(comp == c)[0][0] for c in order])
        C0 = Xd[first]
        out = L.lloyd(Xd, fmt, C0, 1)
        inv = np.empty(M, dtype=np.int64)
        inv[order] = np.arange(M)
        assert np.array_equal(out["labels"], inv[comp]), fmt
        means = np.stack([Xd[comp == c].mean(axis=0) for c in order])
        assert np.allclose(out["C"], means, rtol=1e-14, atol=1e-12), fmt
        out3 = L.lloyd(Xd, fmt, C0, 3)
        assert np.array_equal(out3["labels"], inv[comp]), fmt
        assert np.array_equal(out3["C"], out["C"]), fmt   # exact fixed point


# -------------------------------------------------------------- invariants


def _onehot_sums(X, labels, k):
    import scipy.sparse as sp
    n = X.shape[0]
    M = sp.csr_matrix((np.ones(n), (labels, np.arange(n))), shape=(k, n))
    return np.asarray(M @ X)


def pin_invariants(L):
    rng = np.random.default_rng(9)
    for fmt in ("bf16", "fp16", "fp32", "fp64"):
        Xt, C0t, _, _ = datagen.mixture(1500, 8, 12, dtype="fp32" if fmt == "fp64" else fmt,
                                        center_dist="normal", center_scale=2.0, sigma=1.0, weights=None,
                                        workload_code=98, seed=4, k=12)
        X = Xt[0].to(torch.float32).numpy().astype(np.float64)
        C = C0t[0].numpy().astype(np.float64)
        C[5] = C[4]                    # a duplicate pair forces exact ties / an empty cluster
        k = C.shape[0]
        J_prev = None
        for t in range(6):
            Ch = L.round_to_format(C, fmt)
            labels, dmin = L.assign(X, Ch)
            D2 = L.sq_dist_direct(X, Ch)
            assert np.array_equal(labels, D2.argmin(axis=1)), (fmt, t)        # lowest-index minimiser
            assert np.array_equal(dmin, D2[np.arange(X.shape[0]), labels]), (fmt, t)
            J = L.inertia(dmin)
            assert abs(J - float(np.sort(D2.min(axis=1)).sum())) <= 1e-12 * J
            Cn, cnt = L.update(X, labels, C, k)
            assert cnt.sum() == X.shape[0] and np.array_equal(cnt, np.bincount(labels, minlength=k))
            S = _onehot_sums(X, labels, k)
            nz = cnt > 0
            assert np.allclose(Cn[nz], S[nz] / cnt[nz, None], rtol=1e-13, atol=1e-13), (fmt, t)
            assert np.array_equal(Cn[~nz], C[~nz]), (fmt, t)
            if J_prev is not None:
                # J_t <= J_{t-1} + sum_k n_k ||C_t,k - round(C_t,k)||^2
                assert J <= J_prev + R + 1e-12 * J_prev, (fmt, t, J, J_prev, R)
            R = float((cnt * ((Cn - L.round_to_format(Cn, fmt)) ** 2).sum(axis=1)).sum())
            if fmt == "fp64":
                assert R == 0.0
            J_prev = J
            C = Cn
        # the labels also match the definition on a shuffled copy of the centroids
        perm = rng.permutation(k)
        lab_p, _ = L.assign(X, L.round_to_format(C, fmt)[perm])
        lab, _ = L.assign(X, L.round_to_format(C, fmt))
        d_p = L.sq_dist_direct(X, L.round_to_format(C, fmt)[perm])
        assert np.array_equal(d_p[np.arange(X.shape[0]), lab_p],
                              L.sq_dist_direct(X, L.round_to_format(C, fmt))[np.arange(X.shape[0]), lab])


# --------------------------------------------------------- library routines


def pin_libraries(L):
    from scipy.cluster.vq import vq
    rng = np.random.default_rng(21)
    X = rng.standard_normal((4000, 12)) * 2
    C = rng.standard_normal((37, 12)) * 2
    lab, dmin = L.assign(X, C)
    code, dist = vq(X, C)
    assert np.array_equal(lab, code)
    assert np.allclose(dmin, dist ** 2, rtol=1e-10)
    try:
        from sklearn.cluster import KMeans
    except ImportError:  # pragma: no cover - scikit-learn is in the image
        return
    Xt, C0t, _, _ = datagen.mixture(6000, 10, 16, dtype="fp32", center_dist="normal", center_scale=3.0,
                                    sigma=1.0, weights=None, workload_code=97, seed=8, k=16)
    X = Xt[0].numpy().astype(np.float64)
    C0 = C0t[0].numpy().astype(np.float64)
    out = L.lloyd(X, "fp64", C0, 6)
    assert np.all(out["counts"] > 0)
    km = KMeans(n_clusters=16, init=C0, n_init=1, max_iter=6, tol=0.0, algorithm="lloyd").fit(X)
    assert np.allclose(km.cluster_centers_, out["C"], rtol=1e-10, atol=1e-10)


ALL_PINS = [pin_rounding, pin_decode, pin_bruteforce, pin_closed_forms, pin_planted, pin_invariants,
            pin_libraries]


# ------------------------------------------------------ comparison helpers


def pin_helpers(L):
    """near_tie_report and centroid_rel_err against hand-computed cases."""
    X = np.array([[1.0, 0.0], [0.0, 2.0], [3.0, 3.0]])
    C = np.array([[1.0, 0.0], [1.0 + 1e-7, 0.0], [0.0, 2.0], [5.0, 5.0]])
    # row 0: centroids 0 and 1 are a near-tie (gap 1e-14 << 1e-5 * ||x||^2 = 1e-5)
    # row 1: candidate picks 3 (far): a real failure; row 2: exact
    rep = L.near_tie_report(X, C, np.array([1, 3, 3]), np.array([0, 2, 3]))
    assert rep["mismatch"] == 2 and rep["excused"] == 1 and rep["failed"] == 1 and rep["fail_rows"] == [1]
    rep = L.near_tie_report(X, C, np.array([0, 2, 3]), np.array([0, 2, 3]))
    assert rep["mismatch"] == 0 and rep["failed"] == 0
    # x = 0: the tolerance is zero, so even an exact tie is not excused
    rep = L.near_tie_report(np.zeros((1, 2)), np.array([[1.0, 0.0], [-1.0, 0.0]]), np.array([1]), np.array([0]))
    assert rep["failed"] == 1
    # centroid error: ||(3,4) - (0,0)|| / max(||(0,0)||, 1e-3 * 2000) = 5 / 2
    assert abs(L.centroid_rel_err([[3.0, 4.0], [1.0, 1.0]], [[0.0, 0.0], [1.0, 1.0]], 2000.0) - 2.5) < 1e-15
    assert abs(L.centroid_rel_err([[1.0, 1.0 + 1e-3]], [[1.0, 1.0]], 1.0) - 1e-3 / np.sqrt(2)) < 1e-15


ALL_PINS.append(pin_helpers)


# ------------------------------------------------ top-2 and soft assignment


def _int_problem(rng, n, k, d):
    """Small integer points and centroids with planted duplicate centroids
    (exact distance ties)."""
    X = rng.integers(-3, 4, size=(n, d))
    C = rng.integers(-3, 4, size=(k, d))
    C[k - 1] = C[1]                 # duplicate: exact ties at every point
    return X, C


def pin_top2(L):
    """Two nearest centroids against exact integer brute force (ties to the
    lower index), against the pinned single assignment, and K = 2."""
    rng = np.random.default_rng(21)
    for n, k, d in ((40, 7, 3), (25, 3, 5), (30, 9, 2)):
        X, C = _int_problem(rng, n, k, d)
        lab, dist = L.assign_top2(X.astype(np.float64), C.astype(np.float64))
        for i in range(n):
            pairs = sorted((int(((X[i] - C[j]) ** 2).sum()), j) for j in range(k))
            assert [pairs[0][1], pairs[1][1]] == list(lab[i]), (i, pairs[:3], lab[i])
            assert [pairs[0][0], pairs[1][0]] == list(dist[i])
    # first column = the (separately pinned) nearest-centroid assignment
    p = datagen.make("c2", n=3000, k=40, seed=3)
    Xd = L.decode(p.X[0].numpy(), "fp16")
    Ch = L.round_to_format(p.C0[0].numpy(), "fp16")
    lab, dist = L.assign_top2(Xd, Ch)
    lab1, d1 = L.assign(Xd, Ch)
    assert np.array_equal(lab[:, 0], lab1) and np.array_equal(dist[:, 0], d1)
    assert np.all(dist[:, 0] <= dist[:, 1]) and np.all(lab[:, 0] != lab[:, 1])
    # K = 2: both centroids, nearer first
    lab, _ = L.assign_top2(np.array([[0.0], [3.0], [1.5]]), np.array([[1.0], [2.0]]))
    assert lab.tolist() == [[0, 1], [1, 0], [0, 1]]


def pin_soft(L):
    """Mixture log-density and most responsible component: closed forms, the
    hard limit, invariants."""
    # K = 1: L = log w0 - d / (2 s2), also far away (a sum without the
    # maximum subtracted underflows there)
    for s2, lw0, x in ((0.5, 0.0, [3.0, 4.0]), (3.0, -1.25, [300.0, 400.0]), (1.0, 2.0, [0.0, 0.0])):
        lab, Lx = L.soft_assign(np.array([x]), np.zeros((1, 2)), np.array([lw0]), s2)
        d = x[0] ** 2 + x[1] ** 2
        assert lab[0] == 0 and abs(Lx[0] - (lw0 - d / (2 * s2))) <= 1e-12 * max(1.0, d / s2)
    # K identical centroids: L = log K - d / (2 s2); the lowest index is most responsible
    for K in (2, 5, 64):
        lab, Lx = L.soft_assign(np.array([[1.0, 2.0, 2.0]]), np.tile([[0.0, 0.0, 0.0]], (K, 1)), None, 2.0)
        assert lab[0] == 0 and abs(Lx[0] - (np.log(K) - 9.0 / 4.0)) < 1e-12
    # two centroids symmetric about x
    lab, Lx = L.soft_assign(np.array([[0.0, 0.0]]), np.array([[-1.0, 0.0], [1.0, 0.0]]), None, 0.25)
    assert lab[0] == 0 and abs(Lx[0] - (np.log(2.0) - 2.0)) < 1e-12
    # hard limit: with equal weights the most responsible component is the nearest centroid
    p = datagen.make("c2", n=2000, k=30, seed=5)
    Xd = L.decode(p.X[0].numpy(), "fp16")
    Ch = L.round_to_format(p.C0[0].numpy(), "fp16")
    near, dmin = L.assign(Xd, Ch)
    for s2 in (0.1, 1.0, 50.0):
        lab, Lx = L.soft_assign(Xd, Ch, None, s2)
        assert np.array_equal(lab, near)
        # bounds: the largest term <= L <= the largest term + log K
        top = -dmin / (2 * s2)
        assert np.all(Lx >= top - 1e-9 * np.abs(top)) and np.all(Lx <= top + np.log(30) + 1e-9 * np.abs(top))
    # responsibilities sum to one; a common shift of the log-weights shifts L and keeps the mode
    lw = np.random.default_rng(2).normal(size=30)
    lab, Lx = L.soft_assign(Xd[:200], Ch, lw, 2.0)
    A = lw[None, :] - L.sq_dist_direct(Xd[:200], Ch) / 4.0
    assert np.allclose(np.exp(A - Lx[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.array_equal(lab, A.argmax(axis=1))
    lab2, Lx2 = L.soft_assign(Xd[:200], Ch, lw + 3.5, 2.0)
    assert np.array_equal(lab, lab2) and np.allclose(Lx2, Lx + 3.5, rtol=0, atol=1e-10)


ALL_PINS += [pin_top2, pin_soft]


def pin_gauss(L):
    """Signed-weight Gauss sums: closed forms, cancellation, linearity, the
    wide-kernel limit, and agreement with the pinned soft assignment."""
    # one source: G = w exp(-d / (2 s2))
    for s2, w0, x in ((0.5, 2.5, [3.0, 4.0]), (4.0, -1.5, [1.0, -2.0])):
        G = L.gauss_sum(np.array([x]), np.zeros((1, 2)), np.array([w0]), s2)
        d = x[0] ** 2 + x[1] ** 2
        assert abs(G[0] - w0 * np.exp(-d / (2 * s2))) <= 1e-15 * abs(w0)
    # two identical sources with opposite weights cancel exactly
    G = L.gauss_sum(np.array([[0.3, -0.7], [2.0, 1.0]]), np.array([[1.0, 1.0], [1.0, 1.0]]), np.array([1.75, -1.75]),
                    1.3)
    assert np.all(G == 0.0)
    rng = np.random.default_rng(8)
    X = rng.normal(size=(300, 8))
    Y = rng.normal(size=(40, 8)) * 1.5
    w1, w2 = rng.normal(size=40), rng.normal(size=40)
    # linear in the weights; the order of the sources does not matter
    G1, G2 = L.gauss_sum(X, Y, w1, 2.0), L.gauss_sum(X, Y, w2, 2.0)
    assert np.allclose(L.gauss_sum(X, Y, 3.0 * w1 - 0.5 * w2, 2.0), 3.0 * G1 - 0.5 * G2, rtol=1e-12, atol=1e-12)
    perm = rng.permutation(40)
    assert np.allclose(L.gauss_sum(X, Y[perm], w1[perm], 2.0), G1, rtol=1e-12, atol=1e-14)
    # a very wide kernel sums the weights
    assert np.allclose(L.gauss_sum(X, Y, w1, 1e14), w1.sum(), rtol=1e-9, atol=1e-9)
    # positive weights: log G is the (pinned) mixture log density with log-weights log w
    wp = np.abs(w1) + 0.1
    _, Ls = L.soft_assign(X, Y, np.log(wp), 0.7)
    assert np.allclose(np.log(L.gauss_sum(X, Y, wp, 0.7)), Ls, rtol=0, atol=1e-10)


ALL_PINS.append(pin_gauss)


def pin_seeding(L):
    """k-means++ on hand-computed 1-D cases (including the boundary of the
    inverse CDF), invariants, the degenerate all-identical case, and D^2
    sampling frequencies."""
    X = np.array([[0.0], [1.0], [3.0], [7.0]])          # from row 0: D2 = 0, 1, 9, 49 (cumsum 0, 1, 10, 59)
    for u1, want in ((0.5, 3), (0.01, 1), (10.0 / 59.0 - 1e-12, 2), (10.0 / 59.0 + 1e-12, 3), (0.999, 3)):
        idx, _ = L.kmeanspp(X, [0.0, u1])
        assert idx.tolist() == [0, want], (u1, idx)
    # targets exactly on a cumulative sum (dyadic total): the pick is the next row
    Z = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0], [1.0, 1.0, 1.0], [2.0, 0.0, 0.0]])   # D2 0, 1, 3, 4; cumsum 0, 1, 4, 8
    assert L.kmeanspp(Z, [0.0, 0.5])[0].tolist() == [0, 3]      # target 4 = cumsum[2]
    assert L.kmeanspp(Z, [0.0, 0.125])[0].tolist() == [0, 2]    # target 1 = cumsum[1]
    assert L.kmeanspp(Z, [0.0, 0.0])[0].tolist() == [0, 1]      # target 0: the first row with D2 > 0
    # third pick after rows 0 and 3: D2 = 0, 1, 9, 0 (cumsum 0, 1, 10, 10)
    idx, d2 = L.kmeanspp(X, [0.0, 0.5, 0.05])
    assert idx.tolist() == [0, 3, 1] and d2.tolist() == [0.0, 0.0, 4.0, 0.0]
    idx, _ = L.kmeanspp(X, [0.0, 0.5, 0.5])
    assert idx.tolist() == [0, 3, 2]
    # first pick and random seeding: floor(u n)
    assert L.kmeanspp(X, [0.74])[0].tolist() == [2]
    assert L.seed_random(4, [0.0, 0.2499, 0.25, 0.999]).tolist() == [0, 0, 1, 3]
    # all rows identical: D2 sums to 0, fall back to floor(u n)
    idx, d2 = L.kmeanspp(np.ones((5, 3)), [0.1, 0.9, 0.3])
    assert idx.tolist() == [0, 4, 1] and np.all(d2 == 0)
    # no row with D2 = 0 is picked while the total is positive; final D2 is the distance to the nearest pick
    p = datagen.make("c2", n=1500, k=20, seed=9)
    Xd = L.decode(p.X[0].numpy(), "fp16")
    u = np.random.default_rng(4).random(20)
    idx, d2 = L.kmeanspp(Xd, u)
    assert len(set(idx.tolist())) == 20
    assert np.allclose(d2, L.sq_dist_direct(Xd, Xd[idx]).min(axis=1), rtol=1e-12, atol=0)
    # D^2 sampling: second-pick frequencies follow D2 / sum(D2)
    Y = np.array([[0.0], [1.0], [2.0], [4.0]])         # D2 from row 0: 0, 1, 4, 16
    us = (np.arange(4000) + 0.5) / 4000
    counts = np.bincount([L.kmeanspp(Y, [0.0, v])[0][1] for v in us], minlength=4)
    assert counts.tolist() == [0, 190, 762, 3048]      # midpoints (k + 0.5) / 4000 below 1/21, 5/21, 1


ALL_PINS.append(pin_seeding)
