"""fp64 reference Lloyd iteration (test infrastructure only; see package docstring).

Sources, cited by page title and section:

* [FK] "Flash-KMeans: Fast and Memory-Efficient Exact K-Means" (paper page),
  abstract: k-means runs as an assignment stage followed by a centroid
  update stage; FlashAssign picks each point's nearest centroid, and the
  sort-inverse update reduces the points of each cluster; the result is
  exact k-means.
* [HN] "Hacker Newsが捉えたFlash-KMeans、Exact K-MeansをGPUのonline primitiveへ"
  (article), sections 論文の要点 and Flash-KMeans が変える点: the formulas of
  k-means are unchanged, the method is not an approximation, and the target is
  the classic inner loop (not seeding).
* [GMM] "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering"
  (paper page), abstract: Gaussian-mixture soft clustering computed in one
  pass without materialising the responsibility matrix, and border vectors
  assigned to more than one cluster.
* [GS] "Fast Gauss Sums via Flash Attention" (paper page), abstract: Gauss
  kernel sums with arbitrary signed weights; and the FlashDiffusion card on
  the same listing, abstract: dense Gaussian kernel blocks evaluated in
  fused tiles without the N x N matrix.

Readings taken where the pages are silent (each is also listed in the design
notes):

* distance is squared Euclidean;
* assignment uses centroids rounded to nearest-even into the storage dtype of
  X (``fmt``), with the squared norm taken from the rounded values; the
  centroid state itself is kept unrounded;
* ties go to the lowest centroid index;
* an empty cluster keeps its previous (unrounded) centroid;
* ``lloyd`` runs exactly ``iters`` iterations and returns the labels and
  inertia of the last assignment and the centroids after the last update;
* inertia is the sum over points of the squared distance to the rounded
  centroid the point was assigned to.
"""

from __future__ import annotations

import math

import numpy as np

# (precision p incl. the implicit bit, minimum normal exponent, maximum exponent)
FORMATS = {
    "fp32": (24, -126, 127),
    "fp16": (11, -14, 15),
    "bf16": (8, -126, 127),
    "fp64": None,  # no rounding (used by the pins only)
}


def round_to_format(x, fmt: str) -> np.ndarray:
    """Round fp64 values to the nearest value of a binary floating-point
    format, ties to even, with gradual underflow and overflow to +-inf.

    Written from the definition of the formats: a normal value with exponent
    E has spacing 2**(E-p+1); below the smallest normal exponent the spacing
    stays at 2**(Emin-p+1).  Dividing by the spacing (a power of two, exact)
    leaves an integer-valued quantity that ``np.rint`` rounds half-to-even.
    Returns fp64 values exactly representable in ``fmt``.
    """
    x = np.asarray(x, dtype=np.float64)
    spec = FORMATS[fmt]
    if spec is None:
        return x.copy()
    p, emin, emax = spec
    _, e = np.frexp(x)                      # x = f * 2**e, f in [0.5, 1)
    q = np.maximum(e - 1, emin) - p + 1     # exponent of the spacing
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    r = np.where(np.abs(r) > big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def decode(a, fmt: str) -> np.ndarray:
    """Exact fp64 values of stored inputs.

    ``bf16`` takes the raw uint16 bit patterns (the top half of an IEEE
    binary32), ``fp16`` takes numpy float16 (or its uint16 bits) and ``fp32``
    numpy float32.
    """
    a = np.asarray(a)
    if fmt == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 input must be given as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if fmt == "fp16":
        if a.dtype == np.uint16:
            a = a.view(np.float16)
        return a.astype(np.float64)
    if fmt in ("fp32", "fp64"):
        return a.astype(np.float64)
    raise ValueError(fmt)


def sq_dist_direct(X, C) -> np.ndarray:
    """All squared Euclidean distances sum_d (x_d - c_d)**2 in fp64 by the
    definition (no expansion).  Small inputs only: O(n*k*d) memory per row
    block.  [FK] abstract (distance computation of the assignment stage)."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    out = np.empty((X.shape[0], C.shape[0]))
    rows = max(1, (1 << 22) // max(1, C.shape[0] * C.shape[1]))
    for r0 in range(0, X.shape[0], rows):
        diff = X[r0:r0 + rows, None, :] - C[None, :, :]
        out[r0:r0 + rows] = (diff * diff).sum(axis=2)
    return out


def _rowwise_sq_dist(X, C):
    diff = X - C
    return (diff * diff).sum(axis=1)


def assign(X, Chat, *, block_elems: int = 1 << 24):
    """Assignment stage: label_i = lowest k minimising sum_d (x_id - chat_kd)**2.

    [FK] abstract (assignment stage; FlashAssign's argmin over centroids) and
    [HN] Flash-KMeans が変える点 (nearest centroid per point).

    The value compared is the direct fp64 sum of squared differences.  To
    keep the cost at BLAS speed, a screen first evaluates the same quantity
    through ||x||^2 - 2 x.c + ||c||^2 and discards centroids that are provably
    not minimal: both forms lie within ~(d+3)*2**-53*(||x||^2+||c||^2) of the
    exact value, so every direct-form minimiser lies within
    1e-10*(||x||^2 + max||c||^2) of the screened minimum.  Rows with several
    surviving candidates are decided by the direct form, ties to the lowest
    index.  Returns (labels int64 [n], dmin fp64 [n]) where dmin is the direct
    squared distance to the chosen centroid.
    """
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    n, _ = X.shape
    k = Chat.shape[0]
    xx = np.einsum("ij,ij->i", X, X)
    cc = np.einsum("ij,ij->i", Chat, Chat)
    ccmax = float(cc.max()) if k else 0.0
    labels = np.empty(n, dtype=np.int64)
    rows = max(1, block_elems // max(1, k))
    for r0 in range(0, n, rows):
        Xb = X[r0:r0 + rows]
        dexp = Xb @ Chat.T
        dexp *= -2.0
        dexp += xx[r0:r0 + rows, None]
        dexp += cc[None, :]
        m = dexp.min(axis=1)
        margin = 1e-10 * (xx[r0:r0 + rows] + ccmax) + 1e-300
        cand = dexp <= (m + margin)[:, None]
        lab = cand.argmax(axis=1)          # lowest surviving index
        multi = np.nonzero(cand.sum(axis=1) > 1)[0]
        if multi.size:
            ri, ki = np.nonzero(cand[multi])
            dd = _rowwise_sq_dist(Xb[multi[ri]], Chat[ki])
            order = np.lexsort((ki, dd, ri))   # by row, then distance, then index
            ri_s = ri[order]
            first = np.ones(ri_s.size, dtype=bool)
            first[1:] = ri_s[1:] != ri_s[:-1]
            lab[multi[ri_s[first]]] = ki[order][first]
        labels[r0:r0 + rows] = lab
    dmin = _rowwise_sq_dist(X, Chat[labels])
    return labels, dmin


def assign_top2(X, Chat):
    """Each point's two nearest centroids: the two smallest pairs (d_ik, k) in
    lexicographic order, d_ik the direct fp64 squared distance (so an exact tie
    puts the lower index first).  [GMM] abstract (border vectors assigned to
    more than one cluster; the plainest hard reading is the two nearest).
    Needs k >= 2.  Returns (labels int64 [n, 2], d fp64 [n, 2])."""
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    if Chat.shape[0] < 2:
        raise ValueError("top-2 needs at least two centroids")
    n = X.shape[0]
    labels = np.empty((n, 2), dtype=np.int64)
    dist = np.empty((n, 2))
    rows = max(1, (1 << 22) // max(1, Chat.shape[0] * Chat.shape[1]))
    for r0 in range(0, n, rows):
        Dm = sq_dist_direct(X[r0:r0 + rows], Chat)
        order = np.argsort(Dm, axis=1, kind="stable")[:, :2]   # stable: equal distances keep index order
        labels[r0:r0 + rows] = order
        dist[r0:r0 + rows] = np.take_along_axis(Dm, order, axis=1)
    return labels, dist


def soft_assign(X, Chat, log_w, sigma2: float):
    """Gaussian-mixture E-step statistics of each point without the N x K
    responsibility matrix.  [GMM] abstract (soft clustering; responsibilities
    never materialised).

    Readings: isotropic components sharing the variance sigma2, centred at
    the (dtype-rounded) centroids, with log-weights log_w [k] (zeros when
    None); the constant (2*pi*sigma2)**(-D/2) is left out.  For each point
        a_ik = log_w_k - d_ik / (2 * sigma2),   d_ik the direct fp64 distance,
        L_i  = log sum_k exp(a_ik)                (log of the mixture density),
        map_i = the lowest k maximising a_ik      (its most responsible component);
    the responsibilities are then r_ik = exp(a_ik - L_i).  The sum is taken
    after subtracting the row maximum.  Returns (map int64 [n], L fp64 [n])."""
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    k = Chat.shape[0]
    lw = np.zeros(k) if log_w is None else np.asarray(log_w, np.float64)
    n = X.shape[0]
    lab = np.empty(n, dtype=np.int64)
    L = np.empty(n)
    rows = max(1, (1 << 22) // max(1, k * Chat.shape[1]))
    for r0 in range(0, n, rows):
        A = lw[None, :] - sq_dist_direct(X[r0:r0 + rows], Chat) / (2.0 * sigma2)
        m = A.max(axis=1)
        lab[r0:r0 + rows] = A.argmax(axis=1)          # first maximum: lowest index
        L[r0:r0 + rows] = m + np.log(np.exp(A - m[:, None]).sum(axis=1))
    return lab, L


def gauss_sum(X, Y, w, sigma2: float):
    """Gauss kernel sum at every point: G_i = sum_k w_k exp(-||x_i - y_k||^2 / (2 sigma2)),
    weights of any sign, squared distance the direct fp64 sum.  [GS] abstract
    (Gauss sums with signed weights; matrix-free Gaussian kernel blocks).
    Reading: the bandwidth enters as 2 * sigma2 (the pages fix no convention);
    the sources are given already rounded to the dtype of X, as centroids are.
    Returns G fp64 [n]."""
    X = np.asarray(X, np.float64)
    Y = np.asarray(Y, np.float64)
    w = np.asarray(w, np.float64)
    n = X.shape[0]
    G = np.empty(n)
    rows = max(1, (1 << 22) // max(1, Y.shape[0] * Y.shape[1]))
    for r0 in range(0, n, rows):
        # rounded products, then their sum (no fused multiply-add: w e - w e is exactly 0)
        G[r0:r0 + rows] = (np.exp(-sq_dist_direct(X[r0:r0 + rows], Y) / (2.0 * sigma2)) * w[None, :]).sum(axis=1)
    return G


def seed_random(n: int, u) -> np.ndarray:
    """Random seeding: centroid j is row floor(u_j * n) (with replacement), u_j
    uniforms in [0, 1) supplied by the caller.  The pages only name seeding as
    outside the method's inner loop ([HN] なぜ Hacker News のスレッドが重要だったか);
    this is the plainest random initialisation.  Returns int64 [k]."""
    u = np.asarray(u, np.float64)
    return np.minimum(np.floor(u * n).astype(np.int64), n - 1)


def kmeanspp(X, u) -> tuple[np.ndarray, np.ndarray]:
    """k-means++ (D^2) seeding, the seeding named in [HN] なぜ Hacker News の
    スレッドが重要だったか, with the caller's uniforms u [k]:
      c_0 = row floor(u_0 * n);
      for j >= 1: D2_i = min over the chosen rows c of ||x_i - c||^2 (direct
      fp64), and c_j = row i for the smallest i with
      sum_{i' <= i} D2_i' > u_j * sum_i D2_i  (the inverse CDF of D^2 sampling);
      if sum_i D2_i = 0 (every row coincides with a chosen one), row floor(u_j * n).
    Returns (chosen rows int64 [k], D2 after the last choice fp64 [n])."""
    X = np.asarray(X, np.float64)
    u = np.asarray(u, np.float64)
    n = X.shape[0]
    idx = np.empty(u.shape[0], dtype=np.int64)
    idx[0] = min(int(np.floor(u[0] * n)), n - 1)
    d2 = _rowwise_sq_dist(X, X[idx[0]][None, :])
    for j in range(1, u.shape[0]):
        cum = np.cumsum(d2)
        total = cum[-1]
        if total > 0:
            idx[j] = min(int(np.searchsorted(cum, u[j] * total, side="right")), n - 1)
        else:
            idx[j] = min(int(np.floor(u[j] * n)), n - 1)
        d2 = np.minimum(d2, _rowwise_sq_dist(X, X[idx[j]][None, :]))
    return idx, d2


def update(X, labels, C_prev, k: int):
    """Centroid update stage: c_k = (1/n_k) * sum_{i: label_i = k} x_i, and an
    empty cluster keeps its previous centroid.

    [FK] abstract (centroid update stage; the sort-inverse update is a
    per-cluster reduction of the points assigned to it).  Sums are fp64
    ``np.bincount`` accumulations, one per dimension.  Returns
    (C_new fp64 [k, d], counts int64 [k]).
    """
    X = np.asarray(X, np.float64)
    labels = np.asarray(labels).astype(np.int64, copy=False)
    C_prev = np.asarray(C_prev, np.float64)
    d = X.shape[1]
    counts = np.bincount(labels, minlength=k)
    S = np.empty((k, d))
    step = 16
    for j0 in range(0, d, step):
        cols = np.ascontiguousarray(X[:, j0:j0 + step].T)
        for j in range(cols.shape[0]):
            S[:, j0 + j] = np.bincount(labels, weights=cols[j], minlength=k)
    C_new = C_prev.copy()
    nz = counts > 0
    C_new[nz] = S[nz] / counts[nz, None]
    return C_new, counts


def inertia(dmin) -> float:
    """Sum of the per-point squared distances, correctly rounded (math.fsum)."""
    return math.fsum(np.asarray(dmin, np.float64).tolist())


def lloyd(X, fmt: str, C0, iters: int):
    """Exact Lloyd k-means from C0 for exactly ``iters`` iterations.

    [FK] abstract and [HN] 論文の要点: assignment stage then update stage,
    formulas unchanged.  Each iteration t: Chat_t = round(C_t -> fmt);
    labels_t, dmin_t = assign(X, Chat_t); J_t = sum dmin_t;
    C_{t+1} = update(X, labels_t, C_t).

    Returns dict(labels, C, inertia, history, counts) with labels/inertia of
    the last assignment and C after the last update.
    """
    if iters < 1:
        raise ValueError("iters must be >= 1")
    X = np.asarray(X, np.float64)
    C = np.asarray(C0, np.float64).copy()
    k = C.shape[0]
    hist = []
    labels = counts = None
    J = None
    for _ in range(iters):
        Chat = round_to_format(C, fmt)
        labels, dmin = assign(X, Chat)
        J = inertia(dmin)
        hist.append(J)
        C, counts = update(X, labels, C, k)
    return dict(labels=labels, C=C, inertia=J, history=hist, counts=counts)


def near_tie_report(X, Chat, labels_gpu, labels_orc, *, rel: float = 1e-5):
    """Classify label mismatches between a candidate and the oracle.

    A mismatching row is excused when it is a near-tie: the gap between the
    best and second-best oracle distances is below rel*||x||^2, and the
    candidate's chosen centroid is itself within rel*||x||^2 of the best.
    Returns dict(mismatch, excused, failed, fail_rows, near_ties).
    """
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    lg = np.asarray(labels_gpu).astype(np.int64)
    lo = np.asarray(labels_orc).astype(np.int64)
    bad = np.nonzero(lg != lo)[0]
    out = dict(mismatch=int(bad.size), excused=0, failed=0, fail_rows=[], near_ties=0)
    if bad.size == 0:
        return out
    xx = np.einsum("ij,ij->i", X[bad], X[bad])
    tol = rel * xx
    d_all = sq_dist_direct(X[bad], Chat)
    srt = np.sort(d_all, axis=1)
    best = srt[:, 0]
    second = srt[:, 1] if Chat.shape[0] > 1 else np.full(bad.size, np.inf)
    d_g = d_all[np.arange(bad.size), np.clip(lg[bad], 0, Chat.shape[0] - 1)]
    valid = (lg[bad] >= 0) & (lg[bad] < Chat.shape[0])
    near = (second - best) < tol
    ok = valid & near & ((d_g - best) < tol)
    out["near_ties"] = int(near.sum())
    out["excused"] = int(ok.sum())
    out["failed"] = int((~ok).sum())
    out["fail_rows"] = bad[~ok][:20].tolist()
    return out


def centroid_rel_err(C_cand, C_orc, x_rms: float) -> float:
    """max_k ||c_cand,k - c_orc,k|| / max(||c_orc,k||, 1e-3 * x_rms)."""
    C_cand = np.asarray(C_cand, np.float64)
    C_orc = np.asarray(C_orc, np.float64)
    num = np.linalg.norm(C_cand - C_orc, axis=-1)
    den = np.maximum(np.linalg.norm(C_orc, axis=-1), 1e-3 * float(x_rms))
    return float((num / den).max()) if num.size else 0.0
