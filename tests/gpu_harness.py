"""Teacher-forced parity between the HIP path (through the C ABI binding) and
the fp64 oracle.

Protocol per iteration t (the oracle never sees anything from the GPU except
the state it is asked to check from):
  * assign: the oracle assigns with the GPU's own fp32 centroids C_t (exact in
    fp64, so both sides round the same values); labels must match except
    counted near-ties (gap to the second best below 1e-5*||x||^2 and the GPU's
    choice within that of the best); inertia within 1e-5 relative; min_d2
    within 1e-5 of the row's scale.
  * update: the oracle updates from the GPU's labels L_t; counts must match
    exactly and centroids within 1e-4 (per centroid, norm-relative with a
    floor of 1e-3 * RMS ||x||).
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle

TOL_INERTIA = 1e-5
TOL_CENTROID = 1e-4
TOL_TIE = 1e-5


def rowwise_sq_dist(A, B) -> np.ndarray:
    """Row i: sum_d (A[i, d] - B[i, d])**2 in fp64."""
    diff = np.asarray(A, np.float64) - np.asarray(B, np.float64)
    return np.einsum("ij,ij->i", diff, diff)


def log(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def decode(X: torch.Tensor, fmt: str) -> np.ndarray:
    """Exact fp64 values of a CPU tensor in its storage dtype."""
    X = X.detach().cpu().contiguous()
    if fmt == "bf16":
        return oracle.decode(X.view(torch.int16).numpy().view(np.uint16), "bf16")
    if fmt == "fp16":
        return oracle.decode(X.numpy(), "fp16")
    return oracle.decode(X.numpy(), "fp32")


FMT = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}


def check_assign(Xd, C_gpu, labels_gpu, inertia_gpu, fmt, *, min_d2=None, rows=None, tag=""):
    """Oracle assignment against the GPU's centroids; rows = optional sample."""
    Cd = np.asarray(C_gpu, np.float64)
    Ch = oracle.round_to_format(Cd, fmt)
    sub = Xd if rows is None else Xd[rows]
    lab_g = np.asarray(labels_gpu) if rows is None else np.asarray(labels_gpu)[rows]
    lab_o, dmin = oracle.assign(sub, Ch)
    rep = oracle.near_tie_report(sub, Ch, lab_g, lab_o, rel=TOL_TIE)
    assert rep["failed"] == 0, f"{tag}: label mismatches beyond near-ties: {rep}"
    if min_d2 is not None:
        md = np.asarray(min_d2, np.float64) if rows is None else np.asarray(min_d2, np.float64)[rows]
        ok = lab_g == lab_o
        xx = np.einsum("ij,ij->i", sub, sub)
        err = np.abs(md[ok] - dmin[ok])
        assert np.all(err <= 1e-5 * np.maximum(dmin[ok], 1e-3 * xx[ok]) + 1e-30), \
            f"{tag}: min_d2 off by {err.max()}"
    if rows is None and inertia_gpu is not None:
        J = oracle.inertia(dmin)
        assert abs(float(inertia_gpu) - J) <= TOL_INERTIA * max(J, 1e-30), f"{tag}: inertia {inertia_gpu} vs {J}"
    return rep


def check_inertia_of_labels(Xd, C_gpu, labels_gpu, inertia_gpu, fmt, tag=""):
    """Inertia property at any size: the GPU's inertia equals the fp64 sum of
    squared distances to the (rounded) centroids the GPU chose."""
    Ch = oracle.round_to_format(np.asarray(C_gpu, np.float64), fmt)
    lab = np.asarray(labels_gpu).astype(np.int64)
    J = 0.0
    step = 1 << 20
    for r0 in range(0, Xd.shape[0], step):
        d = Xd[r0:r0 + step] - Ch[lab[r0:r0 + step]]
        J += float(np.einsum("ij,ij->", d, d))
    assert abs(float(inertia_gpu) - J) <= TOL_INERTIA * J, f"{tag}: inertia {inertia_gpu} vs {J}"


def check_update(Xd, labels_gpu, C_prev_gpu, C_new_gpu, counts_gpu, K, tag=""):
    Cp = np.asarray(C_prev_gpu, np.float64)
    Cn, cnt = oracle.update(Xd, np.asarray(labels_gpu), Cp, K)
    assert np.array_equal(np.asarray(counts_gpu), cnt), f"{tag}: counts differ"
    rms = float(np.sqrt(np.einsum("ij,ij->i", Xd, Xd).mean()))
    err = oracle.centroid_rel_err(np.asarray(C_new_gpu), Cn, rms)
    assert err <= TOL_CENTROID, f"{tag}: centroid rel err {err:.3e}"
    # an empty cluster keeps its previous fp32 value bit for bit
    empty = cnt == 0
    assert np.array_equal(np.asarray(C_new_gpu)[empty], np.asarray(C_prev_gpu)[empty]), f"{tag}: empty cluster moved"
    return err


def check_step(km, X, Xd, C, fmt, *, sample=None, rng=None, tag=""):
    """One teacher-forced iteration from the GPU state C [B,K,D] (device):
    GPU assign + update, then the oracle's assign with C (labels on every row,
    or on `sample` seeded rows per instance plus the full-row inertia
    property) and the oracle's update from the GPU labels on every row.
    Returns (labels, C_new, inertia, near-tie count, centroid error)."""
    B, N, _ = X.shape
    K = C.shape[1]
    labels, md, inertia = km.assign(X, C, want_min_d2=True)
    C_new, counts = km.update(X, labels, C)
    torch.cuda.synchronize()
    lab_c, md_c, J_c = labels.cpu().numpy(), md.cpu().numpy(), inertia.cpu().numpy()
    Cc, Cn_c, cnt_c = C.cpu().numpy(), C_new.cpu().numpy(), counts.cpu().numpy()
    ties, cerr = 0, 0.0
    for b in range(B):
        rows = None
        if sample is not None and N > sample:
            rows = np.sort((rng or np.random.default_rng(0)).choice(N, size=sample, replace=False))
        rep = check_assign(Xd[b], Cc[b], lab_c[b], J_c[b], fmt, min_d2=md_c[b], rows=rows, tag=f"{tag} b{b}")
        if rows is not None:
            check_inertia_of_labels(Xd[b], Cc[b], lab_c[b], J_c[b], fmt, tag=f"{tag} b{b}")
        ties += rep["excused"]
        cerr = max(cerr, check_update(Xd[b], lab_c[b], Cc[b], Cn_c[b], cnt_c[b], K, tag=f"{tag} b{b}"))
    log(f"{tag}: ok ({'all' if sample is None or N <= sample else sample} label rows per instance, "
        f"near-ties excused {ties}, centroid err {cerr:.2e})")
    return labels, C_new, inertia, ties, cerr


def teacher_forced(km, X_cpu, C0_cpu, iters, *, sample=None, tag="", check_fit=True, seed=0):
    """Run `iters` GPU iterations step by step and check each one against the
    oracle.  X_cpu [B,N,D], C0_cpu [B,K,D].  Returns per-iteration stats."""
    fmt = FMT[X_cpu.dtype]
    B, N, D = X_cpu.shape
    K = C0_cpu.shape[1]
    X = X_cpu.cuda()
    C = C0_cpu.cuda()
    Xd = [decode(X_cpu[b], fmt) for b in range(B)]
    rng = np.random.default_rng(seed)
    stats = []
    labels_seq, C_seq, J_seq = [], [], []
    for t in range(iters):
        t0 = time.time()
        labels, md, inertia = km.assign(X, C, want_min_d2=True)
        C_new, counts = km.update(X, labels, C)
        torch.cuda.synchronize()
        lab_c, md_c, J_c = labels.cpu().numpy(), md.cpu().numpy(), inertia.cpu().numpy()
        Cc, Cn_c, cnt_c = C.cpu().numpy(), C_new.cpu().numpy(), counts.cpu().numpy()
        ties = 0
        cerr = 0.0
        for b in range(B):
            rows = None
            if sample is not None and N > sample:
                rows = np.sort(rng.choice(N, size=sample, replace=False))
            rep = check_assign(Xd[b], Cc[b], lab_c[b], J_c[b], fmt, min_d2=md_c[b], rows=rows,
                               tag=f"{tag} it{t} b{b}")
            if rows is not None:
                check_inertia_of_labels(Xd[b], Cc[b], lab_c[b], J_c[b], fmt, tag=f"{tag} it{t} b{b}")
            ties += rep["excused"]
            cerr = max(cerr, check_update(Xd[b], lab_c[b], Cc[b], Cn_c[b], cnt_c[b], K, tag=f"{tag} it{t} b{b}"))
        stats.append(dict(it=t, near_ties=ties, centroid_err=cerr, inertia=J_c.tolist()))
        log(f"{tag} it{t}: ok (near-ties excused {ties}, centroid err {cerr:.2e}, {time.time() - t0:.1f}s)")
        labels_seq.append(labels)
        C_seq.append(C_new)
        J_seq.append(inertia)
        C = C_new
    if check_fit:
        # the fused driver runs the same kernels in the same order: bitwise equal
        lf, Cf, Jf, hist = km.fit(X, C0_cpu.cuda(), iters, history=True)
        torch.cuda.synchronize()
        assert torch.equal(lf, labels_seq[-1]), f"{tag}: fit labels differ from step-by-step"
        assert torch.equal(Cf, C_seq[-1]), f"{tag}: fit centroids differ from step-by-step"
        assert torch.equal(Jf, J_seq[-1]), f"{tag}: fit inertia differs"
        assert torch.equal(hist, torch.stack(J_seq)), f"{tag}: fit inertia history differs"
    return stats
