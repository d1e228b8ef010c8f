"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Sizes span several assign tiles (64 centroids, 128-512 points), several sort
tiles (4096 keys) and update chunks (256 sorted rows per chunk, 32 chunks per
group) with ragged tails.  Full-size workloads check sampled rows plus
properties that hold at any size.
"""

import numpy as np
import pytest
import torch

import datagen
import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def km():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_means_clustering_amd as km
    return km


def _stats_ok(stats):
    assert all(s["centroid_err"] <= H.TOL_CENTROID for s in stats)


def test_c1_full(km):
    p = datagen.make("c1")
    _stats_ok(H.teacher_forced(km, p.X, p.C0, p.iters, tag="c1"))


def test_c2_scaled_ragged(km):
    p = datagen.make("c2", n=70001, k=300, seed=1)
    _stats_ok(H.teacher_forced(km, p.X, p.C0, 4, tag="c2s"))


def test_c3_scaled_zipf(km):
    p = datagen.make("c3", n=65539, k=2053, seed=2)
    _stats_ok(H.teacher_forced(km, p.X, p.C0, 3, tag="c3s"))


def test_c4_scaled_batched(km):
    p = datagen.make("c4", n=3001, k=77, batch=5, seed=3)
    _stats_ok(H.teacher_forced(km, p.X, p.C0, 3, tag="c4s"))


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("d", [16, 64, 256])
def test_dims_and_dtypes(km, dtype, d):
    X, C0, _, _ = datagen.mixture(5003, d, 40, dtype=dtype, center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=50, seed=d, k=45)
    _stats_ok(H.teacher_forced(km, X, C0, 2, tag=f"{dtype}-D{d}"))


def test_tiny_ragged(km):
    X, C0, _, _ = datagen.mixture(37, 32, 4, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=51, seed=0, k=5)
    _stats_ok(H.teacher_forced(km, X, C0, 3, tag="tiny"))


def test_k_equals_one(km):
    X, C0, _, _ = datagen.mixture(9000, 128, 3, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=52, seed=0, k=1)
    _stats_ok(H.teacher_forced(km, X, C0, 2, tag="k1"))
    labels, C, J, _ = km.fit(X.cuda(), C0.cuda(), 2)
    assert int(labels.max()) == 0
    mean = X[0].double().mean(0)
    assert torch.allclose(C[0, 0].cpu().double(), mean, rtol=1e-4, atol=1e-5)


def test_k_equals_n_identity(km):
    X, _, _, _ = datagen.mixture(700, 64, 700, dtype="bf16", center_dist="normal", center_scale=3.0, sigma=1.0,
                                 weights=None, workload_code=53, seed=0)
    Xu = torch.unique(X[0].float(), dim=0)
    Xu = Xu[torch.randperm(Xu.shape[0], generator=torch.Generator().manual_seed(0))]
    Xb = Xu.to(torch.bfloat16)[None].contiguous()
    C0 = Xb.float()
    labels, md, J = km.assign(Xb.cuda(), C0.cuda(), want_min_d2=True)
    assert torch.equal(labels.cpu()[0], torch.arange(Xb.shape[1], dtype=torch.int32))
    assert float(J[0]) == 0.0 and float(md.abs().max()) == 0.0
    Cn, cnt = km.update(Xb.cuda(), labels, C0.cuda())
    assert torch.equal(Cn.cpu(), C0) and int(cnt.min()) == 1


def test_duplicate_centroids_lowest_index(km):
    X, C0, _, _ = datagen.mixture(20000, 128, 30, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=54, seed=0, k=40)
    C0 = C0.clone()
    C0[0, 33] = C0[0, 7]       # exact duplicates: index 33 must never win
    C0[0, 39] = C0[0, 2]
    labels, _, _ = km.assign(X.cuda(), C0.cuda())
    lab = labels.cpu()
    assert not bool((lab == 33).any()) and not bool((lab == 39).any())
    assert bool((lab == 7).any()) and bool((lab == 2).any())
    _stats_ok(H.teacher_forced(km, X, C0, 2, tag="dup"))


def test_identical_rows(km):
    X = torch.full((1, 5000, 32), 0.75, dtype=torch.bfloat16)
    X[0, :, 3] = -1.5
    C0 = torch.zeros(1, 6, 32)
    C0[0, :] = X[0, 0].float()
    labels, C, J, _ = km.fit(X.cuda(), C0.cuda(), 2)
    assert int(labels.abs().max()) == 0 and float(J[0]) == 0.0
    assert torch.equal(C.cpu(), C0)


def test_forced_empty_clusters(km):
    X, C0, _, _ = datagen.mixture(30000, 64, 20, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=55, seed=0, k=24)
    C0 = C0.clone()
    C0[0, 5] = 1e4             # far away: empty for every iteration
    C0[0, 17] = -1e4
    stats = H.teacher_forced(km, X, C0, 3, tag="empty")
    _stats_ok(stats)
    _, C, _, _ = km.fit(X.cuda(), C0.cuda(), 3)
    assert torch.equal(C.cpu()[0, 5], C0[0, 5]) and torch.equal(C.cpu()[0, 17], C0[0, 17])


@pytest.mark.parametrize("dtype,d,batch,k", [("bf16", 128, 2, 33), ("fp32", 32, 1, 33), ("fp16", 64, 3, 33),
                                             ("fp16", 64, 3, 300), ("bf16", 64, 5, 120)])
def test_fit_equals_stepwise_calls(km, dtype, d, batch, k):
    """kmeans_fit folds the inertia reduction into the sort and the next
    iteration's centroid preparation into the update (empty clusters keep the
    preparation of their unchanged centroid).  Its labels, centroids and
    inertia history must equal the same iterations run as stand-alone
    kmeans_assign + kmeans_update calls bit for bit, with empty clusters
    present in every instance.  The sort takes one 8-bit pass for K = 33, the
    wide-digit pass for 3 x 300 keys and the segmented pass for 5 x 120."""
    X, C0, _, _ = datagen.mixture(12_345, d, 20, dtype=dtype, center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=57, seed=3, k=k, batch=batch)
    C0 = C0.clone()
    C0[:, 4] = 1e4            # far away: empty in every iteration of every instance
    C0[:, 30] = -1e4
    Xc, C = X.cuda(), C0.cuda()
    iters = 3
    lab_f, C_f, J_f, hist_f = km.fit(Xc, C, iters, history=True)
    Cs = C.clone()
    for t in range(iters):
        lab, _, J = km.assign(Xc, Cs)
        assert torch.equal(J, hist_f[t]), f"{dtype}: inertia of iteration {t} differs"
        Cs, _ = km.update(Xc, lab, Cs)
    assert torch.equal(lab, lab_f) and torch.equal(Cs, C_f) and torch.equal(J, J_f)
    assert torch.equal(C_f[:, 4].cpu(), C0[:, 4]) and torch.equal(C_f[:, 30].cpu(), C0[:, 30])


def test_update_all_rows_one_cluster_large_k(km):
    """Every row in cluster 0 of K=65,536: the offsets of the other 65,535 keys
    form one range filled after the last row, and every one of those clusters
    is empty (count 0, previous centroid kept)."""
    n, k, d = 100_003, 65_536, 64
    X, _, _, _ = datagen.mixture(n, d, 4, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=57, seed=0)
    lab = np.zeros((1, n), dtype=np.int32)
    C_prev = torch.randn(1, k, d, generator=torch.Generator().manual_seed(1))
    C_new, counts = km.update(X.cuda(), torch.from_numpy(lab).cuda(), C_prev.cuda())
    torch.cuda.synchronize()
    err = H.check_update(H.decode(X[0], "fp16"), lab[0], C_prev[0].numpy(), C_new.cpu()[0].numpy(),
                         counts.cpu()[0].numpy(), k, tag="one_cluster_large_k")
    H.log(f"update one cluster, K={k}: centroid err {err:.2e}")


@pytest.mark.parametrize("case", ["zipf", "one_cluster", "two_clusters"])
def test_update_long_segments(km, case):
    """Skewed labels: one segment spans many chunks and groups (the hot-cluster
    contention case of the update)."""
    n, k = 600_001, 1000
    X, _, _, _ = datagen.mixture(n, 128, 8, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=56, seed=0)
    if case == "zipf":
        lab = datagen.zipf_labels(n, k, 1.1, seed=1)
    elif case == "one_cluster":
        lab = np.full((1, n), 731, dtype=np.int32)
    else:
        lab = np.where(np.arange(n) % 3 == 0, 5, 998).astype(np.int32)[None]
    C_prev = torch.randn(1, k, 128, generator=torch.Generator().manual_seed(0))
    labels = torch.from_numpy(lab).cuda()
    C_new, counts = km.update(X.cuda(), labels, C_prev.cuda())
    torch.cuda.synchronize()
    Xd = H.decode(X[0], "bf16")
    err = H.check_update(Xd, lab[0], C_prev[0].numpy(), C_new.cpu()[0].numpy(), counts.cpu()[0].numpy(), k,
                         tag=case)
    H.log(f"update {case}: centroid err {err:.2e}, max count {int(counts.max())}")


def test_batched_equals_unbatched(km):
    p = datagen.make("c4", n=4096, k=64, batch=3, seed=4)
    lb, Cb, Jb, _ = km.fit(p.X.cuda(), p.C0.cuda(), 3)
    for b in range(3):
        l1, C1, J1, _ = km.fit(p.X[b:b + 1].contiguous().cuda(), p.C0[b:b + 1].contiguous().cuda(), 3)
        assert torch.equal(l1[0], lb[b]) and torch.equal(C1[0], Cb[b]) and torch.equal(J1[0], Jb[b])
    # 2-D inputs are the B = 1 case
    l2, C2, J2, _ = km.fit(p.X[0].contiguous().cuda(), p.C0[0].contiguous().cuda(), 3)
    assert torch.equal(l2, lb[0]) and torch.equal(C2, Cb[0])


@pytest.mark.parametrize("n,k,batch", [(3001, 256, 7), (1025, 255, 7), (65_536, 200, 3), (70_001, 256, 2),
                                       (5, 2, 300), (1, 1, 257)])
def test_batched_update_skewed_labels(km, n, k, batch):
    """Batched update against the oracle, instance by instance.  With K <= 256
    the key sort takes one pass over tiles that stay inside an instance while
    an instance spans at most 64 tiles of 1024 keys (a ragged tail in the
    first case; in the second each instance's one-key tail takes a tile of
    its own, 14 tiles where the unsegmented sort has 8; exactly 64 tiles in
    the third), and two passes beyond that (the fourth).  Labels: one
    instance entirely in the last cluster, one holding only the first and
    last clusters, one Zipf-skewed, the rest uniform.  The last two cases are
    hundreds of tiny instances (B*K of 600 and 257 with K <= 2), which do not
    take the segmented pass (it would need a nearly empty tile per instance)
    but the one-pass wide-digit sort of their 10- and 9-bit keys."""
    d = 64
    X, _, _, _ = datagen.mixture(n, d, 8, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=57, seed=n, batch=batch)
    rng = np.random.default_rng(k)
    lab = rng.integers(0, k, size=(batch, n)).astype(np.int32)
    lab[0] = k - 1
    lab[1] = np.where(rng.random(n) < 0.5, 0, k - 1)
    if batch > 2:
        lab[2] = datagen.zipf_labels(n, k, 1.1, seed=3)[0]
    C_prev = torch.randn(batch, k, d, generator=torch.Generator().manual_seed(5))
    C_new, counts = km.update(X.cuda(), torch.from_numpy(lab).cuda(), C_prev.cuda())
    torch.cuda.synchronize()
    C_new, counts = C_new.cpu().numpy(), counts.cpu().numpy()
    worst = 0.0
    for b in range(batch):
        err = H.check_update(H.decode(X[b], "fp16"), lab[b], C_prev[b].numpy(), C_new[b], counts[b], k,
                             tag=f"batched n={n} k={k} b={b}")
        worst = max(worst, err)
    H.log(f"batched update n={n} k={k} B={batch}: worst centroid err {worst:.2e}")


@pytest.mark.parametrize("n,k", [(20_011, 300), (2_200_011, 5_000)])
def test_update_misaligned_labels_equal_aligned(km, n, k):
    """The sort reads labels four per 16-byte load where a tile is whole and
    aligned, one at a time otherwise: labels at an address 4 bytes past a
    16-byte boundary (every tile on the second path) give the same centroids
    and counts bit for bit as the same labels aligned.  Shapes: one
    wide-digit pass over 1,024-key tiles (K = 300) and two 8-bit passes over
    4,096-key tiles (K = 5,000), both with a ragged last tile."""
    X, C0, _, _ = _mixture(n, 64, k, "bf16", seed=31)
    Xc, C = X[0].cuda(), C0[0].cuda()
    lab, _, _ = km.assign(Xc, C)
    buf = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    lab_m = buf[1:]
    lab_m.copy_(lab)
    assert lab_m.data_ptr() % 16 == 4
    C_a, n_a = km.update(Xc, lab, C)
    C_m, n_m = km.update(Xc, lab_m, C)
    torch.cuda.synchronize()
    assert torch.equal(n_a, n_m) and torch.equal(C_a, C_m)


@pytest.mark.parametrize("n", [2052 * 4096 - 5, 9_000_001])
def test_update_scan_over_several_rounds(km, n):
    """More than 2,048 tiles of 4,096 keys: the digit scan covers 2,048 tile
    counts per round, so these take two rounds, with 16-byte loads (2,052
    tiles) and with the per-count path (2,198 tiles, not a multiple of 4);
    both passes of the 16-bit sort (K = 5,000) scan.  Counts exactly and
    centroids within tolerance against the oracle."""
    K = 5_000
    X, C0, _, _ = _mixture(n, 16, K, "fp16", seed=n % 1009)
    Xc, C = X[0].cuda(), C0[0].cuda()
    lab, _, _ = km.assign(Xc, C)
    C_new, counts = km.update(Xc, lab, C)
    torch.cuda.synchronize()
    err = H.check_update(H.decode(X[0], "fp16"), lab.cpu().numpy(), C.cpu().numpy(), C_new.cpu().numpy(),
                         counts.cpu().numpy(), K, tag=f"n={n}")
    print(f"n={n}: centroid rel err {err:.2e}")


@pytest.mark.parametrize("n,k,batch", [(20_011, 300, 1), (2_200_011, 5_000, 1), (30_001, 200, 3), (70_001, 64, 1)])
def test_update_out_of_range_labels_clamp(km, n, k, batch):
    """Labels outside [0, K) handed to kmeans_update are a caller error with
    unspecified results that must stay memory safe: the sort clamps each
    such label to K - 1 (negative ones included), so the update equals, bit
    for bit, the update of the clamped labels.  Shapes: one wide-digit pass,
    the two-pass 16-bit sort, the segmented batched pass and one scanned
    8-bit pass, each with a ragged last tile."""
    X, C0, _, _ = _mixture(n, 32, k, "fp16", seed=n % 97 + k, batch=batch)
    Xc = X.cuda() if batch > 1 else X[0].cuda()
    C = C0.cuda() if batch > 1 else C0[0].cuda()
    lab, _, _ = km.assign(Xc, C)
    bad = torch.tensor([-1, -(2 ** 31), k, k + 5, 2 ** 31 - 1], dtype=torch.int32, device="cuda")
    raw = lab.clone().reshape(-1)
    idx = torch.arange(0, raw.numel(), 7, device="cuda")
    raw[idx] = bad[torch.arange(idx.numel(), device="cuda") % bad.numel()]
    clamped = torch.where((raw >= 0) & (raw < k), raw, torch.full_like(raw, k - 1))
    C_r, n_r = km.update(Xc, raw.reshape(lab.shape), C)
    C_c, n_c = km.update(Xc, clamped.reshape(lab.shape), C)
    torch.cuda.synchronize()
    assert torch.equal(n_r, n_c) and torch.equal(C_r, C_c)
    assert int(n_r.sum()) == batch * n


@pytest.mark.parametrize("n,k,batch", [(20_011, 257, 1), (50_000, 2048, 1), (30_001, 300, 2), (9_001, 290, 7)])
def test_wide_digit_update(km, n, k, batch):
    """Keys of 9 to 11 bits (B*K from 257 to 2048) sort in one pass with a
    digit that wide while its histogram stays within 2^20 words: 9 and 11
    bits unbatched, 10 and 11 bits over instances whose K is too large for
    the segmented pass.  Skewed labels (one instance all in the last
    cluster, one Zipf) against the oracle."""
    d = 32
    X, _, _, _ = datagen.mixture(n, d, 8, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=58, seed=k, batch=batch)
    rng = np.random.default_rng(n)
    lab = rng.integers(0, k, size=(batch, n)).astype(np.int32)
    lab[0, : n // 3] = k - 1
    if batch > 1:
        lab[1] = datagen.zipf_labels(n, k, 1.1, seed=5)[0]
    C_prev = torch.randn(batch, k, d, generator=torch.Generator().manual_seed(7))
    C_new, counts = km.update(X.cuda(), torch.from_numpy(lab).cuda(), C_prev.cuda())
    torch.cuda.synchronize()
    C_new, counts = C_new.cpu().numpy(), counts.cpu().numpy()
    worst = 0.0
    for b in range(batch):
        worst = max(worst, H.check_update(H.decode(X[b], "bf16"), lab[b], C_prev[b].numpy(), C_new[b], counts[b], k,
                                          tag=f"wide n={n} k={k} b={b}"))
    H.log(f"wide-digit update n={n} k={k} B={batch}: worst centroid err {worst:.2e}")


def test_binding_rejects_mismatched_arguments(km):
    """The Python binding checks shapes, devices and caller buffers before any
    launch: a mismatch raises KMeansError instead of reaching a kernel."""
    X = torch.zeros(2, 100, 32, dtype=torch.float16, device="cuda")
    C = torch.zeros(2, 10, 32, dtype=torch.float32, device="cuda")
    lab = torch.zeros(2, 100, dtype=torch.int32, device="cuda")
    bad = [
        lambda: km.assign(X, torch.zeros(2, 10, 16, device="cuda")),                 # D differs
        lambda: km.assign(X, torch.zeros(3, 10, 32, device="cuda")),                 # B differs
        lambda: km.assign(X, C, labels=torch.zeros(2, 99, dtype=torch.int32, device="cuda")),
        lambda: km.update(X, lab[:, :50].contiguous(), C),                           # labels too short
        lambda: km.update(X, lab, C, C_new=torch.zeros(2, 9, 32, device="cuda")),    # C_new too small
        lambda: km.assign(X, C, ws=torch.zeros(1 << 20, dtype=torch.uint8)),         # workspace on the host
        lambda: km.assign(X, C, ws=torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")[::2]),  # strided
        lambda: km.assign_soft(X, C, 1.0, log_w=torch.zeros(2, 9, device="cuda")),
        lambda: km.gauss_sum(X, C, torch.zeros(2, 9, device="cuda"), 1.0),
        lambda: km.fit(X, torch.zeros(10, 32, device="cuda"), 2),                    # [K, D] with B = 2
    ]
    for i, call in enumerate(bad):
        with pytest.raises(km.KMeansError):
            call()
    # the good call still works, with a caller workspace of another dtype
    ws = torch.empty(km.workspace_bytes(100, 32, 10, 2, torch.float16) // 4 + 1, dtype=torch.float32, device="cuda")
    labels, _, J = km.assign(X, C, ws=ws)
    torch.cuda.synchronize()
    assert labels.shape == (2, 100) and torch.all(J == 0)


def test_determinism_and_resume(km):
    p = datagen.make("c3", n=50000, k=777, seed=6)
    X, C0 = p.X.cuda(), p.C0.cuda()
    a = km.fit(X, C0, 4, history=True)
    b = km.fit(X, C0, 4, history=True)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # resume: 4 iterations == 1 iteration, then 3 more from its centroids
    _, C1, _, _ = km.fit(X, C0, 1)
    c = km.fit(X, C1, 3, history=True)
    assert torch.equal(c[0], a[0]) and torch.equal(c[1], a[1]) and torch.equal(c[3], a[3][1:])


def test_no_nk_buffer(km):
    """The assignment never holds an N x K buffer: peak device memory during a
    call stays at inputs + outputs + the declared workspace."""
    n, k, d = 1 << 18, 4096, 128
    X = torch.randn(n, d, device="cuda").to(torch.bfloat16)
    C = torch.randn(k, d, device="cuda")
    ws = torch.empty(km.workspace_bytes(n, d, k, 1, torch.bfloat16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    km.assign(X, C, ws=ws)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    assert extra < n * 16 + (1 << 20), extra          # labels + inertia only
    assert ws.numel() < n * k // 16                   # workspace is O(N + K), not O(N*K)


def test_streamed_matches_in_core(km):
    p = datagen.make("c5", n=300_000, k=128, seed=7)
    X = p.X[0]
    budget = 2 * 40_000 * 128 * 2                    # 40k-row slots: 8 chunks
    Xp = X.pin_memory()
    lab_s, C_s, J_s, hist_s = km.fit_streamed(Xp, p.C0[0].cuda(), 3, budget, history=True)
    lab_i, C_i, J_i, hist_i = km.fit(X.cuda(), p.C0[0].cuda(), 3, history=True)
    torch.cuda.synchronize()
    # same kernels per row: labels of the first iteration agree exactly; the
    # later ones may differ only through centroid rounding at the 1e-7 level
    assert abs(hist_s[0] - float(hist_i[0, 0])) <= 1e-9 * hist_s[0]
    assert abs(J_s - float(J_i[0])) <= 1e-5 * J_s
    Xd = H.decode(X, "fp16")
    rms = float(np.sqrt(np.einsum("ij,ij->i", Xd, Xd).mean()))
    import oracle
    assert oracle.centroid_rel_err(C_s.cpu().numpy(), C_i.cpu().numpy(), rms) <= 1e-4
    mism = int((lab_s != lab_i.cpu()).sum())
    assert mism <= 1e-4 * X.shape[0], mism
    # the per-chunk timeline of that 3-iteration fit: 8 chunks per iteration,
    # each window ordered, a chunk's compute after its copy in, and its
    # labels out after its compute
    km.fit_streamed(Xp, p.C0[0].cuda(), 3, budget)
    tl = km.stream_timeline()
    assert len(tl) == 3 * 8 and [(int(r[0]), int(r[1])) for r in tl] == [(t, c) for t in range(3) for c in range(8)]
    eps = 1e-3
    for r in tl:
        assert r[2] <= r[3] and r[4] <= r[5] and r[6] <= r[7], r
        assert r[4] >= r[3] - eps and r[6] >= r[5] - eps, r
    _check_streamed_against_oracle(km, Xp, Xd, p.C0[0], 3, budget, (lab_s, C_s, J_s), tag="streamed")


def _check_streamed_against_oracle(km, Xp, Xd, C0, iters, budget, last, *, sample=None, tag=""):
    """Teacher-forced parity of the streamed path's own results (its
    accumulate-mode segment sums and fp64 means): the first iteration from C0,
    and the last of `iters` from the state the streamed path reached before
    it.  Labels against the oracle's assignment (every row, or a seeded
    sample plus the full-row inertia property), centroids against the
    oracle's update from the streamed labels; empty clusters keep the
    previous centroid bit for bit."""
    fmt = H.FMT[Xp.dtype]
    rng = np.random.default_rng(1)
    rows = None if sample is None or Xp.shape[0] <= sample else np.sort(
        rng.choice(Xp.shape[0], size=sample, replace=False))

    def one(C_prev, lab, C_new, J, t):
        Cp = C_prev.cpu().numpy() if isinstance(C_prev, torch.Tensor) else np.asarray(C_prev)
        rep = H.check_assign(Xd, Cp, lab.numpy(), J, fmt, rows=rows, tag=f"{tag} it{t}")
        if rows is not None:
            H.check_inertia_of_labels(Xd, Cp, lab.numpy(), J, fmt, tag=f"{tag} it{t}")
        Cn, cnt = oracle.update(Xd, lab.numpy(), Cp.astype(np.float64), Cp.shape[0])
        rms = float(np.sqrt(np.einsum("ij,ij->i", Xd, Xd).mean()))
        Cg = C_new.cpu().numpy()
        err = oracle.centroid_rel_err(Cg, Cn, rms)
        assert err <= H.TOL_CENTROID, f"{tag} it{t}: streamed centroid rel err {err:.3e}"
        assert np.array_equal(Cg[cnt == 0], Cp[cnt == 0]), f"{tag} it{t}: an empty cluster moved"
        H.log(f"{tag} it{t}: streamed update ok (centroid err {err:.2e}, empty clusters {int((cnt == 0).sum())}, "
              f"near-ties excused {rep['excused']})")

    lab1, C1, J1, _ = km.fit_streamed(Xp, C0.cuda(), 1, budget)
    one(C0, lab1, C1, J1, 0)
    if iters > 1:
        _, C_prev, _, _ = km.fit_streamed(Xp, C0.cuda(), iters - 1, budget)
        lab, C_last, J = last
        one(C_prev, lab, C_last, J, iters - 1)


@pytest.mark.parametrize("last", [500_000, 2_000_000])
def test_streamed_last_chunk_across_the_tile_size_change(km, last):
    """Slots of just over 2^21 rows and a last chunk of fewer: sort tiles and
    segment chunks are smaller up to 2^21 rows, so the last chunk needs a
    workspace layout of its own (at 500,000 rows its K = 1024 keys also take
    the one-pass wide-digit sort).  Streamed against in-core."""
    chunk, d, k = 2_097_152 + 1000, 16, 1024
    n = chunk + last
    X, C0, _, _ = datagen.mixture(n, d, 64, dtype="fp16", center_dist="normal", center_scale=3.0, sigma=1.0,
                                  weights=None, workload_code=63, seed=last, k=k)
    X, C0 = X[0], C0[0]
    budget = 2 * chunk * d * 2                      # two slots of `chunk` rows: two chunks
    Xp = X.pin_memory()
    lab_s, C_s, J_s, hist_s = km.fit_streamed(Xp, C0.cuda(), 2, budget, history=True)
    lab_i, C_i, J_i, hist_i = km.fit(X.cuda(), C0.cuda(), 2, history=True)
    torch.cuda.synchronize()
    assert abs(hist_s[0] - float(hist_i[0, 0])) <= 1e-9 * hist_s[0]
    assert abs(J_s - float(J_i[0])) <= 1e-5 * J_s
    Xd = H.decode(X, "fp16")
    rms = float(np.sqrt(np.einsum("ij,ij->i", Xd, Xd).mean()))
    import oracle
    assert oracle.centroid_rel_err(C_s.cpu().numpy(), C_i.cpu().numpy(), rms) <= 1e-4
    mism = int((lab_s != lab_i.cpu()).sum())
    assert mism <= 1e-4 * n, mism
    _check_streamed_against_oracle(km, Xp, Xd, C0, 2, budget, (lab_s, C_s, J_s), tag=f"streamed-last{last}")


def _first_and_last(km, p, *, sample, tag):
    """Full-size parity of a workload at its first and last iteration: the
    oracle checks iteration 0 from C0 and iteration iters-1 from the state the
    fit reached after iters-1 iterations (teacher-forced, labels on every row
    or on `sample` seeded rows per instance, update and inertia on every row);
    the fit's final labels, centroids and inertia equal those stepwise results
    bit for bit."""
    fmt = H.FMT[p.X.dtype]
    X = p.X.cuda()
    C0 = p.C0.cuda()
    Xd = [H.decode(p.X[b], fmt) for b in range(p.B)]
    rng = np.random.default_rng(17)
    H.check_step(km, X, Xd, C0, fmt, sample=sample, rng=rng, tag=f"{tag} it0")
    _, C_prev, _, _ = km.fit(X, C0, p.iters - 1)
    lab, C_last, J, _, _ = H.check_step(km, X, Xd, C_prev, fmt, sample=sample, rng=rng,
                                        tag=f"{tag} it{p.iters - 1}")
    lf, Cf, Jf, _ = km.fit(X, C0, p.iters)
    torch.cuda.synchronize()
    assert torch.equal(lf, lab) and torch.equal(Cf, C_last) and torch.equal(Jf, J), f"{tag}: fit differs"


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_c4_full(km):
    """All 8 iterations of the 64 instances, every row, teacher-forced."""
    p = datagen.make("c4")
    _stats_ok(H.teacher_forced(km, p.X, p.C0, p.iters, tag="c4", check_fit=True))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_c2_full(km):
    """All 20 iterations of N = 1,048,576, K = 1,024, fp16, every row,
    teacher-forced, and the fit equal to the stepwise calls."""
    p = datagen.make("c2")
    _stats_ok(H.teacher_forced(km, p.X, p.C0, p.iters, tag="c2", check_fit=True))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_c3_full_first_and_last(km):
    """The headline workload (N = 8,388,608, K = 65,536, bf16; the (3 point
    blocks, 8 waves) assignment): labels of 2^18 seeded rows at iterations 0
    and 9 of 10, the update and inertia on every row."""
    _first_and_last(km, datagen.make("c3"), sample=1 << 18, tag="c3")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_c3_every_iteration(km):
    """The headline workload at each of its 10 iterations, teacher-forced:
    labels of 2^14 seeded rows per iteration, the update and the inertia of
    the GPU's labels on every row, and the fit equal to the stepwise calls."""
    p = datagen.make("c3")
    _stats_ok(H.teacher_forced(km, p.X, p.C0, p.iters, sample=1 << 14, tag="c3", check_fit=True))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_c5_scaled_streamed_against_oracle(km):
    """The out-of-core workload at N = 2^22 (1 GiB of pinned fp16 rows, K =
    4,096, device slots of 1/16 of X: 16 chunks): first and last of 3
    iterations against the oracle, labels on 2^18 seeded rows."""
    p = datagen.make("c5", n=1 << 22)
    Xp = p.X[0].pin_memory()
    budget = Xp.numel() * Xp.element_size() // 8
    lab, C, J, _ = km.fit_streamed(Xp, p.C0[0].cuda(), p.iters, budget, history=True)
    _check_streamed_against_oracle(km, Xp, H.decode(p.X[0], "fp16"), p.C0[0], p.iters, budget, (lab, C, J),
                                   sample=1 << 18, tag="c5s")


@pytest.mark.parametrize("case", ["c1", "c4"])
def test_fit_graph_replays_match_direct_launches(km, case, monkeypatch):
    """kmeans_fit replays a captured HIP graph for a repeated argument list.
    Every replay, with other GPU work and host synchronisation in between, and
    with the input contents changed between calls, must equal direct launches
    bit for bit.  The batched case has B*K = 300 keys, so its sort is the
    one-pass segmented sort."""
    p = datagen.make(case, n=6000, k=100, batch=3, seed=11) if case == "c4" else datagen.make(case, n=20000, seed=11)
    X = (p.X if p.B > 1 else p.X[0]).cuda()
    C0 = (p.C0 if p.B > 1 else p.C0[0]).cuda()
    B = p.B
    iters = 4
    ws = torch.empty(km.workspace_bytes(p.N, p.D, p.K, B, X.dtype), dtype=torch.uint8, device="cuda")

    def direct(Xd, Cd):
        monkeypatch.setenv("FLASHKM_FIT_GRAPH", "0")
        r = km.fit(Xd, Cd, iters, history=True, ws=ws)
        torch.cuda.synchronize()
        monkeypatch.delenv("FLASHKM_FIT_GRAPH")
        return [t.clone() for t in r]

    ref = direct(X, C0)
    out = (torch.empty_like(ref[0]), torch.empty_like(ref[1]), torch.empty_like(ref[2]), torch.empty_like(ref[3]))
    for rep in range(3):
        got = km.fit(X, C0, iters, history=True, ws=ws, out=out)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"{case}: replay {rep} differs from direct launches"
        # unrelated eager work between replays (library kernels and torch ops)
        lab, _, _ = km.assign(X, C0, ws=ws)
        km.update(X, lab, C0, ws=ws)
        _ = (X.float().sum() + C0.sum()).item()
    # new contents in the same buffers: the replay reads them
    X.copy_(torch.flip(X, dims=[-2]))
    ref2 = direct(X, C0)
    got = km.fit(X, C0, iters, history=True, ws=ws, out=out)
    torch.cuda.synchronize()
    for a, b in zip(got, ref2):
        assert torch.equal(a, b), f"{case}: replay after an input change differs from direct launches"


@pytest.mark.parametrize("dtype,d", [("fp16", 128), ("fp32", 32), ("bf16", 64)])
def test_tune_and_every_config_agree(km, dtype, d, tmp_path):
    """kmeans_tune returns a compiled configuration and records it; every
    compiled configuration, forced through a tuning-table file, gives the same
    labels and distances bit for bit (and the same inertia up to the order of
    its fp64 partial sums)."""
    X, C0, _, _ = datagen.mixture(40_009, d, 60, dtype=dtype, center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=58, seed=d, k=211)
    X, C = X[0].cuda(), C0[0].cuda()
    pb, waves, ms = km.tune(X, C)
    compiled = km.assign_configs(X.dtype, d)
    assert (3, 8) in compiled and len(compiled) == 6   # rows of at most 256 bytes here: every configuration
    assert (pb, waves) in compiled and ms > 0
    dt = {"fp32": 0, "fp16": 1, "bf16": 2}[dtype]
    ref = None
    for c in compiled:
        f = tmp_path / f"t{c[0]}_{c[1]}.txt"
        f.write_text(f"{dt} {d} {X.shape[0]} 1 {C.shape[0]} {c[0]} {c[1]}\n")
        km.tune_load(str(f))
        lab, md, J = km.assign(X, C, want_min_d2=True)
        torch.cuda.synchronize()
        got = (lab.cpu(), md.cpu(), float(J[0]))
        if ref is None:
            ref = got
        else:
            assert torch.equal(got[0], ref[0]), f"{dtype} D={d}: labels differ for config {c}"
            assert torch.equal(got[1], ref[1]), f"{dtype} D={d}: distances differ for config {c}"
            assert abs(got[2] - ref[2]) <= 1e-12 * abs(ref[2]), f"{dtype} D={d}: inertia differs for config {c}"
    # the oracle agrees with the (shared) result
    Xd = H.decode(X.cpu(), dtype)
    H.check_assign(Xd, C.cpu().numpy(), ref[0].numpy(), ref[2], dtype, min_d2=ref[1].numpy(), tag=f"tune-{dtype}-{d}")


def _force_config(km, tmp_path, dtype, d, n, batch, k, cfg):
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[dtype]
    f = tmp_path / f"cfg_{dt}_{d}_{n}_{batch}_{k}_{cfg[0]}_{cfg[1]}.txt"
    f.write_text(f"{dt} {d} {n} {batch} {k} {cfg[0]} {cfg[1]}\n")
    km.tune_load(str(f))


def test_three_block_config_ragged_every_row(km, tmp_path):
    """The (3 point blocks, 8 waves) assignment that the built-in rule takes
    for long sweeps (the headline workload), forced on a ragged shape: 200,003
    points (a partial last job of 768 points), K = 300 (a full and a partial
    centroid tile), bf16, D = 128.  Every row against the oracle, and bit for
    bit against the (2, 8) configuration; then a teacher-forced iteration."""
    n, d, k = 200_003, 128, 300
    X, C0, _, _ = datagen.mixture(n, d, 150, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=0.5,
                                  weights=datagen.zipf_weights(150, 1.1), workload_code=66, seed=0, k=k)
    Xc, C = X.cuda(), C0.cuda()
    got = {}
    for cfg in [(3, 8), (2, 8)]:
        _force_config(km, tmp_path, torch.bfloat16, d, n, 1, k, cfg)
        lab, md, J = km.assign(Xc, C, want_min_d2=True)
        torch.cuda.synchronize()
        got[cfg] = (lab.cpu(), md.cpu(), float(J[0]))
    assert torch.equal(got[(3, 8)][0], got[(2, 8)][0]) and torch.equal(got[(3, 8)][1], got[(2, 8)][1])
    assert abs(got[(3, 8)][2] - got[(2, 8)][2]) <= 1e-12 * got[(2, 8)][2]
    Xd = H.decode(X[0], "bf16")
    rep = H.check_assign(Xd, C0[0].numpy(), got[(3, 8)][0][0].numpy(), got[(3, 8)][2], "bf16",
                         min_d2=got[(3, 8)][1][0].numpy(), tag="pb3")
    H.log(f"pb3 every row: near-ties excused {rep['excused']}")
    _force_config(km, tmp_path, torch.bfloat16, d, n, 1, k, (3, 8))
    _stats_ok(H.teacher_forced(km, X, C0, 2, tag="pb3-fit"))


def test_zero_rows_exact(km):
    """Rows x = 0 (every element): the near-tie tolerance 1e-5 ||x||^2 is zero
    there, so their labels must equal the oracle's exactly; their distance is
    ||c||^2 of the chosen centroid."""
    for dtype, d in [("bf16", 128), ("fp16", 64), ("fp32", 32)]:
        X, C0, _, _ = datagen.mixture(20_000, d, 40, dtype=dtype, center_dist="normal", center_scale=2.0,
                                      sigma=1.0, weights=None, workload_code=67, seed=d, k=97)
        X = X.clone()
        zero = np.arange(0, 20_000, 97)
        X[0, zero] = 0
        labels, md, J = km.assign(X.cuda(), C0.cuda(), want_min_d2=True)
        torch.cuda.synchronize()
        Xd = H.decode(X[0], dtype)
        Ch = oracle.round_to_format(C0[0].numpy().astype(np.float64), dtype)
        lab_o, dmin = oracle.assign(Xd[zero], Ch)
        assert np.array_equal(labels[0].cpu().numpy()[zero], lab_o), f"{dtype}: a zero row's label differs"
        assert np.allclose(md[0].cpu().numpy()[zero], dmin, rtol=1e-6, atol=0), f"{dtype}: zero-row distance"
        _stats_ok(H.teacher_forced(km, X, C0, 2, tag=f"zero-{dtype}"))


@pytest.mark.parametrize("k", [256, 257])
def test_resident_tile_switch(km, k):
    """K = 256 / 257 at 8 instances of 65,537 points (2,056 jobs of 256
    points): the built-in rule takes the resident-tile form with all K
    centroids in one 256-row tile at K = 256, and (2 blocks, 8 waves) with a
    second, one-row tile at K = 257.  Both against the oracle on every row."""
    X, C0, _, _ = datagen.mixture(65_537, 128, 64, dtype="fp16", center_dist="normal", center_scale=1.0, sigma=0.3,
                                  weights=None, workload_code=68, seed=k, k=k, batch=8)
    _stats_ok(H.teacher_forced(km, X, C0, 2, tag=f"res-K{k}"))


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", [8191, 8192])
def test_long_sweep_switch(km, k, tmp_path):
    """K = 8191 / 8192 at N = 3,145,729 (4,097 jobs of 768 points): the
    built-in rule takes (3 blocks, 8 waves) from K = 8192 and (2, 8) below.
    Labels on 2^15 seeded rows against the oracle, the update and inertia on
    every row, and the picked configuration bit for bit against the other."""
    n = 3_145_729
    X, C0, _, _ = datagen.mixture(n, 128, 4096, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=0.5,
                                  weights=datagen.zipf_weights(4096, 1.1), workload_code=69, seed=k, k=k)
    Xc, C = X.cuda(), C0.cuda()
    lab, md, J = km.assign(Xc, C, want_min_d2=True)
    other = (2, 8) if k == 8192 else (3, 8)
    _force_config(km, tmp_path, torch.bfloat16, 128, n, 1, k, other)
    lab2, md2, J2 = km.assign(Xc, C, want_min_d2=True)
    torch.cuda.synchronize()
    assert torch.equal(lab, lab2) and torch.equal(md, md2), f"K={k}: configurations disagree"
    assert abs(float(J[0]) - float(J2[0])) <= 1e-12 * float(J[0])
    Xd = [H.decode(X[0], "bf16")]
    H.check_step(km, Xc, Xd, C, "bf16", sample=1 << 15, rng=np.random.default_rng(k), tag=f"sweep-K{k}")


def test_k_equals_n_through_fit(km):
    """K = N distinct bf16 rows of D = 128 with C0 = X, through kmeans_fit:
    every row is its own cluster, so labels are the identity, the inertia is
    exactly 0 and every centroid stays its row."""
    X, _, _, _ = datagen.mixture(1500, 128, 1500, dtype="bf16", center_dist="normal", center_scale=3.0, sigma=1.0,
                                 weights=None, workload_code=70, seed=0)
    Xu = torch.unique(X[0].float(), dim=0)
    Xu = Xu[torch.randperm(Xu.shape[0], generator=torch.Generator().manual_seed(1))]
    Xb = Xu.to(torch.bfloat16)
    C0 = Xb.float()
    labels, C, J, hist = km.fit(Xb.cuda(), C0.cuda(), 3, history=True)
    torch.cuda.synchronize()
    assert torch.equal(labels.cpu(), torch.arange(Xb.shape[0], dtype=torch.int32))
    assert torch.equal(C.cpu(), C0) and float(J[0]) == 0.0 and float(hist.abs().max()) == 0.0


def test_fit_replay_follows_a_new_tuning_entry(km, tmp_path, monkeypatch):
    """A fit captured under one assignment configuration, then a tuning-table
    entry that selects another for the same shape: the next fit with the same
    arguments runs the new configuration.  Labels, centroids and inertia do
    not depend on the configuration, but the caller's workspace shows which
    one ran (each writes its own number of per-wave inertia partials), so the
    workspace is filled with a sentinel before every run and must equal, byte
    for byte, the workspace of direct launches of the configuration in force."""
    n, d, k, iters = 100_003, 64, 200, 3
    X, C0, _, _ = datagen.mixture(n, d, 50, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=71, seed=0, k=k)
    Xc, C = X[0].cuda(), C0[0].cuda()
    ws = torch.empty(km.workspace_bytes(n, d, k, 1, torch.float16), dtype=torch.uint8, device="cuda")
    out = (torch.empty(n, dtype=torch.int32, device="cuda"), torch.empty_like(C),
           torch.empty(1, dtype=torch.float64, device="cuda"), torch.empty((iters, 1), dtype=torch.float64,
                                                                          device="cuda"))

    def run(graph):
        ws.fill_(255)
        if not graph:
            monkeypatch.setenv("FLASHKM_FIT_GRAPH", "0")
        r = km.fit(Xc, C, iters, history=True, ws=ws, out=None if not graph else out)
        torch.cuda.synchronize()
        if not graph:
            monkeypatch.delenv("FLASHKM_FIT_GRAPH")
        return [t.clone() for t in r], ws.clone()

    res = {}
    for cfg in [(1, 4), (3, 8)]:
        _force_config(km, tmp_path, torch.float16, d, n, 1, k, cfg)
        ref, ws_ref = run(graph=False)
        got, ws_got = run(graph=True)       # same arguments every time
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"config {cfg}: the fit differs from direct launches of that configuration"
        assert torch.equal(ws_got, ws_ref), f"config {cfg}: the replayed fit ran another configuration"
        res[cfg] = ws_ref
    # the two configurations are distinguishable, so a stale replay would have failed above
    assert not torch.equal(res[(1, 4)], res[(3, 8)])


def test_resident_tile_batched_agrees(km, tmp_path):
    """The resident-tile forms of (1 block, 8 waves) and (2 blocks, 8 waves),
    taken when all K centroids fit one tile: a workgroup's contiguous run of
    jobs crosses instance boundaries here (3 instances of 100,003 points,
    about 4.6 jobs of 256 or 2.3 of 512 points per workgroup, the last job of
    each instance partial), so the tile is reloaded inside the run.  Labels
    and distances equal the plain (1, 4) configuration bit for bit, and the
    oracle."""
    n, d, k, batch = 100_003, 64, 200, 3
    X, C0, _, _ = datagen.mixture(n, d, 40, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=64, seed=1, k=k, batch=batch)
    X, C = X.cuda(), C0.cuda()
    ref = None
    for c in [(1, 8), (1, 4), (2, 8)]:
        f = tmp_path / f"r{c[0]}_{c[1]}.txt"
        f.write_text(f"2 {d} {n} {batch} {k} {c[0]} {c[1]}\n")
        km.tune_load(str(f))
        lab, md, J = km.assign(X, C, want_min_d2=True)
        torch.cuda.synchronize()
        got = (lab.cpu(), md.cpu(), J.cpu())
        if ref is None:
            ref = got
        else:
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"config {c} differs"
            assert torch.allclose(got[2], ref[2], rtol=1e-12, atol=0.0), f"config {c}: inertia differs"
    for b in range(batch):
        H.check_assign(H.decode(X[b].cpu(), "bf16"), C[b].cpu().numpy(), ref[0][b].numpy(), float(ref[2][b]), "bf16",
                       min_d2=ref[1][b].numpy(), tag=f"resident b={b}")


@pytest.mark.parametrize("pb", [1, 2])
def test_fit_with_resident_tile_equals_stepwise(km, tmp_path, pb):
    """A fit whose assignment runs a resident-tile form (one or two point
    blocks, forced through the tuning table for this shape): the captured and
    replayed fit equals the same iterations as stand-alone calls bit for bit."""
    n, d, k, batch, iters = 20_011, 64, 100, 3, 3
    X, C0, _, _ = datagen.mixture(n, d, 30, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                  weights=None, workload_code=65, seed=2, k=k, batch=batch)
    f = tmp_path / f"resident{pb}.txt"
    f.write_text(f"1 {d} {n} {batch} {k} {pb} 8\n")
    km.tune_load(str(f))
    Xc, C = X.cuda(), C0.cuda()
    Cs = C.clone()
    for t in range(iters):
        lab, _, J = km.assign(Xc, Cs)
        Cs, _ = km.update(Xc, lab, Cs)
    for rep in range(2):  # capture, then replay
        lab_f, C_f, J_f, _ = km.fit(Xc, C, iters, history=True)
        torch.cuda.synchronize()
        assert torch.equal(lab, lab_f) and torch.equal(Cs, C_f) and torch.equal(J, J_f), f"replay {rep} differs"


def _mixture(n, d, k, dtype, seed, batch=1, m=None):
    return datagen.mixture(n, d, m or max(2, k // 2), dtype=dtype, center_dist="normal", center_scale=2.0,
                           sigma=1.0, weights=None, workload_code=59, seed=seed, batch=batch, k=k)


@pytest.mark.parametrize("dtype,d,n,k,batch", [("bf16", 128, 20_011, 300, 1), ("fp16", 64, 9_001, 2, 2),
                                               ("fp32", 32, 30_000, 77, 1), ("bf16", 256, 5_003, 130, 3),
                                               ("fp16", 16, 12_345, 513, 1)])
def test_top2_matches_oracle(km, dtype, d, n, k, batch):
    """Two nearest centroids per point against the oracle: the GPU's pair has
    the true first and second smallest distances (up to the near-tie
    tolerance), its distances are the direct distances of its labels, and
    exact label mismatches are counted as near-ties."""
    X, C0, _, _ = _mixture(n, d, k, dtype, seed=d + k, batch=batch)
    lab2, d2 = km.assign_top2(X.cuda(), C0.cuda())
    torch.cuda.synchronize()
    lab2, d2 = lab2.cpu().numpy(), d2.cpu().numpy()
    mism = 0
    for b in range(batch):
        Xd = H.decode(X[b], dtype)
        Ch = oracle.round_to_format(C0[b].numpy().astype(np.float64), dtype)
        lo, do = oracle.assign_top2(Xd, Ch)
        g = lab2[b].astype(np.int64)
        assert np.all((g >= 0) & (g < k)) and np.all(g[:, 0] != g[:, 1])
        dg = np.stack([H.rowwise_sq_dist(Xd, Ch[g[:, j]]) for j in range(2)], axis=1)
        tol = H.TOL_TIE * np.einsum("ij,ij->i", Xd, Xd)
        assert np.all(np.abs(dg - do) <= tol[:, None] + 1e-30), f"top2 {dtype} D={d}: a pick is not a top-2 distance"
        assert np.all(np.abs(d2[b] - dg) <= 1e-5 * np.maximum(dg, 1e-3 * tol[:, None] / H.TOL_TIE) + 1e-30)
        mism += int(np.count_nonzero(g != lo))
    H.log(f"top2 {dtype} D={d} n={n} k={k} B={batch}: {mism} label entries differ, all within near-tie tolerance")


@pytest.mark.parametrize("dtype,d,n,k,sigma2,batch", [("bf16", 128, 20_011, 300, 2.0, 1),
                                                      ("fp16", 64, 9_001, 5, 0.5, 2),
                                                      ("fp32", 32, 30_000, 77, 20.0, 1),
                                                      ("bf16", 256, 5_003, 130, 8.0, 2),
                                                      ("fp16", 16, 12_345, 1, 1.0, 1)])
def test_soft_assign_matches_oracle(km, dtype, d, n, k, sigma2, batch):
    """Gaussian-mixture log density and most responsible component against
    the oracle, with per-instance log-weights.  A score error e (distance
    units) moves every a_k by e / (2 sigma2), so labels may differ only where
    the two best a_k are within tol_a = 1e-5 ||x||^2 / (2 sigma2) +
    1e-6 (1 + max|log w|); log densities agree within 2 tol_a + 1e-5 (1 + |L|)."""
    X, C0, _, _ = _mixture(n, d, k, dtype, seed=3 * d + k, batch=batch)
    lw = torch.randn(batch, k, generator=torch.Generator().manual_seed(k)) * 0.7
    lab, L, tot = km.assign_soft(X.cuda(), C0.cuda(), sigma2, log_w=lw.cuda())
    torch.cuda.synchronize()
    lab, L, tot = lab.cpu().numpy(), L.cpu().numpy().astype(np.float64), tot.cpu().numpy()
    near = 0
    for b in range(batch):
        Xd = H.decode(X[b], dtype)
        Ch = oracle.round_to_format(C0[b].numpy().astype(np.float64), dtype)
        lwb = lw[b].numpy().astype(np.float64)
        lo, Lo = oracle.soft_assign(Xd, Ch, lwb, sigma2)
        xx = np.einsum("ij,ij->i", Xd, Xd)
        tol_a = H.TOL_TIE * xx / (2 * sigma2) + 1e-6 * (1 + np.abs(lwb).max())
        bad = np.nonzero(lab[b] != lo)[0]
        if bad.size:
            A = lwb[None, :] - oracle.sq_dist_direct(Xd[bad], Ch) / (2 * sigma2)
            gap = A[np.arange(bad.size), lo[bad]] - A[np.arange(bad.size), lab[b][bad]]
            assert np.all(gap <= tol_a[bad]), f"soft {dtype} D={d}: label mismatch beyond near-ties"
            near += bad.size
        err = np.abs(L[b] - Lo)
        lim = 2 * tol_a + 1e-5 * (1 + np.abs(Lo))
        assert np.all(err <= lim), f"soft {dtype} D={d}: log density off by {err.max():.3e}"
        assert abs(tot[b] - Lo.sum()) <= lim.sum(), f"soft {dtype} D={d}: total {tot[b]} vs {Lo.sum()}"
    H.log(f"soft {dtype} D={d} n={n} k={k} s2={sigma2} B={batch}: {near} near-tie labels")


@pytest.mark.parametrize("dtype,d,n,k,sigma2,batch", [("bf16", 128, 20_011, 300, 100.0, 1),
                                                      ("fp16", 64, 9_001, 33, 50.0, 2),
                                                      ("fp32", 32, 30_000, 77, 20.0, 1),
                                                      ("bf16", 256, 5_003, 130, 200.0, 2),
                                                      ("fp16", 16, 12_345, 1, 10.0, 1)])
def test_gauss_sum_matches_oracle(km, dtype, d, n, k, sigma2, batch):
    """Signed-weight Gauss sums against the oracle.  A score error e moves each
    term's exponent by e / (2 sigma2), so the error bound is relative to
    S_i = sum_k |w_k| exp(-d_ik / (2 sigma2)): (tol_a + 5e-6) S_i with
    tol_a = 1e-5 ||x||^2 / (2 sigma2), plus 1e-30 sum|w| for fp32 underflow."""
    X, Y, _, _ = _mixture(n, d, k, dtype, seed=5 * d + k, batch=batch)
    w = torch.randn(batch, k, generator=torch.Generator().manual_seed(d + k))
    G, tot = km.gauss_sum(X.cuda(), Y.cuda(), w.cuda(), sigma2)
    torch.cuda.synchronize()
    G, tot = G.cpu().numpy().astype(np.float64), tot.cpu().numpy()
    worst = 0.0
    for b in range(batch):
        Xd = H.decode(X[b], dtype)
        Yh = oracle.round_to_format(Y[b].numpy().astype(np.float64), dtype)
        wb = w[b].numpy().astype(np.float64)
        Go = oracle.gauss_sum(Xd, Yh, wb, sigma2)
        S = oracle.gauss_sum(Xd, Yh, np.abs(wb), sigma2)
        tol_a = H.TOL_TIE * np.einsum("ij,ij->i", Xd, Xd) / (2 * sigma2)
        lim = (tol_a + 5e-6) * S + 1e-30 * np.abs(wb).sum()
        err = np.abs(G[b] - Go)
        assert np.all(err <= lim), f"gauss {dtype} D={d}: error {err.max():.3e} vs bound {lim[err.argmax()]:.3e}"
        assert abs(tot[b] - Go.sum()) <= lim.sum(), f"gauss {dtype} D={d}: total {tot[b]} vs {Go.sum()}"
        worst = max(worst, float(np.max(err / np.maximum(S, 1e-300))))
    H.log(f"gauss {dtype} D={d} n={n} k={k} s2={sigma2} B={batch}: max error / S = {worst:.1e}")


def _check_kpp(Xd, u, idx, eps, tag):
    """Teacher-forced validity of k-means++ picks: with D2 from the GPU's own
    earlier picks (oracle distances), pick j must sit in the inverse-CDF cell
    of u_j * sum(D2) up to the relative rounding eps of the GPU's fp32 D2."""
    n = Xd.shape[0]
    assert idx[0] == min(int(np.floor(u[0] * n)), n - 1), tag
    d2 = H.rowwise_sq_dist(Xd, np.broadcast_to(Xd[idx[0]], Xd.shape))
    for j in range(1, len(u)):
        cum = np.cumsum(d2)
        T = cum[-1]
        g = int(idx[j])
        if T > 0:
            t = u[j] * T
            lo = cum[g - 1] if g > 0 else 0.0
            assert d2[g] > 0 and cum[g] > t - eps * T and lo <= t + eps * T, (tag, j, g, lo, cum[g], t)
        else:
            assert g == min(int(np.floor(u[j] * n)), n - 1), (tag, j)
        d2 = np.minimum(d2, H.rowwise_sq_dist(Xd, np.broadcast_to(Xd[g], Xd.shape)))
    return d2


@pytest.mark.parametrize("dtype,d,n,k,batch", [("bf16", 128, 20_011, 64, 1), ("fp16", 64, 9_001, 33, 3),
                                               ("fp32", 32, 30_000, 20, 1), ("bf16", 256, 5_003, 17, 2),
                                               ("fp16", 16, 12_345, 48, 1)])
def test_seeding_matches_oracle(km, dtype, d, n, k, batch):
    X, _, _, _ = _mixture(n, d, k, dtype, seed=7 * d + k, batch=batch)
    u = torch.rand(batch, k, dtype=torch.float64, generator=torch.Generator().manual_seed(n))
    Xg, ug = X.cuda(), u.cuda()
    ridx, rC, _ = km.seed(Xg, ug, method="random")
    kidx, kC, kd2 = km.seed(Xg, ug, method="kmeans++", want_d2=True)
    torch.cuda.synchronize()
    exact = 0
    for b in range(batch):
        Xd = H.decode(X[b], dtype)
        ub = u[b].numpy()
        assert np.array_equal(ridx[b].cpu().numpy(), oracle.seed_random(n, ub)), "random seeding rows"
        assert np.array_equal(rC[b].cpu().numpy().astype(np.float64), Xd[ridx[b].cpu().numpy()])
        ki = kidx[b].cpu().numpy()
        assert np.array_equal(kC[b].cpu().numpy().astype(np.float64), Xd[ki]), "centroids are the picked rows"
        d2 = _check_kpp(Xd, ub, ki, 3e-5, f"kmeans++ {dtype} D={d} b={b}")
        got = kd2[b].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - d2) <= 1e-5 * d2 + 1e-30), "final D2"
        exact += int(np.count_nonzero(ki == oracle.kmeanspp(Xd, ub)[0]))
    H.log(f"seeding {dtype} D={d} n={n} k={k} B={batch}: {exact} of {batch * k} k-means++ picks equal the "
          f"free-running oracle's")


def test_seeding_identical_rows_falls_back_to_uniform(km):
    X = torch.full((1, 3000, 32), 0.5, dtype=torch.float16)
    u = torch.rand(1, 9, dtype=torch.float64, generator=torch.Generator().manual_seed(2))
    idx, C, d2 = km.seed(X.cuda(), u.cuda(), method="kmeans++", want_d2=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy()[0], oracle.seed_random(3000, u[0].numpy()))
    assert float(d2.abs().max()) == 0.0 and torch.all(C.cpu() == 0.5)


@pytest.mark.parametrize("case", ["zipf", "one_cluster"])
def test_update_large_problem_path(km, case):
    """Above 2^21 rows the update uses its large chunk and tile sizes: a ragged
    problem there, with skewed labels, against the oracle."""
    n, k, d = 2_100_003, 5_000, 32
    X, _, _, _ = datagen.mixture(n, d, 16, dtype="fp32", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=60, seed=1)
    if case == "zipf":
        lab = datagen.zipf_labels(n, k, 1.1, seed=2)
    else:
        lab = np.full((1, n), 2_718, dtype=np.int32)
    C_prev = torch.randn(1, k, d, generator=torch.Generator().manual_seed(3))
    C_new, counts = km.update(X.cuda(), torch.from_numpy(lab).cuda(), C_prev.cuda())
    torch.cuda.synchronize()
    err = H.check_update(H.decode(X[0], "fp32"), lab[0], C_prev[0].numpy(), C_new.cpu()[0].numpy(),
                         counts.cpu()[0].numpy(), k, tag=f"large-{case}")
    H.log(f"update large path {case}: centroid err {err:.2e}")


@pytest.mark.parametrize("case", ["packed_largest", "pairs_smallest", "two_low_digits"])
def test_update_two_pass_intermediate(km, case):
    """Two-pass sorts (keys of 12 to 16 bits) over fewer than 2^24 rows pass
    4-byte elements (high key byte and row) between the passes and restore
    the low byte from the position; from 2^24 rows the 8-byte pairs are kept.
    Against the oracle: the largest row count of the packed form and the
    smallest of the pair form (Zipf labels over K = 65,536), and labels whose
    low byte is only 0 or 255, so 254 of the 256 low digits are empty."""
    k, d = 65_536, 16
    n = {"packed_largest": (1 << 24) - 1, "pairs_smallest": 1 << 24, "two_low_digits": 300_007}[case]
    X, _, _, _ = datagen.mixture(n, d, 16, dtype="fp32", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=61, seed=1)
    if case == "two_low_digits":
        i = np.arange(n)
        lab = ((i * 7919 % 256) * 256 + np.where(i % 3 == 0, 255, 0)).astype(np.int32)[None]
    else:
        lab = datagen.zipf_labels(n, k, 1.1, seed=4)
    C_prev = torch.randn(1, k, d, generator=torch.Generator().manual_seed(3))
    C_new, counts = km.update(X.cuda(), torch.from_numpy(lab).cuda(), C_prev.cuda())
    torch.cuda.synchronize()
    err = H.check_update(H.decode(X[0], "fp32"), lab[0], C_prev[0].numpy(), C_new.cpu()[0].numpy(),
                         counts.cpu()[0].numpy(), k, tag=f"two-pass-{case}")
    H.log(f"update two-pass {case} n={n}: centroid err {err:.2e}")
