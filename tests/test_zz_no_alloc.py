"""The allocation-free assignment entry point (kmeans_assign_noalloc, scratch
in the library's static device array) against kmeans_assign (caller
workspace) through the C ABI: two calls in a row, the second on a smaller
input, each bit for bit equal to the workspace entry point, and the oracle
agreeing on the first.  No device memory is allocated by the call."""

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


def _one(km, X, C):
    B = X.shape[0] if X.dim() == 3 else 1
    lab = torch.empty(X.shape[:-1], dtype=torch.int32, device="cuda")
    md = torch.empty(X.shape[:-1], dtype=torch.float32, device="cuda")
    J = torch.empty(B, dtype=torch.float64, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    km.assign_noalloc(X, C, labels=lab, inertia=J, min_d2=md)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before        # nothing allocated through torch
    ref = km.assign(X, C, want_min_d2=True)
    torch.cuda.synchronize()
    assert torch.equal(lab, ref[0]), "labels differ from kmeans_assign"
    assert torch.equal(md, ref[1]), "distances differ from kmeans_assign"
    assert torch.equal(J, ref[2]), "inertia differs from kmeans_assign"
    return lab, md, J


def test_noalloc_assign_equals_workspace_assign_twice(km):
    # first call: bf16, D = 128, several centroid tiles and a ragged last job
    X1, C1, _, _ = datagen.mixture(50_003, 128, 500, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=0.5,
                                   weights=None, workload_code=72, seed=0, k=1000)
    lab1, md1, J1 = _one(km, X1[0].cuda(), C1[0].cuda())
    Xd = H.decode(X1[0], "bf16")
    rep = H.check_assign(Xd, C1[0].numpy(), lab1.cpu().numpy(), float(J1[0]), "bf16", min_d2=md1.cpu().numpy(),
                         tag="noalloc")
    H.log(f"noalloc first call: near-ties excused {rep['excused']}")
    # second call, smaller and batched: the scratch still holds the first
    # call's (larger) contents, which must not leak into this result
    X2, C2, _, _ = datagen.mixture(3_001, 64, 40, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                   weights=None, workload_code=73, seed=1, k=77, batch=2)
    lab2, md2, J2 = _one(km, X2.cuda(), C2.cuda())
    for b in range(2):
        H.check_assign(H.decode(X2[b], "fp16"), C2[b].numpy(), lab2[b].cpu().numpy(), float(J2[b]), "fp16",
                       min_d2=md2[b].cpu().numpy(), tag=f"noalloc-2 b{b}")


def test_noalloc_assign_rejects_oversized_shapes(km):
    X = torch.zeros(70_000, 256, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(65_537, 256, device="cuda")
    lab = torch.empty(70_000, dtype=torch.int32, device="cuda")
    J = torch.empty(1, dtype=torch.float64, device="cuda")
    with pytest.raises(km.KMeansError) as e:
        km.assign_noalloc(X, C, labels=lab, inertia=J)
    assert e.value.status == 3


def test_noalloc_assign_replays_in_a_captured_graph(km):
    """A caller under graph capture: the allocation-free assignment captured
    into a torch CUDA graph (after an eager call has set the library up on
    this device: scratch address, grid query) and replayed three times, the
    outputs cleared before each replay and other eager work (a workspace
    assignment of another shape) plus a synchronisation between replays.
    Every replay equals the eager call bit for bit."""
    X, C, _, _ = datagen.mixture(20_011, 64, 40, dtype="bf16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                 weights=None, workload_code=74, seed=2, k=300)
    X, C = X[0].cuda(), C[0].cuda()
    lab = torch.empty(X.shape[0], dtype=torch.int32, device="cuda")
    md = torch.empty(X.shape[0], dtype=torch.float32, device="cuda")
    J = torch.empty(1, dtype=torch.float64, device="cuda")
    km.assign_noalloc(X, C, labels=lab, inertia=J, min_d2=md)
    torch.cuda.synchronize()
    ref = (lab.clone(), md.clone(), J.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch asks before a capture
        km.assign_noalloc(X, C, labels=lab, inertia=J, min_d2=md)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        km.assign_noalloc(X, C, labels=lab, inertia=J, min_d2=md)
    torch.cuda.synchronize()
    Xo, Co, _, _ = datagen.mixture(9_001, 128, 30, dtype="fp16", center_dist="normal", center_scale=2.0, sigma=1.0,
                                   weights=None, workload_code=75, seed=3, k=500)
    Xo, Co = Xo[0].cuda(), Co[0].cuda()
    for r in range(3):
        lab.fill_(-1)
        md.fill_(-1.0)
        J.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lab, ref[0]), f"replay {r}: labels differ from the eager call"
        assert torch.equal(md, ref[1]), f"replay {r}: distances differ from the eager call"
        assert torch.equal(J, ref[2]), f"replay {r}: inertia differs from the eager call"
        km.assign(Xo, Co)
        torch.cuda.synchronize()
