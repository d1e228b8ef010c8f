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
