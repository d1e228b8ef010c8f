"""Seeded synthetic inputs for exact Lloyd k-means.

This module only draws inputs: Gaussian-mixture point sets X, initial
centroids C0 picked from the data, and (for update stress tests) label
vectors with skewed cluster sizes.  It contains none of the k-means
arithmetic, so both the fp64 oracle and the HIP path can consume its output
as plain data.

Recipe (the same for every workload):

* RNG: ``numpy.random.default_rng`` on children of
  ``SeedSequence([0x4B4D, workload_code, seed])``.  Child 0 draws the
  mixture centres, child 1 the initial-centroid rows, child 2+j draws row
  block j (component ids, then noise).  Row blocks are a fixed 2**18 rows,
  so the output does not depend on how many threads generate it.
* Per row: component id ``z ~ Categorical(w)`` (by inverse CDF of a uniform
  draw), noise ``eps ~ N(0, I_D)`` drawn in fp32, ``x = mu_z + sigma * eps``
  in fp32, then rounded to nearest-even into the storage dtype.
* ``C0 = X[idx]`` converted exactly to fp32, where ``idx`` is a seeded sample
  of K distinct rows (per instance when batched).

The five named workloads are the Flash-KMeans evaluation shapes used for
this library (the pages give no dataset, so these synthetic mixtures are the
workload): ``c1`` … ``c5``; ``scaled()`` shrinks any of them for tests while
keeping its distribution.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import hashlib
import os

import numpy as np
import torch

__all__ = [
    "Problem",
    "WORKLOADS",
    "make",
    "mixture",
    "zipf_weights",
    "zipf_labels",
    "uniform_labels",
    "digest",
]

_BLOCK_ROWS = 1 << 18
_TORCH_DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Problem:
    """One k-means problem instance batch.

    X: CPU tensor [B, N, D] in the storage dtype (fp32 / fp16 / bf16).
    C0: CPU fp32 tensor [B, K, D].
    comp: int32 numpy array [B, N] of the true mixture component of each row.
    """

    name: str
    X: torch.Tensor
    C0: torch.Tensor
    K: int
    iters: int
    dtype: str
    comp: np.ndarray
    centers: np.ndarray
    sigma: float

    @property
    def B(self) -> int:
        return int(self.X.shape[0])

    @property
    def N(self) -> int:
        return int(self.X.shape[1])

    @property
    def D(self) -> int:
        return int(self.X.shape[2])


def zipf_weights(m: int, s: float) -> np.ndarray:
    """Finite Zipf law over ranks 1..m: w_r proportional to r**-s (fp64, sums to 1)."""
    r = np.arange(1, m + 1, dtype=np.float64)
    w = r ** (-float(s))
    return w / w.sum()


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen_block(seed_seq, rows, centers, cdf, sigma, out_np_f32):
    rng = np.random.default_rng(seed_seq)
    u = rng.random(rows)
    z = np.searchsorted(cdf, u, side="right").astype(np.int64)
    np.minimum(z, centers.shape[0] - 1, out=z)
    eps = rng.standard_normal((rows, centers.shape[1]), dtype=np.float32)
    eps *= np.float32(sigma)
    eps += centers[z]
    out_np_f32[...] = eps
    return z.astype(np.int32)


def mixture(
    n: int,
    d: int,
    m: int,
    *,
    dtype: str,
    center_dist: str,
    center_scale: float,
    sigma: float,
    weights: np.ndarray | None,
    workload_code: int,
    seed: int,
    batch: int = 1,
    k: int | None = None,
    init: str = "sample",
):
    """Draw ``batch`` independent mixtures of ``m`` Gaussian components.

    center_dist: "uniform" (centres U[-center_scale, center_scale]^d) or
    "normal" (centres N(0, center_scale**2 I)).
    Returns (X [B,N,D] torch in ``dtype``, C0 [B,K,D] fp32 torch, comp, centers).
    """
    if dtype not in _TORCH_DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_TORCH_DTYPES)}")
    root = np.random.SeedSequence([0x4B4D, int(workload_code), int(seed)])
    nblk = (n + _BLOCK_ROWS - 1) // _BLOCK_ROWS
    kids = root.spawn(2 + batch * nblk)
    crng = np.random.default_rng(kids[0])
    if center_dist == "uniform":
        centers = crng.uniform(-center_scale, center_scale, size=(batch, m, d))
    elif center_dist == "normal":
        centers = crng.standard_normal((batch, m, d)) * center_scale
    else:
        raise ValueError(center_dist)
    centers = centers.astype(np.float32)
    w = np.full(m, 1.0 / m) if weights is None else np.asarray(weights, np.float64)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]

    tdt = _TORCH_DTYPES[dtype]
    X = torch.empty((batch, n, d), dtype=tdt)
    comp = np.empty((batch, n), dtype=np.int32)

    def work(b, j):
        r0 = j * _BLOCK_ROWS
        rows = min(_BLOCK_ROWS, n - r0)
        buf = np.empty((rows, d), dtype=np.float32)
        comp[b, r0:r0 + rows] = _gen_block(kids[2 + b * nblk + j], rows, centers[b], cdf, sigma, buf)
        X[b, r0:r0 + rows] = torch.from_numpy(buf).to(tdt)

    jobs = [(b, j) for b in range(batch) for j in range(nblk)]
    if len(jobs) == 1:
        work(*jobs[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda bj: work(*bj), jobs))

    C0 = None
    if k is not None:
        irng = np.random.default_rng(kids[1])
        C0 = torch.empty((batch, k, d), dtype=torch.float32)
        for b in range(batch):
            if init == "permutation":
                idx = irng.permutation(n)[:k]
            else:
                idx = irng.choice(n, size=k, replace=False)
            C0[b] = X[b, torch.from_numpy(np.sort(idx) if init == "sorted" else idx)].to(torch.float32)
    return X, C0, comp, centers


# name -> (description, builder kwargs).  Sizes are the full evaluation shapes.
WORKLOADS = {
    "c1": dict(
        desc="N=65,536 D=32 fp32, 64-component mixture, centres U[-5,5]^D, sigma 1, K=64, 10 iterations",
        n=65536, d=32, m=64, dtype="fp32", center_dist="uniform", center_scale=5.0,
        sigma=1.0, zipf=None, k=64, iters=10, batch=1, init="permutation", code=1),
    "c2": dict(
        desc="N=1,048,576 D=128 fp16, 1,024-component mixture, centres N(0,4I), sigma 1, K=1,024, 20 iterations",
        n=1 << 20, d=128, m=1024, dtype="fp16", center_dist="normal", center_scale=2.0,
        sigma=1.0, zipf=None, k=1024, iters=20, batch=1, init="sample", code=2),
    "c3": dict(
        desc="N=8,388,608 D=128 bf16, 65,536-component mixture with Zipf(1.1) weights, centres N(0,4I), "
             "sigma 0.5, K=65,536, 10 iterations",
        n=1 << 23, d=128, m=65536, dtype="bf16", center_dist="normal", center_scale=2.0,
        sigma=0.5, zipf=1.1, k=65536, iters=10, batch=1, init="sample", code=3),
    "c4": dict(
        desc="B=64 instances x N=16,384 D=128 fp16, 256-component mixtures, centres N(0,I), sigma 0.3, "
             "K=256 per instance, 8 iterations",
        n=16384, d=128, m=256, dtype="fp16", center_dist="normal", center_scale=1.0,
        sigma=0.3, zipf=None, k=256, iters=8, batch=64, init="sample", code=4),
    "c5": dict(
        desc="N=1,000,000,000 D=128 fp16 host-resident, 4,096-component mixture, centres N(0,4I), sigma 1, "
             "K=4,096, 3 iterations",
        n=1_000_000_000, d=128, m=4096, dtype="fp16", center_dist="normal", center_scale=2.0,
        sigma=1.0, zipf=None, k=4096, iters=3, batch=1, init="sample", code=5),
}


def make(name: str, *, n: int | None = None, k: int | None = None, m: int | None = None,
         batch: int | None = None, d: int | None = None, iters: int | None = None,
         seed: int = 0) -> Problem:
    """Build a named workload, optionally scaled down (n rows, k centroids,
    m mixture components, batch instances, d dims).  When only ``k`` is given
    the mixture keeps ``m = k`` components, matching the full configs."""
    w = dict(WORKLOADS[name])
    n = w["n"] if n is None else int(n)
    k = w["k"] if k is None else int(k)
    if m is None:
        m = w["m"] if k == w["k"] else k
    batch = w["batch"] if batch is None else int(batch)
    d = w["d"] if d is None else int(d)
    iters = w["iters"] if iters is None else int(iters)
    weights = zipf_weights(m, w["zipf"]) if w["zipf"] else None
    X, C0, comp, centers = mixture(
        n, d, m, dtype=w["dtype"], center_dist=w["center_dist"], center_scale=w["center_scale"],
        sigma=w["sigma"], weights=weights, workload_code=w["code"], seed=seed, batch=batch,
        k=k, init=w["init"])
    return Problem(name=name, X=X, C0=C0, K=k, iters=iters, dtype=w["dtype"], comp=comp,
                   centers=centers, sigma=w["sigma"])


def zipf_labels(n: int, k: int, s: float = 1.1, *, seed: int = 0, batch: int = 1) -> np.ndarray:
    """Labels [batch, n] int32 drawn i.i.d. from the finite Zipf(s) law over k
    clusters, with the ranks shuffled over cluster ids so the hot cluster is
    not always id 0."""
    rng = np.random.default_rng(np.random.SeedSequence([0x4B4D, 0x21F, int(seed)]))
    cdf = np.cumsum(zipf_weights(k, s))
    cdf /= cdf[-1]
    perm = rng.permutation(k).astype(np.int32)
    out = np.empty((batch, n), dtype=np.int32)
    for b in range(batch):
        r = np.searchsorted(cdf, rng.random(n), side="right")
        np.minimum(r, k - 1, out=r)
        out[b] = perm[r]
    return out


def uniform_labels(n: int, k: int, *, seed: int = 0, batch: int = 1) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([0x4B4D, 0x3A1, int(seed)]))
    return rng.integers(0, k, size=(batch, n), dtype=np.int32)


def digest(*tensors) -> str:
    """SHA-256 over the raw bytes of the given tensors / arrays."""
    h = hashlib.sha256()
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype in (torch.bfloat16, torch.float16):
                t = t.view(torch.int16)
            t = t.numpy()
        h.update(np.ascontiguousarray(t).tobytes())
    return h.hexdigest()
