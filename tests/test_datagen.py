"""Seeded input generator: determinism, shapes and distribution (CPU only)."""

import numpy as np
import torch

import datagen


def test_deterministic_and_shapes():
    a = datagen.make("c2", n=5000, k=64)
    b = datagen.make("c2", n=5000, k=64)
    assert a.X.shape == (1, 5000, 128) and a.X.dtype == torch.float16
    assert a.C0.shape == (1, 64, 128) and a.C0.dtype == torch.float32
    assert datagen.digest(a.X, a.C0) == datagen.digest(b.X, b.C0)
    c = datagen.make("c2", n=5000, k=64, seed=1)
    assert datagen.digest(a.X) != datagen.digest(c.X)


def test_init_rows_come_from_data_and_are_distinct():
    p = datagen.make("c4", n=2048, k=32, batch=3)
    assert p.X.shape == (3, 2048, 128)
    for b in range(3):
        X = p.X[b].to(torch.float32)
        C = p.C0[b]
        # every initial centroid is exactly one of the rows of its own instance
        hit = (X[None, :, :] == C[:, None, :]).all(dim=2).any(dim=1)
        assert bool(hit.all())
        assert len({tuple(r.tolist()) for r in C}) == 32


def test_block_independence_of_thread_count(monkeypatch):
    a = datagen.make("c3", n=300_000, k=256)
    monkeypatch.setattr(datagen, "_threads", lambda: 1)
    b = datagen.make("c3", n=300_000, k=256)
    assert datagen.digest(a.X) == datagen.digest(b.X)
    assert a.X.dtype == torch.bfloat16


def test_zipf_weights_and_labels():
    w = datagen.zipf_weights(65536, 1.1)
    assert abs(w.sum() - 1) < 1e-12 and np.all(np.diff(w) < 0)
    assert abs(w[0] - 0.137) < 0.002          # top component ~13.7% of rows
    lab = datagen.zipf_labels(1 << 20, 65536, seed=2)
    assert lab.shape == (1, 1 << 20) and lab.min() >= 0 and lab.max() < 65536
    cnt = np.bincount(lab[0], minlength=65536)
    assert abs(cnt.max() / lab.size - w[0]) < 0.005


def test_mixture_statistics():
    p = datagen.make("c1", n=65536, k=64)
    X = p.X[0].numpy().astype(np.float64)
    resid = X - p.centers[0][p.comp[0]]
    assert abs(resid.std() - 1.0) < 0.01 and abs(resid.mean()) < 0.01
    assert p.centers.min() >= -5 and p.centers.max() <= 5
