"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Every mutant is a plausible slip — a dropped term, a wrong sign or tie rule,
an off-by-one, a wrong divisor, a skipped rounding — applied to the oracle
with monkeypatch, so the real oracle is untouched.
"""

import numpy as np
import pytest

import oracle.fp64 as L
from tests import oracle_pins as P

_real_assign = L.assign
_real_update = L.update
_real_round = L.round_to_format
_real_decode = L.decode
_real_lloyd = L.lloyd


def _assign_highest_tie(X, Chat, **kw):
    D = L.sq_dist_direct(X, Chat)
    lab = D.shape[1] - 1 - np.argmin(D[:, ::-1], axis=1)
    return lab, D[np.arange(D.shape[0]), lab]


def _assign_no_cnorm(X, Chat, **kw):
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    lab = np.argmin(-2.0 * X @ Chat.T, axis=1)        # dropped ||c||^2
    return lab, ((X - Chat[lab]) ** 2).sum(1)


def _assign_sign(X, Chat, **kw):
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    D = (X * X).sum(1)[:, None] + 2.0 * X @ Chat.T + (Chat * Chat).sum(1)[None]   # wrong sign
    lab = np.argmin(D, axis=1)
    return lab, ((X - Chat[lab]) ** 2).sum(1)


def _assign_transposed_dim(X, Chat, **kw):
    X = np.asarray(X, np.float64)
    Chat = np.asarray(Chat, np.float64)
    return _real_assign(X, Chat[:, ::-1])                 # dims reversed on one operand


def _update_empty_zero(X, labels, C_prev, k):
    C, n = _real_update(X, labels, C_prev, k)
    C[n == 0] = 0.0
    return C, n


def _update_div_n(X, labels, C_prev, k):
    C, n = _real_update(X, labels, C_prev, k)
    nz = n > 0
    C[nz] *= n[nz, None] / max(1, len(labels))
    return C, n


def _update_offbyone(X, labels, C_prev, k):
    return _real_update(X, np.roll(np.asarray(labels), 1), C_prev, k)


def _round_trunc(x, fmt):
    x = np.asarray(x, np.float64)
    spec = L.FORMATS[fmt]
    if spec is None:
        return x.copy()
    p, emin, _ = spec
    _, e = np.frexp(x)
    q = np.maximum(e - 1, emin) - p + 1
    return np.ldexp(np.trunc(np.ldexp(x, -q)), q)


def _round_half_away(x, fmt):
    x = np.asarray(x, np.float64)
    spec = L.FORMATS[fmt]
    if spec is None:
        return x.copy()
    p, emin, _ = spec
    _, e = np.frexp(x)
    q = np.maximum(e - 1, emin) - p + 1
    s = np.ldexp(x, -q)
    return np.ldexp(np.sign(s) * np.floor(np.abs(s) + 0.5), q)


def _round_identity(x, fmt):
    return np.asarray(x, np.float64).copy()


def _decode_bad_shift(a, fmt):
    a = np.asarray(a)
    if fmt == "bf16":
        return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _real_decode(a, fmt)


def _lloyd_post_labels(X, fmt, C0, iters):
    out = _real_lloyd(X, fmt, C0, iters)
    lab, dmin = _real_assign(X, _real_round(out["C"], fmt))   # extra assignment after the last update
    out["labels"] = lab
    out["inertia"] = L.inertia(dmin)
    return out


def _lloyd_unrounded_inertia(X, fmt, C0, iters):
    out = _real_lloyd(X, fmt, C0, iters)
    C = np.asarray(C0, np.float64)
    hist = []
    for _ in range(iters):
        lab, _ = _real_assign(X, _real_round(C, fmt))
        hist.append(L.inertia(((np.asarray(X, np.float64) - C[lab]) ** 2).sum(1)))
        C, _ = _real_update(X, lab, C, C.shape[0])
    out["history"] = hist
    out["inertia"] = hist[-1]
    return out


_real_top2 = L.assign_top2
_real_soft = L.soft_assign


def _top2_high_tie(X, Chat):
    Dm = L.sq_dist_direct(X, Chat)
    k = Dm.shape[1]
    order = (k - 1 - np.argsort(Dm[:, ::-1], axis=1, kind="stable"))[:, :2]   # ties to the higher index
    return order, np.take_along_axis(Dm, order, axis=1)


def _top2_second_is_third(X, Chat):
    Dm = L.sq_dist_direct(X, Chat)
    order = np.argsort(Dm, axis=1, kind="stable")[:, [0, 2 if Dm.shape[1] > 2 else 1]]   # off by one
    return order, np.take_along_axis(Dm, order, axis=1)


def _soft_no_shift(X, Chat, log_w, sigma2):
    k = np.asarray(Chat).shape[0]
    lw = np.zeros(k) if log_w is None else np.asarray(log_w, np.float64)
    A = lw[None, :] - L.sq_dist_direct(X, Chat) / (2.0 * sigma2)
    with np.errstate(divide="ignore"):
        return A.argmax(axis=1), np.log(np.exp(A).sum(axis=1))    # no maximum subtracted


def _soft_no_half(X, Chat, log_w, sigma2):
    return _real_soft(X, Chat, log_w, sigma2 / 2.0)                # d / sigma2 instead of d / (2 sigma2)


def _soft_weight_sign(X, Chat, log_w, sigma2):
    return _real_soft(X, Chat, None if log_w is None else -np.asarray(log_w), sigma2)


def _soft_mode_last(X, Chat, log_w, sigma2):
    k = np.asarray(Chat).shape[0]
    lab, Lx = _real_soft(X, Chat, log_w, sigma2)
    lw = np.zeros(k) if log_w is None else np.asarray(log_w, np.float64)
    A = lw[None, :] - L.sq_dist_direct(X, Chat) / (2.0 * sigma2)
    return k - 1 - A[:, ::-1].argmax(axis=1), Lx                    # ties to the highest index


_real_gauss = L.gauss_sum


def _gauss_no_half(X, Y, w, sigma2):
    return _real_gauss(X, Y, w, sigma2 / 2.0)                       # exp(-d / s2)


def _gauss_unweighted(X, Y, w, sigma2):
    return _real_gauss(X, Y, np.ones_like(np.asarray(w, np.float64)), sigma2)


def _gauss_sign(X, Y, w, sigma2):
    Dm = L.sq_dist_direct(X, Y)
    with np.errstate(over="ignore"):
        return np.exp(Dm / (2.0 * sigma2)) @ np.asarray(w, np.float64)   # wrong sign in the exponent


def _gauss_weight_shift(X, Y, w, sigma2):
    return _real_gauss(X, Y, np.roll(np.asarray(w, np.float64), 1), sigma2)   # weights off by one source


_real_kpp = L.kmeanspp


def _kpp_left(X, u):
    X = np.asarray(X, np.float64)
    u = np.asarray(u, np.float64)
    n = X.shape[0]
    idx = [min(int(np.floor(u[0] * n)), n - 1)]
    d2 = ((X - X[idx[0]]) ** 2).sum(1)
    for j in range(1, len(u)):
        cum = np.cumsum(d2)
        idx.append(min(int(np.searchsorted(cum, u[j] * cum[-1], side="left")), n - 1) if cum[-1] > 0
                   else min(int(np.floor(u[j] * n)), n - 1))     # >= instead of >
        d2 = np.minimum(d2, ((X - X[idx[-1]]) ** 2).sum(1))
    return np.array(idx), d2


def _kpp_dist_not_squared(X, u):
    X = np.asarray(X, np.float64)
    u = np.asarray(u, np.float64)
    n = X.shape[0]
    idx = [min(int(np.floor(u[0] * n)), n - 1)]
    d = np.sqrt(((X - X[idx[0]]) ** 2).sum(1))
    for j in range(1, len(u)):
        cum = np.cumsum(d)                                          # D instead of D^2
        idx.append(min(int(np.searchsorted(cum, u[j] * cum[-1], side="right")), n - 1) if cum[-1] > 0
                   else min(int(np.floor(u[j] * n)), n - 1))
        d = np.minimum(d, np.sqrt(((X - X[idx[-1]]) ** 2).sum(1)))
    return np.array(idx), d * d


def _kpp_first_center_only(X, u):
    X = np.asarray(X, np.float64)
    u = np.asarray(u, np.float64)
    n = X.shape[0]
    idx = [min(int(np.floor(u[0] * n)), n - 1)]
    d2 = ((X - X[idx[0]]) ** 2).sum(1)
    for j in range(1, len(u)):                                     # D2 never updated
        cum = np.cumsum(d2)
        idx.append(min(int(np.searchsorted(cum, u[j] * cum[-1], side="right")), n - 1))
    return np.array(idx), d2


def _seed_round(n, u):
    return np.minimum(np.round(np.asarray(u, np.float64) * n).astype(np.int64), n - 1)


MUTANTS = {
    "kpp_left": ("kmeanspp", _kpp_left),
    "kpp_dist_not_squared": ("kmeanspp", _kpp_dist_not_squared),
    "kpp_first_center_only": ("kmeanspp", _kpp_first_center_only),
    "seed_round": ("seed_random", _seed_round),
    "gauss_no_half": ("gauss_sum", _gauss_no_half),
    "gauss_unweighted": ("gauss_sum", _gauss_unweighted),
    "gauss_sign": ("gauss_sum", _gauss_sign),
    "gauss_weight_shift": ("gauss_sum", _gauss_weight_shift),
    "top2_high_tie": ("assign_top2", _top2_high_tie),
    "top2_second_is_third": ("assign_top2", _top2_second_is_third),
    "soft_no_shift": ("soft_assign", _soft_no_shift),
    "soft_no_half": ("soft_assign", _soft_no_half),
    "soft_weight_sign": ("soft_assign", _soft_weight_sign),
    "soft_mode_last": ("soft_assign", _soft_mode_last),
    "assign_highest_tie": ("assign", _assign_highest_tie),
    "assign_no_cnorm": ("assign", _assign_no_cnorm),
    "assign_sign": ("assign", _assign_sign),
    "assign_transposed_dim": ("assign", _assign_transposed_dim),
    "update_empty_zero": ("update", _update_empty_zero),
    "update_div_n": ("update", _update_div_n),
    "update_offbyone": ("update", _update_offbyone),
    "round_trunc": ("round_to_format", _round_trunc),
    "round_half_away": ("round_to_format", _round_half_away),
    "round_identity": ("round_to_format", _round_identity),
    "decode_bad_shift": ("decode", _decode_bad_shift),
    "lloyd_post_labels": ("lloyd", _lloyd_post_labels),
    "lloyd_unrounded_inertia": ("lloyd", _lloyd_unrounded_inertia),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(L, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(L)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
