"""Pins of the oracle's Block AttnRes read-out (softmax over the blocks of w . norm(V_n), then
the weighted sum of the blocks), checked on the CPU.

What fixes the values: closed forms (one block gives that block; w = 0 gives the mean of the
blocks and lse = log n; equal blocks give that block), the limit of a dominant score (the read-out
picks the block the query points to), scale covariance (norm(cV) = norm(V) with eps = 0, so
h(cV) = c h(V)), invariance under reordering the blocks, explicit loops with the math module on
tiny shapes, and the online-softmax merge of the two-phase inference (yeyulingfeng page, AttnRes
section): combining (h, lse) of the stored blocks with one more block gives the read-out over all.
Each plausible mistake below must fail at least one pin.
"""
import math

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(930932)


class Impl:
    def __init__(self, attnres=None, lse=None):
        self.attnres = attnres or oracle.attnres
        self.lse = lse or oracle.attnres_lse


def pin_one_block(impl):
    V = RNG.standard_normal((1, 4, 6))
    w = RNG.standard_normal(6)
    lg = oracle.rms_norm(V, 1e-6)[0] @ w
    return float(max(np.max(np.abs(impl.attnres(V, w, 1e-6) - V[0])), np.max(np.abs(impl.lse(V, w, 1e-6) - lg))))


def pin_zero_query_is_mean(impl):
    V = RNG.standard_normal((5, 3, 8))
    h = impl.attnres(V, np.zeros(8), 1e-6)
    return float(max(np.max(np.abs(h - V.mean(axis=0))), np.max(np.abs(impl.lse(V, np.zeros(8), 1e-6) - math.log(5)))))


def pin_equal_blocks(impl):
    U = RNG.standard_normal((1, 3, 8))
    V = np.repeat(U, 4, axis=0)
    return float(np.max(np.abs(impl.attnres(V, RNG.standard_normal(8), 1e-6) - U[0])))


def pin_dominant_score_picks_block(impl):
    # blocks c_n e_n: norm gives 2 e_n (d = 4), so the scores are 2 w_n; w = 30 e_2 picks block 2
    V = np.zeros((4, 1, 4))
    for n in range(4):
        V[n, 0, n] = 1.0 + n
    w = np.zeros(4)
    w[2] = 30.0
    return float(np.max(np.abs(impl.attnres(V, w, 0.0) - V[2])))


def pin_scale_covariance(impl):
    V = RNG.standard_normal((3, 4, 8))
    w = RNG.standard_normal(8)
    return float(np.max(np.abs(impl.attnres(3.5 * V, w, 0.0) - 3.5 * impl.attnres(V, w, 0.0))))


def pin_block_order(impl):
    V = RNG.standard_normal((4, 3, 8))
    w = RNG.standard_normal(8)
    p = [2, 0, 3, 1]
    return float(np.max(np.abs(impl.attnres(V[p], w, 1e-6) - impl.attnres(V, w, 1e-6))))


def pin_loops(impl):
    n, T, d, eps = 3, 2, 4, 1e-6
    V = RNG.standard_normal((n, T, d))
    w = RNG.standard_normal(d)
    h0 = np.zeros((T, d))
    lse0 = np.zeros(T)
    for t in range(T):
        sc = []
        for b in range(n):
            ms = sum(V[b, t, c] ** 2 for c in range(d)) / d
            sc.append(sum(w[c] * V[b, t, c] / math.sqrt(ms + eps) for c in range(d)))
        z = sum(math.exp(s) for s in sc)
        lse0[t] = math.log(z)
        for c in range(d):
            h0[t, c] = sum(math.exp(sc[b]) / z * V[b, t, c] for b in range(n))
    return float(max(np.max(np.abs(impl.attnres(V, w, eps) - h0)), np.max(np.abs(impl.lse(V, w, eps) - lse0))))


def pin_online_merge(impl):
    n, T, d, eps = 5, 6, 16, 1e-6
    V = RNG.standard_normal((n, T, d)) * RNG.uniform(0.5, 3.0, (n, T, 1))
    w = RNG.standard_normal(d) * 2.0
    hist, part = V[:-1], V[-1:]
    oh, lh = impl.attnres(hist, w, eps), impl.lse(hist, w, eps)
    lp = impl.lse(part, w, eps)                       # one block: its own score
    m = np.maximum(lh, lp)
    a, b = np.exp(lh - m), np.exp(lp - m)
    merged = (a[:, None] * oh + b[:, None] * part[0]) / (a + b)[:, None]
    return float(max(np.max(np.abs(merged - impl.attnres(V, w, eps))),
                     np.max(np.abs(m + np.log(a + b) - impl.lse(V, w, eps)))))


PINS = [(pin_one_block, 1e-13), (pin_zero_query_is_mean, 1e-13), (pin_equal_blocks, 1e-13),
        (pin_dominant_score_picks_block, 1e-20), (pin_scale_covariance, 1e-12), (pin_block_order, 1e-13),
        (pin_loops, 1e-12), (pin_online_merge, 1e-12)]


@pytest.mark.parametrize("pin,tol", PINS, ids=[p.__name__ for p, _ in PINS])
def test_oracle_attnres_pin(pin, tol):
    assert pin(Impl()) <= tol


def _softmax(lg, axis):
    a = np.exp(lg - lg.max(axis=axis, keepdims=True))
    return a / a.sum(axis=axis, keepdims=True)


def _mix(weight_fn):
    def f(V, w, eps):
        V = np.asarray(V, np.float64)
        return np.einsum("nt,ntd->td", weight_fn(V, np.asarray(w, np.float64), eps), V)
    return f


_lg = lambda V, w, eps: np.einsum("ntd,d->nt", oracle.rms_norm(V, eps), w)
MUTANTS = {
    "softmax_over_tokens": Impl(attnres=_mix(lambda V, w, eps: _softmax(_lg(V, w, eps), 1))),
    "no_norm": Impl(attnres=_mix(lambda V, w, eps: _softmax(np.einsum("ntd,d->nt", V, w), 0))),
    "norm_over_blocks": Impl(attnres=_mix(lambda V, w, eps: _softmax(
        np.einsum("ntd,d->nt", V / np.sqrt(np.mean(V * V, axis=0, keepdims=True) + eps), w), 0))),
    "negated_scores": Impl(attnres=_mix(lambda V, w, eps: _softmax(-_lg(V, w, eps), 0))),
    "unnormalised_weights": Impl(attnres=_mix(lambda V, w, eps: np.exp(_lg(V, w, eps) - _lg(V, w, eps).max(0)))),
    "mix_normed_values": Impl(attnres=lambda V, w, eps: np.einsum("nt,ntd->td", _softmax(_lg(V, w, eps), 0),
                                                                  oracle.rms_norm(V, eps))),
    "lse_is_max": Impl(lse=lambda V, w, eps: _lg(V, w, eps).max(0)),
    "lse_of_mean": Impl(lse=lambda V, w, eps: np.log(np.mean(np.exp(_lg(V, w, eps)), axis=0))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attnres_mutant_is_caught(name):
    caught = []
    for pin, tol in PINS:
        try:
            err = pin(MUTANTS[name])
        except Exception:
            err = float("inf")
        if not (err <= tol):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
