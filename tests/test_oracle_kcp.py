"""Pins of the oracle's segment map (S_out = A S_in + B over a segment of one chain) and of the
hop that chains segments, checked on the CPU.

What fixes the values (no page prints a worked example):
  * the recurrence itself (pinned on its own in test_oracle_pins.py): for any incoming state S0
    the state the recurrence reaches over the segment must equal A S0 + B (brute force over
    random, non-symmetric S0, with d_k != d_v so a transposed operand cannot pass);
  * closed forms: with beta = 0 the segment only decays, A = Diag(exp(sum_t g_t)) and B = 0;
    with alpha = 1, beta = 1 and orthonormal keys every write is a projection, so
    A = I - sum_i k_i k_i^T and B = sum_i k_i v_i^T;
  * structure: the map of a concatenation is the composition of the maps (A2 A1, A2 B1 + B2),
    and the read-out of a later segment from the chained state equals the whole chain's.
Each plausible mistake below (a transposed or reversed product, the decay on the wrong side of
the write, a dropped term in the hop) is implemented as an alternative and must fail a pin.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(930941)


class Impl:
    def __init__(self, seg=None, comb=None):
        self.seg = seg or oracle.segment_map
        self.comb = comb or oracle.state_combine


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _segment(L, dk, dv, beta_lo=0.1, beta_hi=1.0):
    k = _unit_rows(RNG.standard_normal((L, dk))).astype(np.float32)
    v = RNG.standard_normal((L, dv)).astype(np.float32)
    g = (-np.abs(RNG.standard_normal((L, dk))) * 0.3).astype(np.float32)
    beta = RNG.uniform(beta_lo, beta_hi, L).astype(np.float32)
    return k, v, g, beta


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def pin_affine_matches_recurrence(impl):
    L, dk, dv = 23, 6, 4
    k, v, g, beta = _segment(L, dk, dv)
    A, B = impl.seg(k, v, g, beta)
    worst = 0.0
    for _ in range(3):
        S0 = RNG.standard_normal((dk, dv)).astype(np.float32)
        _, S_end = oracle.chain(np.zeros((L, dk), np.float32), k, v, g, beta, 1.0, S0)
        worst = max(worst, _rel(impl.comb(A, S0, B), S_end))
    return worst


def pin_no_write_is_decay(impl):
    L, dk, dv = 9, 5, 3
    k, v, g, _ = _segment(L, dk, dv)
    A, B = impl.seg(k, v, g, np.zeros(L, np.float32))
    want = np.diag(np.exp(np.asarray(g, np.float64).sum(axis=0)))
    return max(_rel(A, want), float(np.max(np.abs(B))))


def pin_orthonormal_projections(impl):
    dk, dv, m = 7, 3, 4
    Q, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    k = Q[:, :m].T.astype(np.float32)                # m orthonormal keys (rows)
    kd = k.astype(np.float64)
    v = RNG.standard_normal((m, dv)).astype(np.float32)
    A, B = impl.seg(k, v, np.zeros((m, dk), np.float32), np.ones(m, np.float32))
    # fp32 storage of the keys makes them orthonormal to ~1e-7 only; compare at that level
    return max(_rel(A, np.eye(dk) - kd.T @ kd), _rel(B, kd.T @ v.astype(np.float64)))


def pin_composition(impl):
    L, s, dk, dv = 30, 11, 5, 5                      # square state: orientation errors keep the shape
    k, v, g, beta = _segment(L, dk, dv)
    A, B = impl.seg(k, v, g, beta)
    A1, B1 = impl.seg(k[:s], v[:s], g[:s], beta[:s])
    A2, B2 = impl.seg(k[s:], v[s:], g[s:], beta[s:])
    return max(_rel(A2 @ A1, A), _rel(impl.comb(A2, B1, B2), B))


def pin_chained_read_out(impl):
    """o of the second segment, run from the state the hop hands over, equals the whole chain's."""
    L, s, dk, dv = 26, 10, 6, 4
    k, v, g, beta = _segment(L, dk, dv)
    q = _unit_rows(RNG.standard_normal((L, dk))).astype(np.float32)
    S0 = RNG.standard_normal((dk, dv)).astype(np.float32)
    o_all, S_all = oracle.chain(q, k, v, g, beta, 0.5, S0)
    A1, B1 = impl.seg(k[:s], v[:s], g[:s], beta[:s])
    S_mid = impl.comb(A1, S0, B1).astype(np.float32)
    o2, S2 = oracle.chain(q[s:], k[s:], v[s:], g[s:], beta[s:], 0.5, S_mid)
    # S_mid is stored in fp32 (as the chain takes it): agreement to fp32 rounding of the state
    return max(_rel(o2, o_all[s:]), _rel(S2, S_all))


PINS = [(pin_affine_matches_recurrence, 1e-12), (pin_no_write_is_decay, 1e-13),
        (pin_orthonormal_projections, 1e-6), (pin_composition, 1e-12),
        (pin_chained_read_out, 1e-6)]


@pytest.mark.parametrize("pin,tol", PINS, ids=[p.__name__ for p, _ in PINS])
def test_oracle_kcp_pin(pin, tol):
    assert pin(Impl()) <= tol


def _seg_with(step):
    """A segment map whose A is built with `step(A, k, a, b)` per token; B as in the oracle."""
    def seg(k, v, g, beta):
        k, g, beta = np.asarray(k, np.float64), np.asarray(g, np.float64), np.asarray(beta, np.float64)
        A = np.eye(k.shape[1])
        for t in range(k.shape[0]):
            A = step(A, k[t], np.exp(g[t]), beta[t])
        _, B = oracle.segment_map(k, v, g, beta)
        return A, B
    return seg


def _tok(k, a, b):
    return (np.eye(len(k)) - b * np.outer(k, k)) * a[None, :]   # (I - b k k^T) Diag(a)


MUTANTS = {
    "A_transposed": Impl(seg=lambda k, v, g, b: tuple(x.T if i == 0 else x for i, x in
                                                      enumerate(oracle.segment_map(k, v, g, b)))),
    "product_reversed": Impl(seg=_seg_with(lambda A, k, a, b: A @ _tok(k, a, b))),
    "decay_after_write": Impl(seg=_seg_with(lambda A, k, a, b: (a[:, None] * (np.eye(len(k)) - b * np.outer(k, k))) @ A)),
    "no_decay_in_A": Impl(seg=_seg_with(lambda A, k, a, b: (np.eye(len(k)) - b * np.outer(k, k)) @ A)),
    "no_beta_in_A": Impl(seg=_seg_with(lambda A, k, a, b: _tok(k, a, 1.0) @ A)),
    "hop_without_offset": Impl(comb=lambda A, S, B: np.asarray(A, np.float64) @ np.asarray(S, np.float64)),
    "hop_operands_swapped": Impl(comb=lambda A, S, B: np.asarray(S, np.float64) @ np.asarray(A, np.float64) + B),
    "hop_A_transposed": Impl(comb=lambda A, S, B: np.asarray(A, np.float64).T @ np.asarray(S, np.float64) + B),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_kcp_mutant_is_caught(name):
    caught = []
    for pin, tol in PINS:
        try:
            err = pin(MUTANTS[name])
        except Exception:   # a shape error inside a pin also counts
            err = float("inf")
        if not (err <= tol):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
