"""Pins of the oracle's low-rank gate (log alpha and beta from the input), checked on the CPU.

What fixes the values (no page prints a worked example):
  * closed forms: with W_up = 0 the gate is -softplus(b) = -log(1 + e^b), -log 2 at b = 0;
    alpha = e^g must equal sigmoid(-pre) (scipy's expit) for a known pre-activation;
  * brute force: explicit loops over every index on tiny shapes, using the math module;
  * structure: the pre-activations recovered from g form a matrix of rank <= r (low rank, page
    "Kimi K3 注意力三件套", KDA section); beta(x) + beta(-x) = 1 and beta(0) = 1/2.
Each plausible mistake below (a wrong sign, a dropped bias, a misread weight layout, a missing
nonlinearity) is implemented as an alternative gate and must fail at least one pin.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle

RNG = np.random.default_rng(930931)


class Impl:
    def __init__(self, z=None, g=None, beta=None):
        self.z = z or oracle.gate_z
        self.g = g or oracle.gate_g
        self.beta = beta or oracle.gate_beta


def pin_zero_up_closed_form(impl):
    H, d, r = 2, 3, 2
    b = np.array([-30.0, -5.0, 0.0, 2.0, 7.5, 30.0])
    z = RNG.standard_normal((4, r))
    g = impl.g(z, np.zeros((H * d, r)), b, H, d)
    want = np.array([-math.log1p(math.exp(x)) for x in b])
    return float(np.max(np.abs(g.reshape(4, H * d) - want[None, :]) / np.maximum(np.abs(want), 1e-300)))


def pin_alpha_is_sigmoid_of_minus_pre(impl):
    s = np.linspace(-40.0, 40.0, 81)                 # known pre-activations: r = 1, w_up = 1, b = 0
    g = impl.g(s[:, None], np.ones((1, 1)), np.zeros(1), 1, 1).reshape(-1)
    want = expit(-s)
    return float(np.max(np.abs(np.exp(g) - want) / want))


def _loops(x, w_down, w_beta, w_up, b, H, d):
    Ntok, Dm = x.shape
    r = w_down.shape[0]
    z = [[sum(float(x[t, m]) * float(w_down[j, m]) for m in range(Dm)) for j in range(r)] for t in range(Ntok)]
    g = np.zeros((Ntok, H, d))
    beta = np.zeros((Ntok, H))
    for t in range(Ntok):
        for h in range(H):
            a = sum(float(x[t, m]) * float(w_beta[h, m]) for m in range(Dm))
            beta[t, h] = 1.0 / (1.0 + math.exp(-a))
            for c in range(d):
                pre = float(b[h * d + c]) + sum(z[t][j] * float(w_up[h * d + c, j]) for j in range(r))
                g[t, h, c] = -math.log(1.0 + math.exp(pre))
    return np.array(z), beta, g


def pin_brute_force_loops(impl):
    Ntok, Dm, r, H, d = 3, 5, 2, 2, 3
    x = RNG.standard_normal((Ntok, Dm))
    w_down = RNG.standard_normal((r, Dm))
    w_beta = RNG.standard_normal((H, Dm))
    w_up = RNG.standard_normal((H * d, r))
    b = RNG.standard_normal(H * d)
    z0, beta0, g0 = _loops(x, w_down, w_beta, w_up, b, H, d)
    z = impl.z(x, w_down)
    e = [np.max(np.abs(z - z0)), np.max(np.abs(impl.beta(x, w_beta) - beta0)),
         np.max(np.abs(impl.g(z, w_up, b, H, d) - g0))]
    return float(max(e))


def pin_square_layouts(impl):
    """Same loops with r = H*d and Dm = r, so a misread (transposed) weight still has the right shape."""
    Ntok, H, d = 3, 2, 2
    r = Dm = H * d
    x = RNG.standard_normal((Ntok, Dm))
    w_down = RNG.standard_normal((r, Dm))
    w_beta = RNG.standard_normal((H, Dm))
    w_up = RNG.standard_normal((H * d, r))
    b = RNG.standard_normal(H * d)
    z0, beta0, g0 = _loops(x, w_down, w_beta, w_up, b, H, d)
    z = impl.z(x, w_down)
    return float(max(np.max(np.abs(z - z0)), np.max(np.abs(impl.g(z, w_up, b, H, d) - g0))))


def pin_low_rank(impl):
    Ntok, Dm, r, H, d = 24, 16, 3, 3, 4
    x = RNG.standard_normal((Ntok, Dm))
    w_down = RNG.standard_normal((r, Dm)) / 4
    w_up = RNG.standard_normal((H * d, r)) / 2
    b = RNG.standard_normal(H * d)
    g = impl.g(impl.z(x, w_down), w_up, b, H, d).reshape(Ntok, H * d)
    with np.errstate(invalid="ignore", divide="ignore"):
        pre = np.log(np.expm1(-g)) - b[None, :]      # inverse of -softplus, minus the bias
    if not np.all(np.isfinite(pre)):
        return float("inf")
    sv = np.linalg.svd(pre, compute_uv=False)
    return float(sv[r] / sv[0])                      # rank <= r: the (r+1)-th singular value vanishes


def pin_beta_symmetry(impl):
    x = RNG.standard_normal((5, 7))
    w = RNG.standard_normal((3, 7))
    e1 = np.max(np.abs(impl.beta(x, w) + impl.beta(-x, w) - 1.0))
    e2 = np.max(np.abs(impl.beta(np.zeros((2, 7)), w) - 0.5))
    e3 = np.max(np.abs(impl.beta(x, w) - expit(np.einsum("tm,hm->th", x, w))))
    return float(max(e1, e2, e3))


PINS = [(pin_zero_up_closed_form, 1e-13), (pin_alpha_is_sigmoid_of_minus_pre, 1e-12),
        (pin_brute_force_loops, 1e-12), (pin_square_layouts, 1e-12), (pin_low_rank, 1e-10),
        (pin_beta_symmetry, 1e-14)]


@pytest.mark.parametrize("pin,tol", PINS, ids=[p.__name__ for p, _ in PINS])
def test_oracle_gate_pin(pin, tol):
    assert pin(Impl()) <= tol


def _g_with(pre_fn, post_fn):
    def g(z, w_up, b, H, d):
        return post_fn(pre_fn(np.asarray(z, np.float64), np.asarray(w_up, np.float64),
                              np.asarray(b, np.float64), H, d)).reshape(len(z), H, d)
    return g


_pre = lambda z, w, b, H, d: z @ w.T + b[None, :]
MUTANTS = {
    "g_sign": Impl(g=_g_with(_pre, lambda p: oracle.softplus(p))),
    "no_bias": Impl(g=_g_with(lambda z, w, b, H, d: z @ w.T, lambda p: -oracle.softplus(p))),
    "bias_per_head": Impl(g=_g_with(lambda z, w, b, H, d: z @ w.T + np.repeat(b[::d], d)[None, :],
                                    lambda p: -oracle.softplus(p))),
    "w_up_layout": Impl(g=_g_with(lambda z, w, b, H, d: z @ w.reshape(w.shape[1], w.shape[0]) + b[None, :],
                                  lambda p: -oracle.softplus(p))),
    "no_nonlinearity": Impl(g=_g_with(_pre, lambda p: -p)),
    "alpha_sigmoid_of_pre": Impl(g=_g_with(_pre, lambda p: np.log(oracle.sigmoid(p)))),
    "w_down_layout": Impl(z=lambda x, w: np.asarray(x, np.float64) @ np.asarray(w, np.float64).reshape(w.shape[1], w.shape[0])),
    "beta_no_sigmoid": Impl(beta=lambda x, w: np.asarray(x, np.float64) @ np.asarray(w, np.float64).T),
    "beta_sign": Impl(beta=lambda x, w: oracle.sigmoid(-(np.asarray(x, np.float64) @ np.asarray(w, np.float64).T))),
    "beta_layout": Impl(beta=lambda x, w: oracle.sigmoid(np.asarray(x, np.float64) @ np.asarray(w, np.float64).reshape(w.shape[1], w.shape[0]))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gate_mutant_is_caught(name):
    caught = []
    for pin, tol in PINS:
        try:
            err = pin(MUTANTS[name])
        except Exception:   # a shape error inside a pin also counts
            err = float("inf")
        if not (err <= tol):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
