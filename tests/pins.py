"""Pins for the fp64 KDA oracle: checks against what the pages and mathematics fix.

Every pin takes a `chain_fn(q, k, v, g, beta, scale, S0) -> (o [L, dv], S [dk, dv])`
(float64 results of one (sequence, head) chain) and returns an error figure that
must stay below the pin's tolerance.  The same pins run against the real oracle
and against deliberately broken copies of it (see test_oracle_mutants.py), so
each plausible mistake is shown to fail at least one of them.

Sources:
  * course page "线性注意力与 KDA" (ai.air7.fun, Day 19): section 2 (S = K^T V of size
    d_k x d_v, o_t = q_t S_t), section 3 (decay then delta write);
  * page "Kimi K3 注意力三件套" (yeyulingfeng.com), KDA section: the factor
    (I - beta_t k_t k_t^T), the delta rule as one gradient-descent step, alpha over d_k;
  * blog post ciyuanerhao post-114: chapter 3 (DeltaNet writes the prediction error; Gated
    DeltaNet adds one decay per token), chapter 4 (per-channel alpha multiplies the rows of S).
"""
from __future__ import annotations

import ctypes
import decimal
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------- helpers
def load_chain_fn(lib_path: str):
    """ctypes wrapper of a compiled `kda_oracle_chain` (the real oracle or a mutant copy)."""
    lib = ctypes.CDLL(lib_path)
    f = lib.kda_oracle_chain
    P, Lg = ctypes.c_void_p, ctypes.c_long
    f.argtypes = [Lg, ctypes.c_int, ctypes.c_int, P, Lg, P, Lg, P, Lg, P, Lg, P, Lg,
                  ctypes.c_double, P, P, Lg, P]
    f.restype = ctypes.c_int

    def chain_fn(q, k, v, g, beta, scale=1.0, S0=None):
        q, k, v, g, beta = (np.ascontiguousarray(a, dtype=np.float32) for a in (q, k, v, g, beta))
        L, dk = q.shape
        dv = v.shape[1]
        S0a = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float32)
        o = np.empty((L, dv), np.float64)
        S = np.empty((dk, dv), np.float64)
        rc = f(L, dk, dv, q.ctypes.data, dk, k.ctypes.data, dk, v.ctypes.data, dv,
               g.ctypes.data, dk, beta.ctypes.data, 1, float(scale),
               None if S0a is None else S0a.ctypes.data, o.ctypes.data, dv, S.ctypes.data)
        assert rc == 0
        return o, S

    chain_fn._lib = lib  # keep the library alive
    return chain_fn


def _rand_case(seed, L, dk, dv, unit_k=False, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk)).astype(np.float32)
    k = rng.standard_normal((L, dk)).astype(np.float32)
    if unit_k:
        k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((L, dv)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((L, dk)) + 0.5))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal(L)))).astype(np.float32)
    S0 = rng.standard_normal((dk, dv)).astype(np.float32) if s0 else None
    return q, k, v, g, beta, S0


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _parse_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


# ----------------------------------------------------------------------------- pins
def pin_hand_example(chain_fn):
    """Hand-derived d_k=2, d_v=3, T=2 example (tests/golden/kda_hand_dk2_dv3.txt).

    g is stored in fp32, so exp(g) differs from the rational alpha by ~1e-7 relative.
    """
    r = _parse_golden("kda_hand_dk2_dv3.txt")
    F = lambda xs: np.array([float(Fraction(x)) for x in xs])
    S0 = F(r["S0"]).reshape(2, 3)
    alpha = F(r["alpha"]).reshape(2, 2)
    beta = F(r["beta"])
    k = F(r["k"]).reshape(2, 2)
    v = F(r["v"]).reshape(2, 3)
    q = F(r["q"]).reshape(2, 2)
    o_ref = F(r["o"]).reshape(2, 3)
    S_ref = F(r["S_final"]).reshape(2, 3)
    o, S = chain_fn(q, k, v, np.log(alpha), beta, 1.0, S0)
    return max(_rel(o, o_ref), _rel(S, S_ref))


pin_hand_example.tol = 1e-6


def pin_product_form(chain_fn, seed=11, L=7, dk=5, dv=4):
    """Unrolled product with the explicit transition M_t = (I - beta_t k_t k_t^T) Diag(alpha_t).

    S_t = P(t,0) S_0 + sum_j P(t,j) beta_j k_j v_j^T with P(t,j) = M_t ... M_{j+1};
    o_t = scale * S_t^T q_t.  (KDA section of the yeyulingfeng page names the factor.)
    """
    q, k, v, g, beta, S0 = _rand_case(seed, L, dk, dv)
    scale = 0.75
    D = lambda a: np.asarray(a, np.float64)
    q, k, v, g, beta, S0d = D(q), D(k), D(v), D(g), D(beta), D(S0)
    I = np.eye(dk)
    M = [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(L)]

    def P(t, j):  # M_t ... M_{j+1} (tokens numbered 1..L; list index t-1)
        out = I.copy()
        for m in range(j + 1, t + 1):
            out = M[m - 1] @ out
        return out

    o_ref = np.zeros((L, dv))
    S_t = None
    for t in range(1, L + 1):
        S_t = P(t, 0) @ S0d
        for j in range(1, t + 1):
            S_t = S_t + P(t, j) @ (beta[j - 1] * np.outer(k[j - 1], v[j - 1]))
        o_ref[t - 1] = scale * S_t.T @ q[t - 1]
    o, S = chain_fn(q, k, v, g, beta, scale, S0)
    return max(_rel(o, o_ref), _rel(S, S_t))


pin_product_form.tol = 1e-12


def pin_high_precision(chain_fn, seed=5, L=5, dk=3, dv=3):
    """The recurrence in 60-digit decimal arithmetic (alpha = exp(g) of the stored fp32 g).

    Inputs are dyadic rationals (exact in fp32); the only non-rational step is exp(g),
    evaluated to 60 digits.  The fp64 oracle must agree to rounding level.
    """
    rng = np.random.default_rng(seed)
    dy = lambda shape, den: (rng.integers(-8, 9, size=shape) / den).astype(np.float32)
    q, k, v, S0 = dy((L, dk), 8), dy((L, dk), 8), dy((L, dv), 4), dy((dk, dv), 4)
    g = (-rng.integers(1, 9, size=(L, dk)) / 8).astype(np.float32)
    beta = (rng.integers(1, 8, size=L) / 8).astype(np.float32)
    ctx = decimal.Context(prec=60)
    Dc = lambda x: decimal.Decimal(float(x))
    S = [[Dc(S0[i, j]) for j in range(dv)] for i in range(dk)]
    o_ref = np.zeros((L, dv))
    for t in range(L):
        a = [ctx.exp(Dc(g[t, i])) for i in range(dk)]
        S = [[ctx.multiply(a[i], S[i][j]) for j in range(dv)] for i in range(dk)]
        p = [sum((S[i][j] * Dc(k[t, i]) for i in range(dk)), decimal.Decimal(0)) for j in range(dv)]
        u = [Dc(beta[t]) * (Dc(v[t, j]) - p[j]) for j in range(dv)]
        S = [[S[i][j] + Dc(k[t, i]) * u[j] for j in range(dv)] for i in range(dk)]
        for j in range(dv):
            o_ref[t, j] = float(sum((S[i][j] * Dc(q[t, i]) for i in range(dk)), decimal.Decimal(0)))
    S_ref = np.array([[float(x) for x in row] for row in S])
    o, Sn = chain_fn(q, k, v, g, beta, 1.0, S0)
    return max(_rel(o, o_ref), _rel(Sn, S_ref))


pin_high_precision.tol = 1e-14


def pin_deltanet(chain_fn, seed=21, L=9, dk=4, dv=6):
    """alpha == 1 reduces KDA to DeltaNet (blog post-114, chapter 3: DeltaNet writes only the
    prediction error; course page, section 3, with the decay factor equal to one).

    Written here in the course page's own orientation, a d_v x d_k memory M (M = S^T):
    M_t = M_{t-1} + beta_t (v_t - M_{t-1} k_t) k_t^T and o_t = M_t q_t, with explicit
    outer products; the oracle keeps the K-major transpose, so the two share no layout.
    """
    q, k, v, _, beta, S0 = _rand_case(seed, L, dk, dv)
    M = S0.astype(np.float64).T.copy()           # d_v x d_k
    o_ref = np.zeros((L, dv))
    for t in range(L):
        kt, vt, qt = (x[t].astype(np.float64) for x in (k, v, q))
        err = vt - M.dot(kt)                      # prediction error of the memory for key k_t
        M = M + float(beta[t]) * np.outer(err, kt)
        o_ref[t] = M.dot(qt)
    o, Sn = chain_fn(q, k, v, np.zeros((L, dk), np.float32), beta, 1.0, S0)
    return max(_rel(o, o_ref), _rel(Sn, M.T))


pin_deltanet.tol = 1e-12


def pin_gated_deltanet_scalar(chain_fn, seed=31, L=9, dk=4, dv=5):
    """All channels sharing one alpha_t gives Gated DeltaNet (blog post-114, chapter 3), with
    the decay applied first as in the course page's section 3.

    Written as a transition plus an input, with the factor named in the KDA section of the page
    "Kimi K3 注意力三件套": S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, formed with
    an explicit d_k x d_k matrix (a scalar a_t commutes with the factor).
    """
    q, k, v, _, beta, S0 = _rand_case(seed, L, dk, dv)
    rng = np.random.default_rng(seed + 1)
    gs = (-rng.uniform(0.05, 2.0, size=L)).astype(np.float32)
    g = np.repeat(gs[:, None], dk, axis=1)
    S = S0.astype(np.float64)
    o_ref = np.zeros((L, dv))
    eye = np.eye(dk)
    for t in range(L):
        kt = k[t].astype(np.float64)
        b = float(beta[t])
        A = math.exp(float(gs[t])) * (eye - b * np.outer(kt, kt))
        S = A.dot(S) + b * np.outer(kt, v[t].astype(np.float64))
        o_ref[t] = S.T.dot(q[t].astype(np.float64))
    o, Sn = chain_fn(q, k, v, g, beta, 1.0, S0)
    return max(_rel(o, o_ref), _rel(Sn, S))


pin_gated_deltanet_scalar.tol = 1e-12


def pin_beta0_identity(chain_fn, seed=41, L=6, dk=4, dv=3):
    """beta = 0 and alpha = 1: the state never changes and o_t = scale * S_0^T q_t."""
    q, k, v, _, _, S0 = _rand_case(seed, L, dk, dv)
    o, S = chain_fn(q, k, v, np.zeros((L, dk), np.float32), np.zeros(L, np.float32), 1.5, S0)
    o_ref = 1.5 * q.astype(np.float64) @ S0.astype(np.float64)
    return max(_rel(o, o_ref), _rel(S, S0))


pin_beta0_identity.tol = 1e-15


def pin_recall(chain_fn, seed=51, L=8, dv=5):
    """Unit key and beta = 1: the state maps k_t to v_t exactly (S_t^T k_t = v_t).

    Keys are signed Hadamard rows / 2 (exactly unit in fp32); reading with q_t = k_t
    and scale 1 gives o_t = S_t^T k_t.
    """
    dk = 4
    Hd = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], np.float64) / 2
    rng = np.random.default_rng(seed)
    k = np.stack([Hd[rng.integers(0, 4)] * rng.choice([-1.0, 1.0]) for _ in range(L)]).astype(np.float32)
    _, _, v, g, _, S0 = _rand_case(seed, L, dk, dv)
    o, _ = chain_fn(k, k, v, g, np.ones(L, np.float32), 1.0, S0)
    return _rel(o, v)


pin_recall.tol = 1e-13


def pin_orthonormal(chain_fn, seed=61, dv=3):
    """Orthonormal keys, alpha = 1, beta = 1, S_0 = 0: plain causal linear attention.

    S_T = sum_j k_j v_j^T and o_t = sum_{j<=t} (q_t . k_j) v_j (course page section 2:
    S = K^T V, o = q S), because orthogonal writes never interfere.
    """
    Hd = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], np.float64) / 2
    rng = np.random.default_rng(seed)
    perm = rng.permutation(4)
    k = Hd[perm].astype(np.float32)
    L, dk = 4, 4
    q = rng.standard_normal((L, dk)).astype(np.float32)
    v = rng.standard_normal((L, dv)).astype(np.float32)
    o, S = chain_fn(q, k, v, np.zeros((L, dk), np.float32), np.ones(L, np.float32), 1.0, None)
    K, V, Q = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    S_ref = K.T @ V
    o_ref = np.tril(Q @ K.T) @ V
    return max(_rel(o, o_ref), _rel(S, S_ref))


pin_orthonormal.tol = 1e-13


def pin_gradient_step(chain_fn, seed=71, dk=4, dv=5):
    """One token is one gradient step on 0.5 ||S~^T k - v||^2 with step beta (KDA section).

    The gradient is taken by central finite differences (exact for a quadratic up to rounding).
    """
    q, k, v, g, beta, S0 = _rand_case(seed, 1, dk, dv)
    St = np.exp(g[0].astype(np.float64))[:, None] * S0.astype(np.float64)
    kk, vv = k[0].astype(np.float64), v[0].astype(np.float64)
    loss = lambda S: 0.5 * float(np.sum((S.T @ kk - vv) ** 2))
    grad = np.zeros_like(St)
    h = 1e-3
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(St)
            E[i, j] = h
            grad[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
    S_ref = St - float(beta[0]) * grad
    _, S = chain_fn(q, k, v, g, beta, 1.0, S0)
    return _rel(S, S_ref)


pin_gradient_step.tol = 1e-9


def pin_linearity(chain_fn, seed=81, L=7, dk=4, dv=4):
    """o and S are linear in (S_0, v) jointly, o is linear in q and in scale."""
    _, k, v, g, beta, S0 = _rand_case(seed, L, dk, dv)
    # dyadic q and q2 so that q + q2 is exact in fp32
    rng = np.random.default_rng(seed + 1)
    q = (rng.integers(-16, 17, size=(L, dk)) / 16).astype(np.float32)
    q2 = (rng.integers(-16, 17, size=(L, dk)) / 16).astype(np.float32)
    o1, S1 = chain_fn(q, k, v, g, beta, 1.0, S0)
    o2, S2 = chain_fn(q, k, (2 * v).astype(np.float32), g, beta, 1.0, (2 * S0).astype(np.float32))
    oa, _ = chain_fn(q2, k, v, g, beta, 1.0, S0)
    ob, _ = chain_fn((q + q2).astype(np.float32), k, v, g, beta, 0.5, S0)
    return max(_rel(o2, 2 * o1), _rel(S2, 2 * S1), _rel(ob, 0.5 * (o1 + oa)))


pin_linearity.tol = 1e-12


def pin_chunk_form(chain_fn, seed=91, L=37, dk=16, dv=12, C=8):
    """The chunkwise (WY / UT-transform) re-association equals the recurrence exactly.

    Independent algorithm in tests/chunk_model.py (intra-chunk parallel, inter-chunk serial);
    a last chunk shorter than C is included.
    """
    from chunk_model import chunk_forward
    q, k, v, g, beta, S0 = _rand_case(seed, L, dk, dv, unit_k=True)
    o_ref, S_ref = chunk_forward(q, k, v, g, beta, 0.9, S0, C)
    o, S = chain_fn(q, k, v, g, beta, 0.9, S0)
    return max(_rel(o, o_ref), _rel(S, S_ref))


pin_chunk_form.tol = 1e-12


def pin_split_resume(chain_fn, seed=101, L=11, dk=5, dv=4):
    """Running T1 then T2 tokens from the carried state equals running T1 + T2 tokens."""
    q, k, v, g, beta, S0 = _rand_case(seed, L, dk, dv)
    o, S = chain_fn(q, k, v, g, beta, 1.0, S0)
    oa, Sa = chain_fn(q[:4], k[:4], v[:4], g[:4], beta[:4], 1.0, S0)
    ob, Sb = chain_fn(q[4:], k[4:], v[4:], g[4:], beta[4:], 1.0, Sa.astype(np.float32))
    # the carried state is rounded to fp32 between the two calls
    return max(_rel(np.concatenate([oa, ob]), o), _rel(Sb, S))


pin_split_resume.tol = 1e-6


PINS = [pin_hand_example, pin_product_form, pin_high_precision, pin_deltanet,
        pin_gated_deltanet_scalar, pin_beta0_identity, pin_recall, pin_orthonormal,
        pin_gradient_step, pin_linearity, pin_chunk_form, pin_split_resume]
