"""Chunkwise form of the KDA recurrence in fp64 numpy (test-side model, not the oracle).

The pages say deployment uses a chunkwise parallel form (WY representation plus UT
transform; page "Kimi K3 注意力三件套", KDA section) and that chunking splits the
update into parallel work inside a block and serial work across blocks (blog
post-114, chapter 3).  They omit the derivation; the form below follows from the
course page's section-3 update by unrolling it over one chunk:

  within a chunk with incoming state S, G_t = sum_{s<=t} g_s (per channel), gamma = G_last:
    Akk[t,j] = beta_t sum_c k_tc k_jc exp(G_tc - G_jc)   (j < t)
    Aqk[t,j] =        sum_c q_tc k_jc exp(G_tc - G_jc)   (j <= t)
    Tm = (I + Akk)^-1
    W  = Tm (beta * K * exp(G)),   U = Tm (beta * V)
    Ud = U - W S
    O  = scale (Q * exp(G)) S + scale Aqk Ud
    S' = exp(gamma) * S + (K * exp(gamma - G))^T Ud
Every exponent is a difference that is <= 0.  The model checks the algebra the GPU
kernels rely on; it is not used as the parity reference.
"""
from __future__ import annotations

import numpy as np


def chunk_forward(q, k, v, g, beta, scale, S0, C):
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, np.float64)
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    o = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        n = Q.shape[0]
        G = np.cumsum(g[sl], axis=0)
        gamma = G[-1]
        diff = G[:, None, :] - G[None, :, :]                   # [t, j, c]
        lower = np.tril(np.ones((n, n), bool))
        E = np.exp(np.where(lower[:, :, None], diff, -np.inf))  # 0 above the diagonal
        Akk = b[:, None] * np.einsum("tc,jc,tjc->tj", K, K, E)
        Akk = np.tril(Akk, -1)
        Aqk = np.einsum("tc,jc,tjc->tj", Q, K, E)
        Tm = np.linalg.inv(np.eye(n) + Akk)
        W = Tm @ (b[:, None] * K * np.exp(G))
        U = Tm @ (b[:, None] * V)
        Ud = U - W @ S
        o[sl] = scale * ((Q * np.exp(G)) @ S + Aqk @ Ud)
        S = np.exp(gamma)[:, None] * S + (K * np.exp(gamma[None, :] - G)).T @ Ud
    return o, S


def _inv_unit_lower_blocked(A, bs=16):
    """(I + A)^-1 for strictly lower A by 16x16 diagonal forward substitution plus block merges."""
    n = A.shape[0]
    T = np.zeros_like(A)
    nb = (n + bs - 1) // bs
    for b in range(nb):
        s = slice(b * bs, min((b + 1) * bs, n))
        m = s.stop - s.start
        Tb = np.eye(m)
        Ab = A[s, s]
        for i in range(m):
            Tb[i, :i] = -Ab[i, :i] @ Tb[:i, :i]
        T[s, s] = Tb
    for I in range(1, nb):
        si = slice(I * bs, min((I + 1) * bs, n))
        for J in range(I):
            sj = slice(J * bs, (J + 1) * bs)
            X = np.zeros((si.stop - si.start, bs))
            for M in range(J, I):
                sm = slice(M * bs, (M + 1) * bs)
                X += A[si, sm] @ T[sm, sj]
            T[si, sj] = -T[si, si] @ X
    return T


def subblock_gram(K, Q, G, b, bs=16, rnd=None):
    """Akk and Aqk with the 16-token sub-block factorisation used by the GPU kernels.

    Block I uses its middle row m_I as reference: row factor exp(G_i - G_mI), column
    factor exp(G_mJ - G_j), and for I > J the per-channel bridge exp(G_mI - G_mJ) <= 1.
    Valid while |G_i - G_mI| stays below the fp32 exponent range inside every block.
    `rnd` rounds MFMA operands (identity in exact mode).
    """
    rnd = rnd or (lambda x: x)
    n = K.shape[0]
    nb = (n + bs - 1) // bs
    mid = [min(I * bs + bs // 2, n - 1) for I in range(nb)]
    Akk = np.zeros((n, n))
    Aqk = np.zeros((n, n))
    for I in range(nb):
        si = slice(I * bs, min((I + 1) * bs, n))
        fa = np.exp(G[si] - G[mid[I]])
        kA, qA = rnd(K[si] * fa), rnd(Q[si] * fa)
        for J in range(I + 1):
            sj = slice(J * bs, min((J + 1) * bs, n))
            fb = np.exp(G[mid[J]] - G[sj])
            if J < I:
                fb = fb * np.exp(G[mid[I]] - G[mid[J]])[None, :]
            kB = rnd(K[sj] * fb)
            Akk[si, sj] = b[si, None] * (kA @ kB.T)
            Aqk[si, sj] = qA @ kB.T
    lower = np.tril(np.ones((n, n), bool))
    return np.where(np.tril(lower, -1), Akk, 0.0), np.where(lower, Aqk, 0.0)


def chunk_forward_gpu_plan(q, k, v, g, beta, scale, S0, C=64, rnd=None, rnd_out=None):
    """The chunk form with the GPU kernels' factorisation and blocked inverse.

    In exact mode (rnd=None) it must equal the recurrence to fp64 rounding.  With `rnd`
    set to a bf16 rounding it emulates where the bf16 path rounds MFMA operands.
    """
    rnd = rnd or (lambda x: x)
    rnd_out = rnd_out or (lambda x: x)
    q, k, v, g = (np.asarray(a, np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, np.float64)
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    o = np.zeros((L, dv))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        G = np.cumsum(g[sl], axis=0)
        gamma = G[-1]
        Akk, Aqk = subblock_gram(K, Q, G, b, rnd=rnd)
        Tm = _inv_unit_lower_blocked(Akk)
        Tb = rnd(Tm)
        W = Tb @ rnd(b[:, None] * K * np.exp(G))
        U = Tb @ rnd(b[:, None] * V)
        W, U, Aqk = rnd(W), rnd(U), rnd(Aqk)
        Qt, Kt = rnd(Q * np.exp(G)), rnd(K * np.exp(gamma[None, :] - G))
        Sb = rnd(S)
        Ud = U - W @ Sb
        Udb = rnd(Ud)
        o[sl] = rnd_out(scale * (Qt @ Sb + Aqk @ Udb))
        S = np.exp(gamma)[:, None] * S + Kt.T @ Udb
    return o, S
