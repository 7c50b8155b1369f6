"""fp64 CPU oracle for the KDA operator -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  It shares no code with the HIP implementation in
`gated_delta_rule_93_amd/` and never imports it.

Contents
  recurrence      token-by-token KDA recurrence in fp64 (C library `kda_oracle.c`,
                  one thread per independent (sequence, head) chain).
  prep            q/k prologue: short causal depthwise conv, SiLU, L2 norm (numpy fp64).
  gate_z, gate_g, gate_beta, gate
                  low-rank gate: z = x W_down^T, log(alpha) = -softplus(z W_up^T + b),
                  beta = sigmoid(x w_beta^T) (numpy fp64).
  attnres, attnres_logits, attnres_lse, rms_norm
                  Block AttnRes read-out: softmax over the blocks of w . norm(V_n), then the
                  weighted sum of the blocks V_n (numpy fp64).
  segment_map, state_combine
                  the affine map S_out = A S_in + B of a segment of one chain, and one hop
                  of the prefix over segments (KCP context parallelism; numpy fp64 + the
                  C recurrence).

Sources (the pages this follows)
  * Course page "线性注意力与 KDA" (ai.air7.fun, Day 19), section 3: the decay
    S~ = alpha_t (.) S_{t-1} per channel, then the delta write
    S_t = S~ + beta_t (v_t - S~ k_t) k_t^T; section 2: o_t = q_t S_t.
  * Page "Kimi K3 注意力三件套" (yeyulingfeng.com), KDA section: alpha_t is a
    vector over the key channels; q and k pass a short causal convolution and
    are L2-normalised.
  * Blog post ciyuanerhao.com post-114, chapter 3 (DeltaNet code: silu, then
    normalize; state in [d_k, d_v] orientation; beta = sigmoid(w_beta(x))) and
    chapter 4 (per-channel alpha multiplies the state rows; alpha = gate(x) is
    computed from the input, per layer, head and channel).
  * Page "Kimi K3 注意力三件套", KDA section: alpha comes from a low-rank
    down-up projection of the input; beta is a single scalar.  AttnRes section:
    softmax weights over the earlier blocks' outputs, summing to one; two-phase
    inference with an online-softmax merge.
  * Blog post-114, chapter 3: chunks are processed in parallel inside and merged
    serially into the state; K3's KCP extends that across devices (the segment map).
  * Blog post-114, chapter 6: the block AttnRes listing (stack the block outputs,
    normalise them as keys, score them with the layer's projection weight, softmax
    over the blocks, weighted sum).

Readings adopted where the pages are silent (each also listed in the design doc):
  state K-major [d_k, d_v] with o = S^T q; decay before the delta read; read-out
  after the update; g = log(alpha) as the input; beta one scalar per token and
  head; prologue = conv (width W, zero history at each sequence start, last tap
  on the current token, no bias) -> SiLU -> x / max(||x||_2, 1e-12) per head;
  gate: log(alpha) = -softplus(up(down(x)) + b) with a per-channel bias b and no
  bias inside the projections, beta = sigmoid(w_beta . x) without bias; AttnRes:
  the "norm" of the listing is an RMS norm over the hidden width with an epsilon
  argument and no learned scale.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (IEEE double arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        f = lib.kda_oracle_chain
        P = ctypes.c_void_p
        Lg = ctypes.c_long
        f.argtypes = [Lg, ctypes.c_int, ctypes.c_int,
                      P, Lg, P, Lg, P, Lg, P, Lg, P, Lg,
                      ctypes.c_double, P, P, Lg, P]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, min(len(os.sched_getaffinity(0)), 16))
    except AttributeError:  # pragma: no cover
        return max(1, min(os.cpu_count() or 1, 16))


def _f32(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def chain(q, k, v, g, beta, scale: float = 1.0, S0=None):
    """One (sequence, head) chain: q, k, g [L, dk]; v [L, dv]; beta [L]; S0 [dk, dv] or None.

    Returns (o [L, dv] float64, S_final [dk, dv] float64).
    """
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    L, dk = q.shape
    dv = v.shape[1]
    S0a = None if S0 is None else _f32(S0)
    o = np.empty((L, dv), np.float64)
    S = np.empty((dk, dv), np.float64)
    rc = _load().kda_oracle_chain(L, dk, dv,
                                  q.ctypes.data, dk, k.ctypes.data, dk, v.ctypes.data, dv,
                                  g.ctypes.data, dk, beta.ctypes.data, 1, float(scale),
                                  None if S0a is None else S0a.ctypes.data,
                                  o.ctypes.data, dv, S.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle chain allocation failed")
    return o, S


class Recurrence:
    """Runs the oracle over the chains of a packed or dense batch without copying the inputs.

    q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H] (fp32 storage);
    S0 [N, H, dk, dv] or None; cu_seqlens [N+1] or None (dense: N = B).
    """

    def __init__(self, q, k, v, g, beta, scale: float = 1.0, S0=None, cu_seqlens=None):
        self.q, self.k, self.v, self.g, self.beta = (_f32(a) for a in (q, k, v, g, beta))
        self.S0 = None if S0 is None else _f32(S0)
        self.scale = float(scale)
        B, T, H, dk = self.q.shape
        self.B, self.T, self.H, self.dk = B, T, H, dk
        self.dv = self.v.shape[3]
        self.cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
        self.N = B if self.cu is None else len(self.cu) - 1

    def bounds(self, n: int) -> Tuple[int, int, int]:
        """(batch row, first token, length) of sequence n."""
        if self.cu is None:
            return n, 0, self.T
        return 0, int(self.cu[n]), int(self.cu[n + 1] - self.cu[n])

    def run_chain(self, n: int, h: int):
        """o [L, dv] and final state of chain (n, h)."""
        b, s, L = self.bounds(n)
        H, dk, dv = self.H, self.dk, self.dv
        itm = 4
        base_tok = (b * self.T + s) * H + h
        o = np.empty((L, dv), np.float64)
        S = np.empty((dk, dv), np.float64)
        S0p = None
        if self.S0 is not None:
            S0p = self.S0.ctypes.data + ((n * H + h) * dk * dv) * itm
        rc = _load().kda_oracle_chain(
            L, dk, dv,
            self.q.ctypes.data + base_tok * dk * itm, H * dk,
            self.k.ctypes.data + base_tok * dk * itm, H * dk,
            self.v.ctypes.data + base_tok * dv * itm, H * dv,
            self.g.ctypes.data + base_tok * dk * itm, H * dk,
            self.beta.ctypes.data + base_tok * itm, H,
            self.scale, S0p, o.ctypes.data, dv, S.ctypes.data)
        if rc != 0:
            raise MemoryError("oracle chain allocation failed")
        return o, S

    def run(self, chains: Optional[Sequence[Tuple[int, int]]] = None, threads: Optional[int] = None):
        """Run chains in parallel threads; returns {(n, h): (o, S)}."""
        if chains is None:
            chains = [(n, h) for n in range(self.N) for h in range(self.H)]
        chains = list(chains)
        threads = threads or default_threads()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            res = list(ex.map(lambda nh: self.run_chain(nh[0], nh[1]), chains))
        return dict(zip(chains, res))

    def run_all(self, threads: Optional[int] = None):
        """Full outputs: o [B, T, H, dv] float64 and S [N, H, dk, dv] float64."""
        res = self.run(threads=threads)
        o = np.zeros((self.B, self.T, self.H, self.dv), np.float64)
        S = np.empty((self.N, self.H, self.dk, self.dv), np.float64)
        for (n, h), (on, Sn) in res.items():
            b, s, L = self.bounds(n)
            o[b, s:s + L, h] = on
            S[n, h] = Sn
        return o, S


def recurrence(q, k, v, g, beta, scale: float = 1.0, S0=None, cu_seqlens=None, threads=None):
    """Whole-batch oracle: returns (o [B, T, H, dv], S_final [N, H, dk, dv]) in float64."""
    return Recurrence(q, k, v, g, beta, scale, S0, cu_seqlens).run_all(threads)


# ----------------------------------------------------------------------------- prologue
def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in fp64 (blog post-114, chapter 3 DeltaNet code: F.silu)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def prep_sequence(x: np.ndarray, w: np.ndarray, H: int, d: int, eps: float = 1e-12) -> np.ndarray:
    """Prologue of one sequence, fp64.

    x [L, H*d] raw q or k values of one sequence (stored values); w [H*d, W] conv taps.
    Step 1, short causal depthwise convolution (page "Kimi K3 注意力三件套", KDA
    section): y_t[c] = sum_{tau=0}^{W-1} w[c, tau] * x_{t-(W-1)+tau}[c], with x = 0
    before the first token of the sequence; the last tap (tau = W-1) is the current token.
    Step 2, SiLU, then step 3, per (token, head) division by max(||.||_2, eps)
    (blog post-114 chapter 3: F.normalize(F.silu(.)), whose default eps is 1e-12).
    Returns [L, H*d] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, C = x.shape
    W = w.shape[1]
    y = np.zeros((L, C), np.float64)
    for tau in range(W):
        shift = (W - 1) - tau          # this tap reads token t - shift
        if shift >= L:
            continue
        y[shift:] += w[:, tau][None, :] * x[:L - shift]
    y = silu(y)
    yh = y.reshape(L, H, d)
    nrm = np.sqrt(np.sum(yh * yh, axis=-1, keepdims=True))
    return (yh / np.maximum(nrm, eps)).reshape(L, C)


def prep(x: np.ndarray, w: np.ndarray, cu_seqlens, H: int, d: int, seqs=None) -> dict:
    """Prologue over a packed batch x [Ntok, H*d] (or [1, Ntok, H, d]); returns {n: y_n [L_n, H*d]}."""
    x = np.asarray(x)
    x = x.reshape(-1, H * d)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seqs = range(len(cu) - 1) if seqs is None else seqs
    return {n: prep_sequence(x[cu[n]:cu[n + 1]], w, H, d) for n in seqs}


# --------------------------------------------------------------------------- low-rank gate
def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) in fp64, written as max(x, 0) + log1p(e^{-|x|}) so no term overflows."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^{-x}) in fp64, evaluated without overflow for either sign of x."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_z(x: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Down projection of the low-rank gate, fp64: z = x W_down^T.

    x [Ntok, Dm] (stored values), w_down [r, Dm].  The page "Kimi K3 注意力三件套" (KDA
    section) says alpha is generated by a low-rank down-up projection of the input; this is
    the "down" half, shared by all heads.  Returns [Ntok, r].
    """
    return np.asarray(x, np.float64) @ np.asarray(w_down, np.float64).T


def gate_g(z: np.ndarray, w_up: np.ndarray, b: np.ndarray, H: int, d: int) -> np.ndarray:
    """Up projection and map onto log(alpha), fp64: g = -softplus(z W_up^T + b).

    z [Ntok, r], w_up [H*d, r] (one row per (head, key channel)), b [H*d].  Blog post-114,
    chapter 4: the gate gives every head and channel its own value computed from the input;
    the page "Kimi K3 注意力三件套" calls it the "up" half of the low-rank projection.  The
    pages name no nonlinearity; -softplus maps the pre-activation onto log(alpha) < 0, i.e.
    alpha = sigmoid(-pre) in (0, 1).  Returns [Ntok, H, d].
    """
    pre = np.asarray(z, np.float64) @ np.asarray(w_up, np.float64).T + np.asarray(b, np.float64)[None, :]
    return (-softplus(pre)).reshape(pre.shape[0], H, d)


def gate_beta(x: np.ndarray, w_beta: np.ndarray) -> np.ndarray:
    """beta = sigmoid(x w_beta^T), fp64: one scalar per token and head (blog post-114, chapter 3
    code: sigmoid of a linear map of x; page "Kimi K3 注意力三件套": beta is a single scalar).
    x [Ntok, Dm], w_beta [H, Dm]; returns [Ntok, H]."""
    return sigmoid(np.asarray(x, np.float64) @ np.asarray(w_beta, np.float64).T)


def gate(x, w_down, w_beta, w_up, b, H: int, d: int):
    """The whole gate in fp64: (z [Ntok, r], beta [Ntok, H], g [Ntok, H, d]), g taken from the
    unrounded z."""
    z = gate_z(x, w_down)
    return z, gate_beta(x, w_beta), gate_g(z, w_up, b, H, d)


# --------------------------------------------------------------------------- Block AttnRes
def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2 over the last axis) + eps), fp64, without a learned scale (a scale
    would multiply the query vector w element-wise, so it is folded into w)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def attnres_logits(V: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Scores of the stored block outputs for one layer's query w: logits[n, t] = w . norm(V[n, t]).

    V [n, T, d] (the blocks' outputs for each token, the last one possibly the partial block),
    w [d].  Blog post-114, chapter 6 (the block AttnRes listing): the stacked block outputs are
    normalised to form the keys and scored against the layer's projection weight."""
    return np.einsum("ntd,d->nt", rms_norm(V, eps), np.asarray(w, np.float64))


def attnres(V: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Block AttnRes read-out for one layer, fp64: h[t] = sum_n softmax_n(logits[:, t]) V[n, t].

    Blog post-114, chapter 6 (softmax of the scores over the blocks, then the weighted sum of
    the blocks); page "Kimi K3 注意力三件套" (AttnRes section: the weights over the blocks sum to
    one and depend on the input).  Returns [T, d]."""
    lg = attnres_logits(V, w, eps)
    a = np.exp(lg - lg.max(axis=0, keepdims=True))
    a /= a.sum(axis=0, keepdims=True)
    return np.einsum("nt,ntd->td", a, np.asarray(V, np.float64))


def attnres_lse(V: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """log sum_n exp(logits[n, t]) over the blocks, [T]: with attnres() the partial result that
    the two-phase inference of the yeyulingfeng page keeps for the online-softmax merge."""
    lg = attnres_logits(V, w, eps)
    m = lg.max(axis=0)
    return m + np.log(np.exp(lg - m[None, :]).sum(axis=0))


# --------------------------------------------------------------------------- segment maps (KCP)
def segment_map(k, v, g, beta):
    """The affine map a segment of one chain applies to the state, fp64: S_out = A S_in + B.

    Blog post-114, chapter 3: the chunked form computes each block's contribution in parallel
    and merges it into the running state serially, and K3's KCP carries the same idea across
    devices; a device's segment is then one large block whose contribution is this map.  Per
    token the recurrence is S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    (decay, then the delta write of the course page's section 3), so
        A = prod over t, latest on the left, of (I - beta_t k_t k_t^T) Diag(alpha_t),
        B = the state the recurrence reaches from S_0 = 0.
    k, g [L, dk]; v [L, dv]; beta [L] (stored values).  Returns (A [dk, dk], B [dk, dv]).
    A is the product written out token by token (numpy); B comes from the C recurrence.
    """
    k, g = np.asarray(k, np.float64), np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    L, dk = k.shape
    A = np.eye(dk)
    for t in range(L):
        A = np.exp(g[t])[:, None] * A                        # Diag(alpha_t) A
        A = A - beta[t] * np.outer(k[t], k[t] @ A)           # (I - beta k k^T) ...
    _, B = chain(np.zeros((L, dk), np.float32), k, v, g, beta, 1.0, None)
    return A, B


def state_combine(A, S, B):
    """One hop of the prefix over segments: the state leaving a segment whose map is (A, B)
    when S enters it, A S + B (fp64)."""
    return np.asarray(A, np.float64) @ np.asarray(S, np.float64) + np.asarray(B, np.float64)
