"""Seeded synthetic inputs for the KDA operator (shared by tests, smoke and bench).

This module only draws random numbers and rounds them to their storage type.
It holds none of the operator's arithmetic, so both the fp64 oracle and the
HIP path can consume its output without sharing any method code.

Distributions (one reading of the workloads described for the operator):
  q, k   ~ N(0, 1), then divided by their L2 norm over the head dimension
           (computed in fp64 before rounding to the storage type);
  v      ~ N(0, 1);
  beta   = sigmoid(N(0, 1))                      (fp32, one scalar per token and head);
  g      = log(alpha) = -softplus(N(0, 1) + 2)   (fp32, one value per key channel);
  S_0    ~ N(0, std) with std 0.02 where the workload has an initial state.
The second argument of N(., .) is a standard deviation.  A "weak decay"
variant uses -softplus(N(0,1) - 5) (alpha close to 1) to stress long-range
state propagation.

Draw order for one generator: q, k, v, x_beta, x_alpha, S_0.
Rounding to bf16 is round-to-nearest-even on the fp32 value.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 93000
CHUNK = 64


# --------------------------------------------------------------------------- bf16 storage
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, kept in fp32 storage."""
    return bf16_to_f32(bf16_bits(x))


def _store(x: np.ndarray, io: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if io == "bf16" else x


def _softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) in fp64 (numpy's overflow-free logaddexp)."""
    return np.logaddexp(0.0, x.astype(np.float64))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x.astype(np.float64)))


def _blocks(n: int, block: int):
    return [(s, min(s + block, n)) for s in range(0, n, block)]


def _parallel(fn, n: int, block: int):
    """Run fn(s, e) over row blocks [s, e) on a few threads (numpy ufuncs release the GIL).
    Every block is an independent elementwise or per-row computation, so the result does
    not depend on the blocking."""
    bl = _blocks(n, block)
    if len(bl) <= 1:
        for s, e in bl:
            fn(s, e)
        return
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, len(bl))) as ex:
        list(ex.map(lambda se: fn(*se), bl))


def _unit_rows(x: np.ndarray, block: int = 1 << 18) -> np.ndarray:
    """Divide each last-axis row by its L2 norm (fp64 norm), returned as fp32."""
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape, dtype=np.float32)

    def blk(s, e):
        b = flat[s:e].astype(np.float64)
        nrm = np.sqrt(np.sum(b * b, axis=-1, keepdims=True))
        out[s:e] = (b / np.maximum(nrm, 1e-300)).astype(np.float32)
    _parallel(blk, flat.shape[0], block)
    return out.reshape(x.shape)


def _map_f32(fn, x: np.ndarray, block: int = 1 << 24) -> np.ndarray:
    """fp32 array of fn(x) (fn evaluated in fp64), computed over flat blocks."""
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float32)

    def blk(s, e):
        out[s:e] = fn(flat[s:e]).astype(np.float32)
    _parallel(blk, flat.shape[0], block)
    return out.reshape(x.shape)


def _store_bf16_inplace(x: np.ndarray, block: int = 1 << 24) -> np.ndarray:
    flat = x.reshape(-1)

    def blk(s, e):
        flat[s:e] = bf16_round(flat[s:e])
    _parallel(blk, flat.shape[0], block)
    return x


# --------------------------------------------------------------------------- containers
@dataclasses.dataclass
class KDAInputs:
    """One batch of operator inputs, all in fp32 storage (bf16-valued when io == 'bf16').

    Layout: q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
    S0 [N, H, dk, dv] or None; cu_seqlens [N + 1] int32 or None (then B == 1).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    S0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    io: str
    scale: float = 1.0

    @property
    def B(self): return self.q.shape[0]
    @property
    def T(self): return self.q.shape[1]
    @property
    def H(self): return self.q.shape[2]
    @property
    def dk(self): return self.q.shape[3]
    @property
    def dv(self): return self.v.shape[3]
    @property
    def N(self):
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def seq_bounds(self, n: int):
        """(batch index, first token, length) of sequence n."""
        if self.cu_seqlens is None:
            return n, 0, self.T
        s, e = int(self.cu_seqlens[n]), int(self.cu_seqlens[n + 1])
        return 0, s, e - s


def draw_tokens(rng: np.random.Generator, shape_tok, H: int, dk: int, dv: int, io: str,
                g_shift: float = 2.0, normalize_qk: bool = True):
    """Draw q, k, v, beta, g for tokens of shape `shape_tok` (e.g. (B, T)), in the fixed order."""
    q = rng.standard_normal((*shape_tok, H, dk), dtype=np.float32)
    k = rng.standard_normal((*shape_tok, H, dk), dtype=np.float32)
    v = rng.standard_normal((*shape_tok, H, dv), dtype=np.float32)
    xb = rng.standard_normal((*shape_tok, H), dtype=np.float32)
    xa = rng.standard_normal((*shape_tok, H, dk), dtype=np.float32)
    if normalize_qk:
        q = _unit_rows(q)
        k = _unit_rows(k)
    beta = _map_f32(_sigmoid, xb)
    g = _map_f32(lambda a: -_softplus(a.astype(np.float64) + g_shift), xa)
    if io == "bf16":
        q, k, v = (_store_bf16_inplace(a) for a in (q, k, v))
    return q, k, v, beta, g


def make_dense(B: int, T: int, H: int, dk: int, dv: int, io: str, seed: int,
               s0_std: Optional[float] = None, g_shift: float = 2.0) -> KDAInputs:
    rng = np.random.default_rng(seed)
    q, k, v, beta, g = draw_tokens(rng, (B, T), H, dk, dv, io, g_shift)
    S0 = None
    if s0_std is not None:
        S0 = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(s0_std))
    return KDAInputs(q, k, v, g, beta, S0, None, io)


def varlen_lengths(n_seq: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=n_seq, endpoint=True).astype(np.int64)


def make_varlen(lengths, H: int, dk: int, dv: int, io: str, seed: int,
                s0_std: Optional[float] = 0.02, g_shift: float = 2.0,
                normalize_qk: bool = True) -> KDAInputs:
    """Packed batch: sequence n is drawn from default_rng([seed, n]) (q, k, v, beta, g, S0)."""
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    Ttot = int(cu[-1])
    q = np.empty((1, Ttot, H, dk), np.float32)
    k = np.empty((1, Ttot, H, dk), np.float32)
    v = np.empty((1, Ttot, H, dv), np.float32)
    g = np.empty((1, Ttot, H, dk), np.float32)
    beta = np.empty((1, Ttot, H), np.float32)
    S0 = np.empty((len(lengths), H, dk, dv), np.float32) if s0_std is not None else None
    for n, L in enumerate(lengths):
        rng = np.random.default_rng([seed, n])
        qn, kn, vn, bn, gn = draw_tokens(rng, (L,), H, dk, dv, io, g_shift, normalize_qk)
        s, e = cu[n], cu[n + 1]
        q[0, s:e], k[0, s:e], v[0, s:e], beta[0, s:e], g[0, s:e] = qn, kn, vn, bn, gn
        if S0 is not None:
            S0[n] = rng.standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    return KDAInputs(q, k, v, g, beta, S0, cu.astype(np.int32), io)


def decode_step_inputs(N: int, H: int, d: int, io: str, seed: int, step: int,
                       g_shift: float = 2.0):
    """Token inputs of one decode step: q, k, v [N, H, d], g [N, H, d], beta [N, H]."""
    rng = np.random.default_rng([seed, step])
    q, k, v, beta, g = draw_tokens(rng, (N,), H, d, d, io, g_shift)
    return q, k, v, g, beta


def decode_initial_state(N: int, H: int, d: int, seed: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng([seed, 1 << 20])
    return rng.standard_normal((N, H, d, d), dtype=np.float32) * np.float32(std)


def prep_inputs(lengths, H: int, d: int, io: str, seed: int, w_std: float = 0.5, width: int = 4):
    """Raw (un-normalised) x [1, Ntok, H, d] ~ N(0,1), conv weights [H*d, width] ~ N(0, w_std)."""
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((H * d, width), dtype=np.float32) * np.float32(w_std))
    x = np.empty((1, int(cu[-1]), H, d), np.float32)
    for n, L in enumerate(lengths):
        r = np.random.default_rng([seed, n])
        x[0, cu[n]:cu[n + 1]] = _store(r.standard_normal((L, H, d), dtype=np.float32), io)
    return x, w, cu.astype(np.int32)


# --------------------------------------------------------------------------- named workloads
def small_fp32() -> KDAInputs:
    """fp32 recurrence: B=1, H=2, T=256, d=64, S0 = 0."""
    return make_dense(1, 256, 2, 64, 64, "f32", SEED_BASE + 0)


def prefill_batch(g_shift: float = 2.0) -> KDAInputs:
    """Chunked prefill: B=4, H=16, T=4096, d=128, bf16 q/k/v, S0 = 0.  g_shift = -5 draws the
    weak-decay variant (alpha ~ 0.99)."""
    return make_dense(4, 4096, 16, 128, 128, "bf16", SEED_BASE + 1, g_shift=g_shift)


LONG_CONTEXT = dict(B=1, T=131072, H=32, d=128, seed=SEED_BASE + 2)


def long_context(g_shift: float = 2.0) -> KDAInputs:
    """Long-context prefill: B=1, H=32, T=131072, d=128, bf16 q/k/v, S0 ~ N(0, 0.02).  g_shift = -5
    draws the weak-decay variant (alpha ~ 0.99)."""
    c = LONG_CONTEXT
    return make_dense(c["B"], c["T"], c["H"], c["d"], c["d"], "bf16", c["seed"], s0_std=0.02, g_shift=g_shift)


def dense_gate(B: int, T: int, H: int, dk: int, dv: int, seed: int, g_shift: float) -> np.ndarray:
    """The g of make_dense(B, T, H, dk, dv, ., seed, g_shift=g_shift) alone, bitwise: the same
    generator is advanced past the draws of q, k, v and x_beta (not processed), then x_alpha is
    drawn and shifted."""
    rng = np.random.default_rng(seed)
    for shape in ((B, T, H, dk), (B, T, H, dk), (B, T, H, dv), (B, T, H)):
        rng.standard_normal(shape, dtype=np.float32)
    xa = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    return _map_f32(lambda a: -_softplus(a.astype(np.float64) + g_shift), xa)


def long_context_gate(g_shift: float) -> np.ndarray:
    """The g of long_context(g_shift) alone (bitwise)."""
    c = LONG_CONTEXT
    return dense_gate(c["B"], c["T"], c["H"], c["d"], c["d"], c["seed"], g_shift)


DECODE_POOL = dict(N=256, H=32, d=128, steps=100, seed=SEED_BASE + 3)
VARLEN_LAYER = dict(n_seq=64, lo=512, hi=16384, H=32, d=128, seed=SEED_BASE + 4)


def varlen_layer_lengths() -> np.ndarray:
    return varlen_lengths(VARLEN_LAYER["n_seq"], VARLEN_LAYER["lo"], VARLEN_LAYER["hi"], VARLEN_LAYER["seed"])


def varlen_layer_sequence(n: int, H: int = 32, d: int = 128, g_shift: float = 2.0):
    """Sequence n of the varlen layer workload: raw q, k ~ N(0,1) (bf16, before the prologue),
    v ~ N(0,1) bf16, beta, g, and S_0 ~ N(0, 0.02), all from default_rng([seed, n])."""
    L = int(varlen_layer_lengths()[n])
    rng = np.random.default_rng([VARLEN_LAYER["seed"], n])
    q, k, v, beta, g = draw_tokens(rng, (L,), H, d, d, "bf16", g_shift, normalize_qk=False)
    S0 = rng.standard_normal((H, d, d), dtype=np.float32) * np.float32(0.02)
    return q, k, v, beta, g, S0


def varlen_layer_conv_weights(H: int = 32, d: int = 128, width: int = 4):
    """w_q, w_k [H*d, width] ~ N(0, 0.5), drawn after the lengths from the workload seed."""
    rng = np.random.default_rng(VARLEN_LAYER["seed"])
    rng.integers(VARLEN_LAYER["lo"], VARLEN_LAYER["hi"], size=VARLEN_LAYER["n_seq"], endpoint=True)
    wq = rng.standard_normal((H * d, width), dtype=np.float32) * np.float32(0.5)
    wk = rng.standard_normal((H * d, width), dtype=np.float32) * np.float32(0.5)
    return wq, wk


def make_scalar_gate(lengths, H: int, d: int, io: str, seed: int, s0_std: Optional[float] = 0.02,
                     g_shift: float = 2.0, dense_B: Optional[int] = None, with_gate: bool = True):
    """Inputs for the one-decay-per-head case: like make_varlen / make_dense but g is [B, T, H]
    (g = -softplus(N(0,1) + g_shift) per token and head), or None when with_gate is False.
    Dense when dense_B is given (then lengths is [T]).  Draw order per sequence: q, k, v,
    x_beta, x_alpha (one per token and head), S_0."""
    if dense_B is not None:
        T = int(lengths[0])
        rng = np.random.default_rng(seed)
        q = _unit_rows(rng.standard_normal((dense_B, T, H, d), dtype=np.float32))
        k = _unit_rows(rng.standard_normal((dense_B, T, H, d), dtype=np.float32))
        v = rng.standard_normal((dense_B, T, H, d), dtype=np.float32)
        xb = rng.standard_normal((dense_B, T, H), dtype=np.float32)
        xa = rng.standard_normal((dense_B, T, H), dtype=np.float32)
        S0 = None if s0_std is None else rng.standard_normal((dense_B, H, d, d), dtype=np.float32) * np.float32(s0_std)
        beta = _map_f32(_sigmoid, xb)
        g = _map_f32(lambda a: -_softplus(a.astype(np.float64) + g_shift), xa) if with_gate else None
        return KDAInputs(_store(q, io), _store(k, io), _store(v, io), g, beta, S0, None, io)
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    Ttot = int(cu[-1])
    q = np.empty((1, Ttot, H, d), np.float32)
    k = np.empty((1, Ttot, H, d), np.float32)
    v = np.empty((1, Ttot, H, d), np.float32)
    beta = np.empty((1, Ttot, H), np.float32)
    g = np.empty((1, Ttot, H), np.float32) if with_gate else None
    S0 = np.empty((len(lengths), H, d, d), np.float32) if s0_std is not None else None
    for n, L in enumerate(lengths):
        rng = np.random.default_rng([seed, n])
        s, e = cu[n], cu[n + 1]
        q[0, s:e] = _store(_unit_rows(rng.standard_normal((L, H, d), dtype=np.float32)), io)
        k[0, s:e] = _store(_unit_rows(rng.standard_normal((L, H, d), dtype=np.float32)), io)
        v[0, s:e] = _store(rng.standard_normal((L, H, d), dtype=np.float32), io)
        beta[0, s:e] = _map_f32(_sigmoid, rng.standard_normal((L, H), dtype=np.float32))
        xa = rng.standard_normal((L, H), dtype=np.float32)
        if with_gate:
            g[0, s:e] = _map_f32(lambda a: -_softplus(a.astype(np.float64) + g_shift), xa)
        if S0 is not None:
            S0[n] = rng.standard_normal((H, d, d), dtype=np.float32) * np.float32(s0_std)
    return KDAInputs(q, k, v, g, beta, S0, cu.astype(np.int32), io)


def broadcast_gate(g_scalar: Optional[np.ndarray], like: np.ndarray) -> np.ndarray:
    """Per-channel log-decay array [..., H, d_k] equal to the per-head g on every channel (zeros for
    g = None, i.e. alpha = 1)."""
    if g_scalar is None:
        return np.zeros(like.shape, np.float32)
    return np.ascontiguousarray(np.broadcast_to(g_scalar[..., None], like.shape), dtype=np.float32)


# --------------------------------------------------------------------------- low-rank gate inputs
def gate_weights(Dm: int, H: int, d: int, r: int, seed: int, b_mean: float = 2.0, b_std: float = 0.5):
    """Synthetic weights of the low-rank gate, bf16 values in fp32 storage except b (fp32):
    w_down [r, Dm] and w_beta [H, Dm] ~ N(0, 1/Dm), w_up [H*d, r] ~ N(0, 1/r), b [H*d] ~ N(b_mean,
    b_std).  With x ~ N(0, 1) both projections are then about N(0, 1), so the gate's pre-activation
    is about N(b_mean, 1.1): the log-decay distribution of the other workloads (b_mean = 2), or a
    weak decay (b_mean = -5).  Draw order: w_down, w_beta, w_up, b."""
    rng = np.random.default_rng([seed, 1])
    w_down = bf16_round(rng.standard_normal((r, Dm), dtype=np.float32) / np.float32(np.sqrt(Dm)))
    w_beta = bf16_round(rng.standard_normal((H, Dm), dtype=np.float32) / np.float32(np.sqrt(Dm)))
    w_up = bf16_round(rng.standard_normal((H * d, r), dtype=np.float32) / np.float32(np.sqrt(r)))
    b = (np.float32(b_mean) + np.float32(b_std) * rng.standard_normal(H * d, dtype=np.float32)).astype(np.float32)
    return w_down, w_beta, w_up, b


def gate_hidden(Ntok: int, Dm: int, seed: int) -> np.ndarray:
    """Hidden states x [Ntok, Dm] ~ N(0, 1), bf16 values in fp32 storage."""
    rng = np.random.default_rng([seed, 2])
    return _store_bf16_inplace(rng.standard_normal((Ntok, Dm), dtype=np.float32))


@dataclasses.dataclass
class LowRankInputs:
    """Operator inputs with the gate given by its rank-r down projection z instead of g:
    q, k, v [B, T, H, d] (bf16 values), beta [B, T, H], z [B, T, r] (bf16 values), w_up [H*d, r]
    (bf16 values), b [H*d], S0 [N, H, d, d] or None, cu_seqlens or None."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    z: np.ndarray
    w_up: np.ndarray
    b: np.ndarray
    S0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]

    @property
    def shape(self):
        return self.q.shape


def make_lowrank(B: int, T: int, H: int, d: int, r: int, seed: int, s0_std: Optional[float] = 0.02,
                 b_mean: float = 2.0, lengths=None) -> LowRankInputs:
    """bf16 inputs for the low-rank-gate forward.  Dense [B, T] when lengths is None, else packed
    (B = 1, T = sum(lengths)).  Draw order: q, k, v, x_beta, z, S_0; then the gate weights from
    gate_weights(seed) (w_up and b are used; w_down and w_beta belong to the prologue)."""
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        B, T = 1, int(cu[-1])
    q = _unit_rows(rng.standard_normal((B, T, H, d), dtype=np.float32))
    k = _unit_rows(rng.standard_normal((B, T, H, d), dtype=np.float32))
    v = rng.standard_normal((B, T, H, d), dtype=np.float32)
    beta = _map_f32(_sigmoid, rng.standard_normal((B, T, H), dtype=np.float32))
    z = rng.standard_normal((B, T, r), dtype=np.float32)
    N = B if cu is None else len(cu) - 1
    S0 = None if s0_std is None else rng.standard_normal((N, H, d, d), dtype=np.float32) * np.float32(s0_std)
    _, _, w_up, b = gate_weights(H * d, H, d, r, seed, b_mean=b_mean)
    return LowRankInputs(bf16_round(q), bf16_round(k), bf16_round(v), beta, bf16_round(z), w_up, b, S0, cu)


# --------------------------------------------------------------------------- Block AttnRes inputs
def attnres_inputs(n: int, T: int, d: int, L: int, seed: int, score_std: float = 1.5):
    """Block outputs V [n, T, d] (bf16 values in fp32 storage; block b ~ N(0, (1 + b/2)^2), so the
    blocks differ in scale as residual streams grow with depth) and L layer queries W [L, d]
    ~ N(0, score_std^2 / d) (bf16 values), so that w . norm(V) ~ N(0, score_std^2).
    Draw order: V (block by block), W."""
    rng = np.random.default_rng([seed, 3])
    V = np.empty((n, T, d), np.float32)
    for b in range(n):
        V[b] = rng.standard_normal((T, d), dtype=np.float32) * np.float32(1.0 + 0.5 * b)
    _store_bf16_inplace(V)
    W = bf16_round(rng.standard_normal((L, d), dtype=np.float32) * np.float32(score_std / np.sqrt(d)))
    return V, W
