"""Python binding of libkda.so, the MI355X Kimi Delta Attention operator (C ABI in include/kda.h).

Argument marshalling only: every step of the operator runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU fallback: if the
library is missing, importing works but the first call raises.

    o, S = fwd(q, k, v, g, beta, scale=1.0, initial_state=None, cu_seqlens=None)
    o, S = fwd_scalar_gate(q, k, v, g_or_None, beta, ...)    # g [B, T, H]: one decay per head
    o, S = fwd_lowrank_gate(q, k, v, z, w_up, b_gate, beta, ...)  # log(alpha) formed from z
    o    = decode_step(q, k, v, g, beta, state, scale=1.0)     # state updated in place
    y    = prep(x, conv_w, cu_seqlens=None)
    z, beta, g = gate(x, w_down, w_beta, w_up=None, b_gate=None, H=..., want_g=False)
    h          = attnres(blocks, w, eps)                     # Block AttnRes read-out
    o, lse     = attnres_inter(blocks, W, eps)               # phase 1 for L layers
    h          = attnres_merge(partial, w, o_l, lse_l, eps)  # phase 2 for one layer
    A, B       = fwd_segment_map(fwd_chunk_local(...), ...)  # S_out = A S_in + B per chain
    S_next     = state_combine(A, S_in, B)                 # one hop between segments
    o, S, ...  = fwd_segmented(q, k, v, g, beta, seg_bounds)  # one sequence in P segments

Layouts: q, k, g [B, T, H, dk]; v, o [B, T, H, dv]; beta [B, T, H]; states [N, H, dk, dv]
fp32 with element (i, j) mapping key channel i to value channel j (o = S^T q).  q, k, v
(and x) are bfloat16 or float32; g = log(alpha), beta and states are float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_LAUNCH, KDA_ERR_TOO_LARGE = range(6)
KDA_F32, KDA_BF16 = 0, 1

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               "g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.kda_status_string.argtypes = [I]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        L.kda_fwd_workspace_bytes.restype = S
        L.kda_fwd_workspace_min_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
        L.kda_fwd_workspace_min_bytes.restype = S
        L.kda_fwd.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, P, F, P, P, P, P, S, P]
        L.kda_fwd.restype = I
        L.kda_fwd_scalar_gate.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, P, F, P, P, P, P, S, P]
        L.kda_fwd_scalar_gate.restype = I
        L.kda_fwd_chunk_local.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, P, P, S, P]
        L.kda_fwd_chunk_local.restype = I
        L.kda_fwd_state_scan.argtypes = [I, I, I, I, I, I, P, I, F, P, P, P, P, S, P]
        L.kda_fwd_state_scan.restype = I
        L.kda_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, F, P, P, P]
        L.kda_decode_step.restype = I
        L.kda_prep.argtypes = [I, I, I, I, I, P, I, P, P, I, P, P]
        L.kda_prep.restype = I
        L.kda_gate.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.kda_gate.restype = I
        L.kda_fwd_lowrank_gate.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, I, P, P, P, F, P, P, P, P, S, P]
        L.kda_fwd_lowrank_gate.restype = I
        L.kda_attnres.argtypes = [I, I, I, I, P, P, F, P, P]
        L.kda_attnres.restype = I
        L.kda_attnres_inter_workspace_bytes.argtypes = [I, I, I]
        L.kda_attnres_inter_workspace_bytes.restype = S
        L.kda_attnres_inter.argtypes = [I, I, I, I, I, P, P, F, P, P, P, S, P]
        L.kda_attnres_inter.restype = I
        L.kda_attnres_merge.argtypes = [I, I, I, P, P, F, P, P, P, P]
        L.kda_attnres_merge.restype = I
        L.kda_fwd_chunk_local_scalar_gate.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, P, P, S, P]
        L.kda_fwd_chunk_local_scalar_gate.restype = I
        L.kda_fwd_chunk_local_lowrank_gate.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, I, P, P, P, P, S, P]
        L.kda_fwd_chunk_local_lowrank_gate.restype = I
        L.kda_fwd_segment_map.argtypes = [I, I, I, I, I, I, P, I, P, P, P, S, P]
        L.kda_fwd_segment_map.restype = I
        L.kda_state_combine.argtypes = [I, I, I, P, P, P, P, P]
        L.kda_state_combine.restype = I
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().kda_status_string(int(code)).decode()


def _check(code: int):
    if code != KDA_OK:
        raise KDAError(code, status_string(code))


def _torch():
    import torch
    return torch


def _io_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def fwd_workspace_bytes(io: int, B: int, T: int, H: int, dk: int, dv: int, N: int, varlen: bool) -> int:
    """Workspace for the prefill in one pass (kda_fwd_workspace_bytes)."""
    return int(lib().kda_fwd_workspace_bytes(io, B, T, H, dk, dv, N, 1 if varlen else 0))


def fwd_workspace_min_bytes(io: int, B: int, T: int, H: int, dk: int, dv: int, N: int, varlen: bool,
                            have_final_state: bool) -> int:
    """Smallest workspace the prefill accepts; less than fwd_workspace_bytes runs it in windows
    (kda_fwd_workspace_min_bytes)."""
    return int(lib().kda_fwd_workspace_min_bytes(io, B, T, H, dk, dv, N, 1 if varlen else 0,
                                                 1 if have_final_state else 0))


def fwd(q, k, v, g, beta, scale: float = 1.0, initial_state=None, cu_seqlens=None,
        output_final_state: bool = True, o=None, final_state=None, workspace=None,
        stream=None) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunked prefill (kda_fwd).  Returns (o, final_state or None)."""
    return _fwd("channel", q, k, v, g, beta, scale, initial_state, cu_seqlens, output_final_state, o,
                final_state, workspace, stream)


def fwd_scalar_gate(q, k, v, g, beta, scale: float = 1.0, initial_state=None, cu_seqlens=None,
                    output_final_state: bool = True, o=None, final_state=None, workspace=None,
                    stream=None) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunked prefill with one log-decay per token and head, g [B, T, H], or g = None for
    alpha = 1 (kda_fwd_scalar_gate).  Returns (o, final_state or None)."""
    return _fwd("scalar", q, k, v, g, beta, scale, initial_state, cu_seqlens, output_final_state, o,
                final_state, workspace, stream)


def fwd_lowrank_gate(q, k, v, z, w_up, b_gate, beta, scale: float = 1.0, initial_state=None, cu_seqlens=None,
                     output_final_state: bool = True, o=None, final_state=None, workspace=None,
                     stream=None) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunked prefill with the gate in low-rank form (kda_fwd_lowrank_gate): z [B, T, r] bf16,
    w_up [H*dk, r] bf16, b_gate [H*dk] fp32; log(alpha) = -softplus(z w_up^T + b_gate) is formed in
    the kernel.  Returns (o, final_state or None)."""
    return _fwd("lowrank", q, k, v, None, beta, scale, initial_state, cu_seqlens, output_final_state, o,
                final_state, workspace, stream, lowrank=(z, w_up, b_gate))


def gate(x, w_down, w_beta, w_up=None, b_gate=None, H: Optional[int] = None, want_g: bool = False,
         z=None, beta=None, g=None, stream=None):
    """Gate prologue (kda_gate) for x [Ntok, Dm] bf16: returns (z [Ntok, r] bf16, beta [Ntok, H] fp32,
    g [Ntok, H, dk] fp32 or None).  w_down [r, Dm], w_beta [H, Dm], w_up [H*dk, r] (bf16), b_gate
    [H*dk] fp32; w_up and b_gate are needed only for g."""
    torch = _torch()
    Ntok, Dm = x.shape
    r = w_down.shape[0]
    H = w_beta.shape[0] if H is None else H
    _need(x, "x", torch.bfloat16)
    _need(w_down, "w_down", torch.bfloat16, (r, Dm))
    _need(w_beta, "w_beta", torch.bfloat16, (H, Dm))
    dk = 128
    if w_up is not None:
        dk = w_up.shape[0] // H
        _need(w_up, "w_up", torch.bfloat16, (H * dk, r))
    if want_g:
        _need(w_up, "w_up", torch.bfloat16)
        _need(b_gate, "b_gate", torch.float32, (H * dk,))
    z = torch.empty((Ntok, r), dtype=torch.bfloat16, device=x.device) if z is None else _need(z, "z", torch.bfloat16, (Ntok, r))
    beta = torch.empty((Ntok, H), dtype=torch.float32, device=x.device) if beta is None else _need(beta, "beta", torch.float32, (Ntok, H))
    if want_g and g is None:
        g = torch.empty((Ntok, H, dk), dtype=torch.float32, device=x.device)
    elif g is not None:
        _need(g, "g", torch.float32, (Ntok, H, dk))
    _check(lib().kda_gate(KDA_BF16, Ntok, Dm, H, dk, r, _ptr(x), _ptr(w_down), _ptr(w_beta), _ptr(w_up),
                          _ptr(b_gate), _ptr(z), _ptr(beta), _ptr(g), _stream(stream)))
    return z, beta, g


def _fwd(kind, q, k, v, g, beta, scale, initial_state, cu_seqlens, output_final_state, o,
         final_state, workspace, stream, lowrank=None):
    torch = _torch()
    io = _io_dtype(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, dk))
    _need(v, "v", q.dtype, (B, T, H, dv))
    if kind == "scalar":
        if g is not None:
            _need(g, "g", torch.float32, (B, T, H))
    elif kind == "lowrank":
        z, w_up, b_gate = lowrank
        r = z.shape[-1]
        _need(z, "z", torch.bfloat16, (B, T, r))
        _need(w_up, "w_up", torch.bfloat16, (H * dk, r))
        _need(b_gate, "b_gate", torch.float32, (H * dk,))
    else:
        _need(g, "g", torch.float32, (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    else:
        _need(o, "o", q.dtype, (B, T, H, dv))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    need = fwd_workspace_bytes(io, B, T, H, dk, dv, N, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if kind == "lowrank":
        _check(lib().kda_fwd_lowrank_gate(io, B, T, H, dk, dv, _ptr(cu_seqlens), N,
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(z), r, _ptr(w_up), _ptr(b_gate),
                                          _ptr(beta), float(scale), _ptr(initial_state), _ptr(final_state),
                                          _ptr(o), _ptr(workspace), workspace.numel(), _stream(stream)))
        return o, final_state
    fn = lib().kda_fwd_scalar_gate if kind == "scalar" else lib().kda_fwd
    _check(fn(io, B, T, H, dk, dv, _ptr(cu_seqlens), N,
              _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
              _ptr(initial_state), _ptr(final_state), _ptr(o),
              _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, final_state


def fwd_chunk_local(q, k, v, g, beta, cu_seqlens=None, workspace=None, stream=None, gate="channel",
                    lowrank=None):
    """First phase of the prefill: the chunk records, into `workspace` (returned).
    gate "channel" (kda_fwd_chunk_local, g [B, T, H, dk]), "scalar" (kda_fwd_chunk_local_scalar_gate,
    g [B, T, H] or None) or "lowrank" (kda_fwd_chunk_local_lowrank_gate, g None and
    lowrank = (z, w_up, b_gate)).  The records feed fwd_state_scan and fwd_segment_map alike."""
    torch = _torch()
    io = _io_dtype(q)
    B, T, H, dk = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (B, T, H, dk))
    _need(v, "v", q.dtype, (B, T, H, dk))
    if gate == "channel":
        _need(g, "g", torch.float32, (B, T, H, dk))
    elif gate == "scalar":
        if g is not None:
            _need(g, "g", torch.float32, (B, T, H))
    elif gate == "lowrank":
        z, w_up, b_gate = lowrank
        r = z.shape[-1]
        _need(z, "z", torch.bfloat16, (B, T, r))
        _need(w_up, "w_up", torch.bfloat16, (H * dk, r))
        _need(b_gate, "b_gate", torch.float32, (H * dk,))
    else:
        raise ValueError(f"unknown gate form {gate!r}")
    _need(beta, "beta", torch.float32, (B, T, H))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
    need = fwd_workspace_bytes(io, B, T, H, dk, dk, N, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    head = (io, B, T, H, dk, dk, _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v))
    tail = (_ptr(beta), _ptr(workspace), workspace.numel(), _stream(stream))
    if gate == "channel":
        _check(lib().kda_fwd_chunk_local(*head, _ptr(g), *tail))
    elif gate == "scalar":
        _check(lib().kda_fwd_chunk_local_scalar_gate(*head, _ptr(g), *tail))
    else:
        _check(lib().kda_fwd_chunk_local_lowrank_gate(*head, _ptr(z), r, _ptr(w_up), _ptr(b_gate), *tail))
    return workspace


def fwd_state_scan(workspace, io: int, B: int, T: int, H: int, dk: int, cu_seqlens=None, scale: float = 1.0,
                   initial_state=None, o=None, final_state=None, stream=None):
    """Second phase of kda_fwd (kda_fwd_state_scan) over the records in `workspace`.
    Returns (o [B, T, H, dk], final_state [N, H, dk, dk])."""
    torch = _torch()
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = torch.bfloat16 if io == KDA_BF16 else torch.float32
    dev = workspace.device
    o = torch.empty((B, T, H, dk), dtype=dt, device=dev) if o is None else _need(o, "o", dt, (B, T, H, dk))
    if final_state is None:
        final_state = torch.empty((N, H, dk, dk), dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, (N, H, dk, dk))
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, dk, dk))
    _check(lib().kda_fwd_state_scan(io, B, T, H, dk, dk, _ptr(cu_seqlens), N, float(scale), _ptr(initial_state),
                                    _ptr(final_state), _ptr(o), _ptr(workspace), workspace.numel(),
                                    _stream(stream)))
    return o, final_state


def fwd_segment_map(workspace, io: int, B: int, T: int, H: int, dk: int, cu_seqlens=None,
                    transition=None, offset=None, stream=None):
    """Affine map S_out = A S_in + B of every chain (kda_fwd_segment_map), from the records that
    fwd_chunk_local left in `workspace`.  Returns (A [N, H, dk, dk], B [N, H, dk, dk])."""
    torch = _torch()
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dev = workspace.device
    if transition is None:
        transition = torch.empty((N, H, dk, dk), dtype=torch.float32, device=dev)
    if offset is None:
        offset = torch.empty((N, H, dk, dk), dtype=torch.float32, device=dev)
    _need(transition, "transition", torch.float32, (N, H, dk, dk))
    _need(offset, "offset", torch.float32, (N, H, dk, dk))
    _check(lib().kda_fwd_segment_map(io, B, T, H, dk, dk, _ptr(cu_seqlens), N, _ptr(transition), _ptr(offset),
                                     _ptr(workspace), workspace.numel(), _stream(stream)))
    return transition, offset


def state_combine(transition, state_in, offset=None, out=None, stream=None):
    """out = transition @ state_in + offset over the leading dimensions (kda_state_combine, fp32);
    offset None is zero (then the call composes two transitions)."""
    torch = _torch()
    d = transition.shape[-1]
    lead = tuple(transition.shape[:-2])
    _need(transition, "transition", torch.float32)
    _need(state_in, "state_in", torch.float32, transition.shape)
    if offset is not None:
        _need(offset, "offset", torch.float32, transition.shape)
    out = torch.empty_like(state_in) if out is None else out
    if offset is None or out.data_ptr() != offset.data_ptr():
        _need(out, "out", torch.float32, transition.shape)
    count = 1
    for x in lead:
        count *= int(x)
    _check(lib().kda_state_combine(count, d, d, _ptr(transition), _ptr(state_in), _ptr(offset), _ptr(out),
                                   _stream(stream)))
    return out


def fwd_segmented(q, k, v, g, beta, seg_bounds, scale: float = 1.0, initial_state=None, stream=None,
                  gate="channel", lowrank=None):
    """One sequence (B = 1) split at `seg_bounds` (int32 device tensor [P + 1], 0 .. T) into P
    segments and run as a context-parallel job would run it, here on one device: the chunk
    records and the affine map of every segment (all segments at once), the P - 1 hops of the
    prefix over segments (kda_state_combine, serial), then the state scan of every segment from
    its incoming state.  `gate` and `lowrank` select the gate form as in fwd_chunk_local.
    Returns (o [1, T, H, dk], final_state [1, H, dk, dk], transition, offset, incoming states
    [P, H, dk, dk])."""
    torch = _torch()
    io = _io_dtype(q)
    B, T, H, dk = q.shape
    if B != 1:
        raise ValueError("fwd_segmented takes one sequence (B = 1)")
    P = seg_bounds.numel() - 1
    if P < 1:
        raise ValueError("seg_bounds needs at least two entries (one segment)")
    ws = fwd_chunk_local(q, k, v, g, beta, seg_bounds, stream=stream, gate=gate, lowrank=lowrank)
    A, Bm = fwd_segment_map(ws, io, 1, T, H, dk, seg_bounds, stream=stream)
    S_in = torch.empty((P, H, dk, dk), dtype=torch.float32, device=q.device)
    if initial_state is None:
        S_in[0].zero_()
    else:
        S_in[0].copy_(_need(initial_state, "initial_state", torch.float32, (1, H, dk, dk))[0])
    for j in range(P - 1):
        state_combine(A[j], S_in[j], Bm[j], out=S_in[j + 1], stream=stream)
    o, S_out = fwd_state_scan(ws, io, 1, T, H, dk, seg_bounds, scale, S_in, stream=stream)
    return o, S_out[P - 1:P], A, Bm, S_in


def decode_step(q, k, v, g, beta, state, scale: float = 1.0, o=None, stream=None):
    """One token for N sequences (kda_decode_step); `state` [N, H, dk, dv] is updated in place."""
    torch = _torch()
    io = _io_dtype(q)
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", q.dtype)
    _need(k, "k", q.dtype, (N, H, dk))
    _need(v, "v", q.dtype, (N, H, dv))
    _need(g, "g", torch.float32, (N, H, dk))
    _need(beta, "beta", torch.float32, (N, H))
    _need(state, "state", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    else:
        _need(o, "o", q.dtype, (N, H, dv))
    _check(lib().kda_decode_step(io, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 float(scale), _ptr(state), _ptr(o), _stream(stream)))
    return o


def prep(x, conv_w, cu_seqlens=None, y=None, stream=None):
    """q/k prologue (kda_prep): causal depthwise conv (width conv_w.shape[1]) -> SiLU -> L2 norm."""
    torch = _torch()
    io = _io_dtype(x)
    B, T, H, d = x.shape
    W = conv_w.shape[1]
    _need(x, "x", x.dtype)
    _need(conv_w, "conv_w", torch.float32, (H * d, W))
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, tuple(x.shape))
    _check(lib().kda_prep(io, B, T, H, d, _ptr(cu_seqlens), N, _ptr(x), _ptr(conv_w), W, _ptr(y),
                          _stream(stream)))
    return y


def _block_ptrs(blocks):
    """blocks: a list of [T, d] bf16 device tensors, or one [n, T, d] tensor -> (ctypes array, n, T, d)."""
    torch = _torch()
    if isinstance(blocks, torch.Tensor):
        blocks = list(blocks.unbind(0))
    if not blocks:
        raise ValueError("at least one block is required")
    T, d = blocks[0].shape
    for i, b in enumerate(blocks):
        _need(b, f"blocks[{i}]", torch.bfloat16, (T, d))
    arr = (ctypes.c_void_p * len(blocks))(*[b.data_ptr() for b in blocks])
    return arr, len(blocks), T, d


def attnres(blocks, w, eps: float = 1e-6, h=None, stream=None):
    """Block AttnRes read-out of one layer (kda_attnres): h [T, d] = sum_n softmax_n(w . norm(V_n)) V_n."""
    torch = _torch()
    arr, n, T, d = _block_ptrs(blocks)
    _need(w, "w", torch.bfloat16, (d,))
    h = torch.empty((T, d), dtype=torch.bfloat16, device=w.device) if h is None else _need(h, "h", torch.bfloat16, (T, d))
    _check(lib().kda_attnres(KDA_BF16, n, T, d, arr, _ptr(w), float(eps), _ptr(h), _stream(stream)))
    return h


def attnres_inter(blocks, W, eps: float = 1e-6, o=None, lse=None, workspace=None, stream=None):
    """Phase 1 of the two-phase AttnRes (kda_attnres_inter) for the L = W.shape[0] layers:
    returns (o [L, T, d] bf16, lse [L, T] fp32)."""
    torch = _torch()
    arr, n, T, d = _block_ptrs(blocks)
    L = W.shape[0]
    _need(W, "W", torch.bfloat16, (L, d))
    o = torch.empty((L, T, d), dtype=torch.bfloat16, device=W.device) if o is None else _need(o, "o", torch.bfloat16, (L, T, d))
    lse = torch.empty((L, T), dtype=torch.float32, device=W.device) if lse is None else _need(lse, "lse", torch.float32, (L, T))
    need = int(lib().kda_attnres_inter_workspace_bytes(n, L, T))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=W.device)
    _check(lib().kda_attnres_inter(KDA_BF16, n, L, T, d, arr, _ptr(W), float(eps), _ptr(o), _ptr(lse),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, lse


def attnres_merge(partial, w, o_l, lse_l, eps: float = 1e-6, h=None, stream=None):
    """Phase 2 for one layer (kda_attnres_merge): merges the partial block [T, d] into the layer's
    phase-1 result (o_l [T, d], lse_l [T]); returns h [T, d]."""
    torch = _torch()
    T, d = partial.shape
    _need(partial, "partial", torch.bfloat16, (T, d))
    _need(w, "w", torch.bfloat16, (d,))
    _need(o_l, "o_l", torch.bfloat16, (T, d))
    _need(lse_l, "lse_l", torch.float32, (T,))
    h = torch.empty_like(partial) if h is None else _need(h, "h", torch.bfloat16, (T, d))
    _check(lib().kda_attnres_merge(KDA_BF16, T, d, _ptr(partial), _ptr(w), float(eps), _ptr(o_l), _ptr(lse_l),
                                   _ptr(h), _stream(stream)))
    return h
