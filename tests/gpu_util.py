"""Helpers for the GPU parity tests: device uploads and the error measures.

Error measures (the fp64 oracle output is the reference r, never rounded):
  fp32 path:          rel_inf(y, r)     = max|y - r| / max|r|                      (gate 1e-4)
  bf16 path, o:       floored_rel(y, r) = max_i |y_i - r_i| / max(|r_i|, rms(r))   (gate 2e-2)
  bf16 path, states:  rms_rel(y, r)     = max|y - r| / rms(r)                      (gate 2e-2)
The bf16 output gate is a maximum relative error whose denominator is floored at the RMS of the
reference, so elements far below the RMS are held to an absolute error of 2e-2 * RMS: the
output is stored in bf16 and heavy-tailed, so rounding the exact answer alone gives
max|y - r| / rms(r) of ~0.04.  States are stored in fp32, so they take the normalised-by-RMS
bound as it stands (err_state).
"""
from __future__ import annotations

import numpy as np
import torch

import kda_inputs as ki

DEV = torch.device("cuda:0")
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def dev_io(x: np.ndarray, io: str) -> torch.Tensor:
    """Upload fp32-stored values as the io dtype (bf16 values are exact in fp32 storage)."""
    if io == "bf16":
        return torch.from_numpy(ki.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_inf(y, r) -> float:
    y, r = np.asarray(y, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(y - r)) / max(np.max(np.abs(r)), 1e-300))


def floored_rel(y, r) -> float:
    y, r = np.asarray(y, np.float64), np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(y - r) / np.maximum(np.abs(r), max(rms, 1e-300))))


def rms_rel(y, r) -> float:
    y, r = np.asarray(y, np.float64), np.asarray(r, np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(y - r)) / max(rms, 1e-300))


def err(y, r, io: str) -> float:
    """Error of an io-dtype output (o, prologue y) against the fp64 reference."""
    return floored_rel(y, r) if io == "bf16" else rel_inf(y, r)


def err_state(y, r, io: str) -> float:
    """Error of an fp32 state (final state of a bf16 or fp32 run) against the fp64 reference."""
    return rms_rel(y, r) if io == "bf16" else rel_inf(y, r)


def tol(io: str) -> float:
    return TOL_BF16 if io == "bf16" else TOL_F32


def upload(inp: ki.KDAInputs):
    """Device tensors of a KDAInputs batch: (q, k, v, g, beta, S0 or None, cu_seqlens or None)."""
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(DEV)
    S0 = None if inp.S0 is None else dev_f32(inp.S0)
    return (dev_io(inp.q, inp.io), dev_io(inp.k, inp.io), dev_io(inp.v, inp.io), dev_f32(inp.g),
            dev_f32(inp.beta), S0, cu)
