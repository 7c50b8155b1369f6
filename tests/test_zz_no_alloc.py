"""kda_fwd_noalloc (the prefill with the library's fixed device scratch, for callers that cannot
allocate) against kda_fwd with a caller workspace, through the C ABI (GPU).

Two calls in a row share the one scratch array, the second with a smaller input; both must give
what kda_fwd gives, bit for bit (the chunks and their arithmetic are the same whatever the
window size).  Sizes whose smallest window exceeds the scratch are refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, err, err_state, host, tol, upload

pytestmark = pytest.mark.gpu

SCRATCH = 128 * 1024 * 1024


def _lib():
    L = kda.lib()
    f = L.kda_fwd_noalloc
    P, I = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [I, I, I, I, I, I, P, I, P, P, P, P, P, ctypes.c_float, P, P, P, P]
    f.restype = I
    return L


def _p(t):
    return None if t is None else t.data_ptr()


def noalloc(inp, final=True):
    q, k, v, g, beta, S0, cu = upload(inp)
    io = kda.KDA_BF16 if inp.io == "bf16" else kda.KDA_F32
    o = torch.full((inp.B, inp.T, inp.H, inp.dv), float("nan"), dtype=q.dtype, device=DEV)
    S = torch.full((inp.N, inp.H, inp.dk, inp.dv), float("nan"), dtype=torch.float32, device=DEV) if final else None
    rc = _lib().kda_fwd_noalloc(io, inp.B, inp.T, inp.H, inp.dk, inp.dv, _p(cu), inp.N, _p(q), _p(k), _p(v), _p(g),
                                _p(beta), 1.0, _p(S0), _p(S), _p(o), torch.cuda.current_stream().cuda_stream)
    assert rc == kda.KDA_OK, kda.status_string(rc)
    return o, S


def with_workspace(inp):
    q, k, v, g, beta, S0, cu = upload(inp)
    return kda.fwd(q, k, v, g, beta, 1.0, S0, cu)


def test_noalloc_two_calls_match_fwd_bitwise():
    # first call: the prefill batch (4 x 4096 tokens, 16 heads): its records (~455 MB) exceed the
    # scratch, so it runs in windows; second call: a smaller packed batch, fits in one window
    big = ki.prefill_batch(g_shift=-5.0)
    small = ki.make_varlen([1, 63, 65, 0, 130, 7, 300], 3, 128, 128, "bf16", 6601, s0_std=0.1)
    need = kda.fwd_workspace_bytes(kda.KDA_BF16, 4, 4096, 16, 128, 128, 4, False)
    assert need > SCRATCH
    o1, S1 = noalloc(big)
    o2, S2 = noalloc(small)
    torch.cuda.synchronize()
    r1, R1 = with_workspace(big)
    r2, R2 = with_workspace(small)
    torch.cuda.synchronize()
    assert torch.equal(o1, r1) and torch.equal(S1, R1)
    assert torch.equal(o2, r2) and torch.equal(S2, R2)
    # and against the oracle (the smaller batch, every chain)
    o_ref, S_ref = oracle.recurrence(small.q, small.k, small.v, small.g, small.beta, 1.0, small.S0, small.cu_seqlens)
    e_o, e_s = err(host(o2), o_ref, "bf16"), err_state(host(S2), S_ref, "bf16")
    print(f"noalloc packed batch: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o <= tol("bf16") and e_s <= tol("bf16")


def test_noalloc_without_final_state_carries_states_in_scratch():
    inp = ki.make_dense(2, 5000, 8, 128, 128, "bf16", 6602, s0_std=0.02, g_shift=-5.0)
    o1, _ = noalloc(inp, final=False)
    r1, _ = with_workspace(inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, r1)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # 4096 sequences x 32 heads: one chunk index alone needs ~14 GB of records
    L = _lib()
    FAKE = 1 << 20
    rc = L.kda_fwd_noalloc(kda.KDA_BF16, 4096, 128, 32, 128, 128, None, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0,
                           None, FAKE, FAKE, None)
    assert rc == kda.KDA_ERR_TOO_LARGE, kda.status_string(rc)
    # invalid arguments are still reported as such
    rc = L.kda_fwd_noalloc(kda.KDA_BF16, 1, 64, 1, 96, 96, None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0,
                           None, None, FAKE, None)
    assert rc == kda.KDA_ERR_UNSUPPORTED
