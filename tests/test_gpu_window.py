"""The prefill in windows (a workspace smaller than one record per chunk): the same results as
the one-pass prefill, bit for bit, for dense and packed batches and every gate form, with the
running state carried in final_state or in the workspace (GPU, through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, err_state, host, tol, upload

pytestmark = pytest.mark.gpu


def _align256(x):
    return (x + 255) // 256 * 256


def window_workspace_bytes(io, B, T, H, d, N, varlen, Wc, have_final_state):
    """Workspace for windows of Wc chunk indices: one window's records (+ the carried states)."""
    rec = kda.fwd_workspace_bytes(io, 1, 64, 1, d, d, 1, False)  # one (chunk, head) record
    nrec = (Wc + N) if varlen else N * Wc
    carry = 0 if have_final_state else _align256(N * H * d * d * 4)
    return _align256(nrec * H * rec) + carry


def one_pass(inp):
    """The two phases called on their own: every chunk's record, then the whole scan."""
    q, k, v, g, beta, S0, cu = upload(inp)
    io = kda.KDA_BF16 if inp.io == "bf16" else kda.KDA_F32
    ws = kda.fwd_chunk_local(q, k, v, g, beta, cu)
    o, S = kda.fwd_state_scan(ws, io, inp.B, inp.T, inp.H, inp.dk, cu, 1.0, S0)
    torch.cuda.synchronize()
    return o, S


def run(inp, ws_bytes=None, final=True, gate="channel", lowrank=None):
    q, k, v, g, beta, S0, cu = upload(inp)
    ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    if gate == "channel":
        o, S = kda.fwd(q, k, v, g, beta, 1.0, S0, cu, output_final_state=final, workspace=ws)
    elif gate == "scalar":
        o, S = kda.fwd_scalar_gate(q, k, v, g[..., 0].contiguous(), beta, 1.0, S0, cu, output_final_state=final,
                                   workspace=ws)
    else:
        z, w_up, b = lowrank
        o, S = kda.fwd_lowrank_gate(q, k, v, z, w_up, b, beta, 1.0, S0, cu, output_final_state=final, workspace=ws)
    torch.cuda.synchronize()
    return o, S


def _cases():
    dense = ki.make_dense(2, 1000, 3, 128, 128, "bf16", 5501, s0_std=0.1, g_shift=-5.0)
    packed = ki.make_varlen([1, 63, 65, 0, 130, 7, 300, 1000], 2, 128, 128, "bf16", 5502, s0_std=0.1, g_shift=-5.0)
    return {"dense": dense, "packed": packed}


@pytest.mark.parametrize("layout", ["dense", "packed"])
@pytest.mark.parametrize("Wc", [1, 3, 7])
@pytest.mark.parametrize("final", [True, False])
def test_windows_equal_one_pass_bitwise(layout, Wc, final):
    inp = _cases()[layout]
    io = kda.KDA_BF16
    varlen = inp.cu_seqlens is not None
    o1, S1 = one_pass(inp)
    nb = window_workspace_bytes(io, inp.B, inp.T, inp.H, inp.dk, inp.N, varlen, Wc, final)
    assert nb < kda.fwd_workspace_bytes(io, inp.B, inp.T, inp.H, inp.dk, inp.dk, inp.N, varlen)
    o2, S2 = run(inp, nb, final)
    assert torch.equal(o1, o2), (layout, Wc, final)
    if final:
        assert torch.equal(S1, S2), (layout, Wc, final)


@pytest.mark.parametrize("gate", ["scalar", "lowrank"])
def test_windows_other_gate_forms_bitwise(gate):
    inp = _cases()["packed"]
    lowrank = None
    if gate == "lowrank":
        r = 32
        rng = np.random.default_rng(5503)
        z = dev_io(rng.standard_normal((1, inp.T, r)).astype(np.float32), "bf16")
        _, _, w_up, _ = ki.gate_weights(256, inp.H, inp.dk, r, 5503)
        b = dev_f32(np.full(inp.H * inp.dk, -5.0, np.float32))
        lowrank = (z, dev_io(w_up, "bf16"), b)
    o1, S1 = run(inp, gate=gate, lowrank=lowrank)
    nb = window_workspace_bytes(kda.KDA_BF16, inp.B, inp.T, inp.H, inp.dk, inp.N, True, 2, True)
    o2, S2 = run(inp, nb, gate=gate, lowrank=lowrank)
    assert torch.equal(o1, o2) and torch.equal(S1, S2), gate


def test_minimum_workspace_against_oracle():
    """The smallest workspace the library accepts (one chunk per window, states carried in the
    workspace): every chain against the fp64 oracle; one byte less is refused."""
    inp = _cases()["packed"]
    io = kda.KDA_BF16
    nmin = kda.fwd_workspace_min_bytes(io, 1, inp.T, inp.H, inp.dk, inp.dk, inp.N, True, False)
    assert nmin == window_workspace_bytes(io, 1, inp.T, inp.H, inp.dk, inp.N, True, 1, False)
    with pytest.raises(kda.KDAError):
        run(inp, nmin - 1, final=False)
    o, _ = run(inp, nmin, final=False)
    o_ref, _ = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, 1.0, inp.S0, inp.cu_seqlens)
    e = err(host(o), o_ref, "bf16")
    print(f"minimum workspace ({nmin} bytes): o err {e:.3e}")
    assert e <= tol("bf16")


def test_prefill_batch_in_windows_bitwise():
    """The prefill batch (B=4, H=16, T=4096, d=128): kda_fwd with the full workspace and in windows of
    16 chunks both equal the two phases called on their own."""
    inp = ki.prefill_batch()
    o1, S1 = one_pass(inp)
    o2, S2 = run(inp)
    nb = window_workspace_bytes(kda.KDA_BF16, 4, 4096, 16, 128, 4, False, 16, True)
    o3, S3 = run(inp, nb)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, S3)
