"""Guard bands: every entry point writes only inside the output buffers it is given.

Each output (and the prefill workspace) is carved out of a larger device allocation whose bytes
before and after it hold a sentinel pattern.  After the call the guard bytes must be unchanged.
The inputs are ragged (packed sequences with partial chunks, empty and one-token sequences,
token counts that do not fill the last workgroup), where an index past the end would land in
the guard band.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
from gpu_util import DEV, dev_f32, dev_io, upload

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of sentinel on each side (a multiple of 256: the views stay aligned)
SENTINEL = 0xA5


class Guarded:
    """A device tensor of `shape`/`dtype` with GUARD sentinel bytes on each side."""

    def __init__(self, shape, dtype, fill=None):
        itemsize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * itemsize
        self.raw = torch.full((GUARD + self.nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def intact(self) -> bool:
        torch.cuda.synchronize()
        lo, hi = self.raw[:GUARD], self.raw[GUARD + self.nbytes:]
        return bool((lo == SENTINEL).all().item()) and bool((hi == SENTINEL).all().item())


def _ragged():
    return ki.make_varlen([1, 63, 65, 0, 130, 7, 191], 3, 128, 128, "bf16", 4401, s0_std=0.1)


@pytest.mark.parametrize("gate", ["channel", "scalar"])
def test_fwd_outputs_and_workspace_stay_in_bounds(gate):
    inp = _ragged()
    q, k, v, g, beta, S0, cu = upload(inp)
    N, H, d = inp.N, inp.H, inp.dk
    o = Guarded((1, inp.T, H, d), torch.bfloat16)
    S = Guarded((N, H, d, d), torch.float32)
    need = kda.fwd_workspace_bytes(kda.KDA_BF16, 1, inp.T, H, d, d, N, True)
    ws = Guarded((need,), torch.uint8)
    if gate == "channel":
        kda.fwd(q, k, v, g, beta, 1.0, S0, cu, o=o.t, final_state=S.t, workspace=ws.t)
    else:
        kda.fwd_scalar_gate(q, k, v, g[..., 0].contiguous(), beta, 1.0, S0, cu, o=o.t, final_state=S.t,
                            workspace=ws.t)
    assert o.intact() and S.intact() and ws.intact()


def test_fwd_dense_ragged_tail_in_bounds():
    inp = ki.make_dense(3, 201, 2, 64, 64, "f32", 4402, s0_std=0.1)
    q, k, v, g, beta, S0, _ = upload(inp)
    o = Guarded((3, 201, 2, 64), torch.float32)
    S = Guarded((3, 2, 64, 64), torch.float32)
    need = kda.fwd_workspace_bytes(kda.KDA_F32, 3, 201, 2, 64, 64, 3, False)
    ws = Guarded((need,), torch.uint8)
    kda.fwd(q, k, v, g, beta, 1.0, S0, o=o.t, final_state=S.t, workspace=ws.t)
    assert o.intact() and S.intact() and ws.intact()


def test_segment_maps_and_hop_in_bounds():
    inp = _ragged()
    q, k, v, g, beta, _, cu = upload(inp)
    N, H, d = inp.N, inp.H, inp.dk
    need = kda.fwd_workspace_bytes(kda.KDA_BF16, 1, inp.T, H, d, d, N, True)
    ws = Guarded((need,), torch.uint8)
    kda.fwd_chunk_local(q, k, v, g, beta, cu, workspace=ws.t)
    A = Guarded((N, H, d, d), torch.float32)
    B = Guarded((N, H, d, d), torch.float32)
    kda.fwd_segment_map(ws.t, kda.KDA_BF16, 1, inp.T, H, d, cu, transition=A.t, offset=B.t)
    out = Guarded((N * H, d, d), torch.float32)
    kda.state_combine(A.t.view(N * H, d, d), B.t.view(N * H, d, d), B.t.view(N * H, d, d), out=out.t)
    assert ws.intact() and A.intact() and B.intact() and out.intact()


@pytest.mark.parametrize("io,d", [("bf16", 128), ("f32", 64)])
def test_prep_output_in_bounds(io, d):
    x, w, cu = ki.prep_inputs([5, 0, 70, 1, 133], 3, d, io, 4403)
    xd = dev_io(x, io)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    y = Guarded(tuple(x.shape), dt)
    kda.prep(xd, dev_f32(w), torch.from_numpy(cu).to(DEV), y=y.t)
    assert y.intact()


def test_decode_state_and_output_in_bounds():
    N, H, d = 5, 3, 128
    q, k, v, g, beta = ki.decode_step_inputs(N, H, d, "bf16", 4404, 0)
    st = Guarded((N, H, d, d), torch.float32, fill=dev_f32(ki.decode_initial_state(N, H, d, 4404)))
    o = Guarded((N, H, d), torch.bfloat16)
    kda.decode_step(dev_io(q, "bf16"), dev_io(k, "bf16"), dev_io(v, "bf16"), dev_f32(g), dev_f32(beta), st.t, o=o.t)
    assert st.intact() and o.intact()


def test_gate_outputs_in_bounds():
    Ntok, Dm, H, d, r = 77, 256, 3, 128, 32
    x = dev_io(ki.gate_hidden(Ntok, Dm, 4405), "bf16")
    w_down, w_beta, w_up, b = ki.gate_weights(Dm, H, d, r, 4405)
    z = Guarded((Ntok, r), torch.bfloat16)
    bt = Guarded((Ntok, H), torch.float32)
    gg = Guarded((Ntok, H, d), torch.float32)
    kda.gate(x, dev_io(w_down, "bf16"), dev_io(w_beta, "bf16"), dev_io(w_up, "bf16"), dev_f32(b), H=H,
             want_g=True, z=z.t, beta=bt.t, g=gg.t)
    assert z.intact() and bt.intact() and gg.intact()


def test_attnres_outputs_in_bounds():
    n, T, d, L = 3, 37, 512, 5
    rng = np.random.default_rng(4406)
    blocks = [dev_io(rng.standard_normal((T, d)).astype(np.float32), "bf16") for _ in range(n)]
    W = dev_io((rng.standard_normal((L, d)) / np.sqrt(d)).astype(np.float32), "bf16")
    h = Guarded((T, d), torch.bfloat16)
    kda.attnres(blocks, W[0].contiguous(), 1e-6, h=h.t)
    o = Guarded((L, T, d), torch.bfloat16)
    lse = Guarded((L, T), torch.float32)
    nws = int(kda.lib().kda_attnres_inter_workspace_bytes(n - 1, L, T))
    ws = Guarded((nws,), torch.uint8)
    kda.attnres_inter(blocks[:-1], W, 1e-6, o=o.t, lse=lse.t, workspace=ws.t)
    h2 = Guarded((T, d), torch.bfloat16)
    kda.attnres_merge(blocks[-1], W[1].contiguous(), o.t[1].contiguous(), lse.t[1].contiguous(), 1e-6, h=h2.t)
    assert h.intact() and o.intact() and lse.intact() and ws.intact() and h2.intact()
