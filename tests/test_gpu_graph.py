"""The library's calls under HIP graph capture (GPU, C ABI).

A packed prefill (chunk-local kernel + state scan), the hand-over of its final states and a run of
decode steps are captured once into a torch.cuda.CUDAGraph (a hipGraph on ROCm) and replayed.  The
library allocates nothing, clears no memory and never synchronises, so the calls can be captured as
they are; every replay, with other eager work and synchronisations between the replays, must equal
the eager run bit for bit.  The replayed outputs are also checked against the fp64 oracle run over
each sequence followed by its decode tokens.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, err_state, host, tol, upload

pytestmark = pytest.mark.gpu

NSTEP = 6


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_prefill_and_decode_steps_replayed_from_a_graph():
    lengths = [300, 1, 129, 64, 77]
    H, d = 4, 128
    N = len(lengths)
    inp = ki.make_varlen(lengths, H, d, d, "bf16", 9300, s0_std=0.02)
    q, k, v, g, beta, S0, cu = upload(inp)
    steps = [ki.decode_step_inputs(N, H, d, "bf16", 9301, s) for s in range(NSTEP)]
    dsteps = [(dev_io(a, "bf16"), dev_io(b, "bf16"), dev_io(c, "bf16"), dev_f32(e), dev_f32(f))
              for (a, b, c, e, f) in steps]
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, 1, inp.T, H, d, d, N, True)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(v)
    S = torch.empty((N, H, d, d), dtype=torch.float32, device=DEV)
    st = torch.empty_like(S)
    od = [torch.empty((N, H, d), dtype=torch.bfloat16, device=DEV) for _ in range(NSTEP)]
    outs = (o, S, st, *od)

    def work():
        kda.fwd(q, k, v, g, beta, 1.0, S0, cu, o=o, final_state=S, workspace=ws)
        st.copy_(S)
        for s in range(NSTEP):
            kda.decode_step(*dsteps[s], st, o=od[s])

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()  # warm-up and capture off the default stream (torch's recipe)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: the outputs and the workspace are overwritten by other calls
        for t in outs:
            t.fill_(float("nan"))
        kda.fwd(q, k, v, g, beta, 0.5, None, cu, o=o, final_state=S, workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), (rep, i)

    # the replayed outputs against the oracle: each sequence, then its NSTEP decode tokens
    o_h, S_h, st_h = host(o), host(S), host(st)
    od_h = [host(t) for t in od]
    worst = [0.0, 0.0, 0.0, 0.0]
    for n in range(N):
        s0, L = int(inp.cu_seqlens[n]), lengths[n]
        for h in range(H):
            cat = lambda x, xs: np.concatenate([x[0, s0:s0 + L, h]] + [a[n, h][None] for a in xs])
            qs = cat(inp.q, [a for a, *_ in steps])
            ks = cat(inp.k, [b for _, b, *_ in steps])
            vs = cat(inp.v, [c for _, _, c, *_ in steps])
            gs = cat(inp.g, [e for *_, e, _ in steps])
            bs = np.concatenate([inp.beta[0, s0:s0 + L, h]] + [np.array([f[n, h]]) for *_, f in steps])
            o_ref, S_end = oracle.chain(qs, ks, vs, gs, bs, 1.0, inp.S0[n, h])
            _, S_pf = oracle.chain(qs[:L], ks[:L], vs[:L], gs[:L], bs[:L], 1.0, inp.S0[n, h])
            if L:
                worst[0] = max(worst[0], err(o_h[0, s0:s0 + L, h], o_ref[:L], "bf16"))
            worst[1] = max(worst[1], err_state(S_h[n, h], S_pf, "bf16"))
            worst[2] = max(worst[2], err(np.stack([x[n, h] for x in od_h]), o_ref[L:], "bf16"))
            worst[3] = max(worst[3], err_state(st_h[n, h], S_end, "bf16"))
    print(f"graph replay vs oracle: prefill o {worst[0]:.2e}, state {worst[1]:.2e}; "
          f"decode o {worst[2]:.2e}, state {worst[3]:.2e}")
    assert max(worst) <= tol("bf16"), worst
