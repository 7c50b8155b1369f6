"""Seeded random shapes of the prefill against the fp64 oracle (GPU, through the C ABI).

Each case draws, from its own seed: dense or packed batch (with empty and one-token sequences),
bf16 or fp32, d_k = d_v = 64 or 128, 1-5 heads, lengths up to a few hundred tokens, with or
without an initial state, with or without a final state, the workload's, a weak or no decay,
one decay per channel or per head, and either the whole workspace or a random one between the
smallest accepted and the whole (the prefill then runs in windows).  Every chain is compared
with the oracle by the output and state measures.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, err, err_state, host, tol, upload

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    rng = np.random.default_rng(9300 + i)
    io = "bf16" if rng.random() < 0.7 else "f32"
    d = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 6))
    s0 = 0.1 if rng.random() < 0.6 else None
    final = bool(rng.random() < 0.8)
    g_shift = float(rng.choice([2.0, -5.0]))
    per_head = bool(rng.random() < 0.25)
    no_decay = bool(rng.random() < 0.1)
    if rng.random() < 0.5:
        lengths = [int(x) for x in rng.integers(0, 400, int(rng.integers(1, 7)))]
        lengths[int(rng.integers(0, len(lengths)))] = int(rng.choice([1, 64, 65, 128]))
        inp = ki.make_varlen(lengths, H, d, d, io, 9400 + i, s0_std=s0, g_shift=g_shift)
        shape = f"packed {lengths}"
    else:
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 500))
        inp = ki.make_dense(B, T, H, d, d, io, 9400 + i, s0_std=s0, g_shift=g_shift)
        shape = f"dense B={B} T={T}"
    if no_decay:
        inp.g[:] = 0.0
    if per_head:  # one log-decay per token and head: channel 0's, on every channel
        inp.g[:] = inp.g[..., :1]
    frac = None if rng.random() < 0.6 else float(rng.random())
    label = (f"case {i}: {shape} H={H} d={d} {io} S0={'yes' if s0 else 'no'} final={final} "
             f"g_shift={g_shift}{' per-head' if per_head else ''}{' alpha=1' if no_decay else ''} "
             f"workspace={'full' if frac is None else f'{frac:.2f} of the way from the smallest'}")
    return inp, final, per_head, frac, label


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_against_oracle(i):
    inp, final, per_head, frac, label = _case(i)
    print(label, flush=True)
    q, k, v, g, beta, S0, cu = upload(inp)
    io = kda.KDA_BF16 if inp.io == "bf16" else kda.KDA_F32
    varlen = cu is not None
    B = 1 if varlen else inp.B
    full = kda.fwd_workspace_bytes(io, B, inp.T, inp.H, inp.dk, inp.dk, inp.N, varlen)
    least = kda.fwd_workspace_min_bytes(io, B, inp.T, inp.H, inp.dk, inp.dk, inp.N, varlen, final)
    nws = full if frac is None else least + int(frac * (full - least)) // 256 * 256
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=DEV)
    if per_head:
        o, S = kda.fwd_scalar_gate(q, k, v, g[..., 0].contiguous(), beta, 1.0, S0, cu, output_final_state=final,
                                   workspace=ws[:nws])
    else:
        o, S = kda.fwd(q, k, v, g, beta, 1.0, S0, cu, output_final_state=final, workspace=ws[:nws])
    torch.cuda.synchronize()
    R = oracle.Recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, 1.0, inp.S0, inp.cu_seqlens)
    worst_o = worst_s = 0.0
    for (n, h), (o_ref, S_ref) in R.run(None).items():
        b, s, L = R.bounds(n)
        if L:
            worst_o = max(worst_o, err(host(o[b, s:s + L, h]), o_ref, inp.io))
        if final:
            worst_s = max(worst_s, err_state(host(S[n, h]), S_ref, inp.io))
    print(f"  o err {worst_o:.3e}, state err {worst_s:.3e}")
    assert worst_o <= tol(inp.io), (label, worst_o)
    assert worst_s <= tol(inp.io), (label, worst_s)
