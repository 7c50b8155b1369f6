"""kda_decode_step against the fp64 oracle (GPU, through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, err_state, host, tol

pytestmark = pytest.mark.gpu


def test_decode_pool_256x32_sampled_chains():
    """256 sequences x 32 heads, d = 128, bf16 tokens, fp32 state in HBM, 100 steps.
    All heads run on the GPU; 48 sampled (sequence, head) chains are checked step by step."""
    c = ki.DECODE_POOL
    N, H, d, steps, seed = c["N"], c["H"], c["d"], c["steps"], c["seed"]
    S0 = ki.decode_initial_state(N, H, d, seed)
    state = dev_f32(S0)
    rng = np.random.default_rng(1)
    picks = [(int(n), int(h)) for n, h in zip(rng.integers(0, N, 48), rng.integers(0, H, 48))]
    hist = {nh: {"q": [], "k": [], "v": [], "g": [], "b": [], "o": []} for nh in picks}
    for s in range(steps):
        q, k, v, g, beta = ki.decode_step_inputs(N, H, d, "bf16", seed, s)
        o = kda.decode_step(dev_io(q, "bf16"), dev_io(k, "bf16"), dev_io(v, "bf16"), dev_f32(g), dev_f32(beta),
                            state)
        oh = host(o)
        for (n, h) in picks:
            rec = hist[(n, h)]
            rec["q"].append(q[n, h]); rec["k"].append(k[n, h]); rec["v"].append(v[n, h])
            rec["g"].append(g[n, h]); rec["b"].append(beta[n, h]); rec["o"].append(oh[n, h])
    S_gpu = host(state)
    worst_o = worst_s = 0.0
    for (n, h), rec in hist.items():
        o_ref, S_ref = oracle.chain(np.stack(rec["q"]), np.stack(rec["k"]), np.stack(rec["v"]),
                                    np.stack(rec["g"]), np.array(rec["b"]), 1.0, S0[n, h])
        worst_o = max(worst_o, err(np.stack(rec["o"]), o_ref, "bf16"))
        worst_s = max(worst_s, err_state(S_gpu[n, h], S_ref, "bf16"))
    print(f"decode 256 x 32 heads: o err {worst_o:.3e}, state err {worst_s:.3e}")
    assert worst_o <= tol("bf16") and worst_s <= tol("bf16")


def test_decode_fp32_equals_recurrence_small():
    """The small fp32 workload (B = 1, H = 2, T = 256, d = 64) run as 256 consecutive decode steps."""
    inp = ki.small_fp32()
    o_ref, S_ref = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta)
    state = torch.zeros((1, inp.H, 64, 64), dtype=torch.float32, device=DEV)
    outs = []
    for t in range(inp.T):
        o = kda.decode_step(dev_io(inp.q[:, t], "f32"), dev_io(inp.k[:, t], "f32"), dev_io(inp.v[:, t], "f32"),
                            dev_f32(inp.g[:, t]), dev_f32(inp.beta[:, t]), state)
        outs.append(host(o))
    o_gpu = np.stack(outs, axis=1)
    e_o, e_s = err(o_gpu, o_ref, "f32"), err_state(host(state), S_ref, "f32")
    print(f"decode fp32 B1 H2 T256 d64: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o <= tol("f32") and e_s <= tol("f32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64), (128, 128)])
def test_decode_shapes(io, dk, dv):
    """Every supported (d_k, d_v) pair in both io types: six steps from a random state, scale 0.5."""
    N, H, steps = 3, 2, 6
    rng = np.random.default_rng(dk + dv)
    S0 = (rng.standard_normal((N, H, dk, dv)) * 0.1).astype(np.float32)
    state = dev_f32(S0)
    toks = [ki.draw_tokens(np.random.default_rng([7, s]), (N,), H, dk, dv, io) for s in range(steps)]
    outs = []
    for (q, k, v, beta, g) in toks:
        outs.append(host(kda.decode_step(dev_io(q, io), dev_io(k, io), dev_io(v, io), dev_f32(g), dev_f32(beta),
                                         state, scale=0.5)))
    S_gpu = host(state)
    worst = 0.0
    for n in range(N):
        for h in range(H):
            st = lambda i: np.stack([t[i][n, h] for t in toks])
            o_ref, S_ref = oracle.chain(st(0), st(1), st(2), st(4), np.array([t[3][n, h] for t in toks]), 0.5,
                                        S0[n, h])
            e = max(err(np.stack([o[n, h] for o in outs]), o_ref, io), err_state(S_gpu[n, h], S_ref, io))
            worst = max(worst, e)
    print(f"decode {io} d_k={dk} d_v={dv}: err {worst:.3e}")
    assert worst <= tol(io)


def test_decode_recall_on_gpu():
    """Unit key and beta = 1: after the step the state maps k to v (S^T k = v), read with q = k."""
    N, H, d = 4, 3, 128
    rng = np.random.default_rng(5)
    k = rng.standard_normal((N, H, d))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((N, H, d)).astype(np.float32)
    g = (-rng.uniform(0, 3, (N, H, d))).astype(np.float32)
    state = dev_f32(rng.standard_normal((N, H, d, d)).astype(np.float32))
    o = kda.decode_step(dev_f32(k), dev_f32(k), dev_f32(v), dev_f32(g), dev_f32(np.ones((N, H), np.float32)), state)
    res = np.max(np.abs(host(o) - v)) / np.max(np.abs(v))
    print(f"recall residual {res:.2e}")
    assert res <= 1e-5
