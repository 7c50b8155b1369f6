"""Parity of the low-rank gate on the GPU with the fp64 oracle.

kda_gate (the prologue: z = x W_down^T stored bf16, beta = sigmoid(x w_beta^T), optional
g = -softplus(z W_up^T + b)) and kda_fwd_lowrank_gate (the operator with g formed inside the
chunk-local kernel).  The oracle's gate is pinned on the CPU (tests/test_oracle_gate.py), its
recurrence by tests/test_oracle_pins.py.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, err_state, floored_rel, host, rel_inf, tol

pytestmark = pytest.mark.gpu


def upload_gate(x, w_down, w_beta, w_up, b):
    return (dev_io(x, "bf16"), dev_io(w_down, "bf16"), dev_io(w_beta, "bf16"), dev_io(w_up, "bf16"), dev_f32(b))


@pytest.mark.parametrize("Ntok,Dm,H,d,r", [(1000, 512, 4, 128, 32), (333, 256, 3, 64, 64), (64, 128, 17, 64, 128),
                                           (7, 64, 2, 128, 96)])
def test_gate_prologue_vs_oracle(Ntok, Dm, H, d, r):
    seed = 93200 + r + H
    w_down, w_beta, w_up, b = ki.gate_weights(Dm, H, d, r, seed)
    x = ki.gate_hidden(Ntok, Dm, seed)
    z_g, beta_g, g_g = kda.gate(*upload_gate(x, w_down, w_beta, w_up, b), want_g=True)
    torch.cuda.synchronize()
    z_g, beta_g, g_g = host(z_g), host(beta_g), host(g_g)
    z_ref, beta_ref, _ = oracle.gate(x, w_down, w_beta, w_up, b, H, d)
    # z is stored in bf16: within one rounding of the fp64 value (plus fp32 summation)
    e_z = floored_rel(z_g, z_ref)
    e_b = rel_inf(beta_g, beta_ref)
    # g from the stored z: the oracle's own z rounded to bf16.  Tokens whose z rounds the same
    # way on both sides (all but rare ties) must agree to fp32 accuracy; the rest within the
    # effect of one bf16 step of z.
    z_st = ki.bf16_round(z_ref.astype(np.float32)).astype(np.float64)
    g_ref = oracle.gate_g(z_st, w_up, b, H, d)
    same = np.all(z_g == z_st, axis=1)
    e_g = rel_inf(g_g[same], g_ref[same]) if same.any() else 0.0
    e_g_rest = floored_rel(g_g[~same], g_ref[~same]) if (~same).any() else 0.0
    print(f"gate Ntok={Ntok} Dm={Dm} H={H} d={d} r={r}: z err {e_z:.2e}, beta err {e_b:.2e}, "
          f"g err {e_g:.2e} ({same.mean():.4f} of tokens with identical z), other g err {e_g_rest:.2e}")
    assert e_z <= 4e-3
    assert e_b <= 1e-5
    assert same.mean() >= 0.98
    assert e_g <= 1e-5 and e_g_rest <= 5e-3


def test_gate_without_g_writes_z_and_beta_only():
    w_down, w_beta, w_up, b = ki.gate_weights(256, 4, 128, 32, 93210)
    x = ki.gate_hidden(200, 256, 93210)
    X = upload_gate(x, w_down, w_beta, w_up, b)
    z1, b1, g1 = kda.gate(*X, want_g=True)
    z2, b2, g2 = kda.gate(X[0], X[1], X[2], H=4)
    torch.cuda.synchronize()
    assert g2 is None and torch.equal(z1, z2) and torch.equal(b1, b2)


def run_lowrank(inp, cu=None):
    q, k, v = (dev_io(a, "bf16") for a in (inp.q, inp.k, inp.v))
    S0 = None if inp.S0 is None else dev_f32(inp.S0)
    cu_t = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(DEV)
    o, S = kda.fwd_lowrank_gate(q, k, v, dev_io(inp.z, "bf16"), dev_io(inp.w_up, "bf16"), dev_f32(inp.b),
                                dev_f32(inp.beta), 1.0, S0, cu_t)
    torch.cuda.synchronize()
    return host(o), host(S)


def check_lowrank(inp, label, chains=None):
    o, S = run_lowrank(inp)
    B, T, H, d = inp.q.shape
    g = oracle.gate_g(inp.z.reshape(B * T, -1), inp.w_up, inp.b, H, d).reshape(B, T, H, d)
    R = oracle.Recurrence(inp.q, inp.k, inp.v, g, inp.beta, 1.0, inp.S0, inp.cu_seqlens)
    worst_o = worst_s = 0.0
    for (n, h), (o_ref, S_ref) in R.run(chains).items():
        bb, s, L = R.bounds(n)
        worst_o = max(worst_o, err(o[bb, s:s + L, h], o_ref, "bf16") if L else 0.0)
        worst_s = max(worst_s, err_state(S[n, h], S_ref, "bf16"))
    print(f"low-rank gate fwd {label}: o err {worst_o:.3e}, state err {worst_s:.3e}")
    assert worst_o <= tol("bf16") and worst_s <= tol("bf16"), (label, worst_o, worst_s)


def test_fwd_lowrank_dense_ragged():
    check_lowrank(ki.make_lowrank(2, 200, 3, 128, 32, 93220), "B=2 T=200 H=3 d=128 r=32")


@pytest.mark.parametrize("d,r", [(64, 64), (128, 128), (64, 96)])
def test_fwd_lowrank_sizes(d, r):
    check_lowrank(ki.make_lowrank(1, 333, 2, d, r, 93221 + r + d), f"d={d} r={r}")


def test_fwd_lowrank_varlen():
    check_lowrank(ki.make_lowrank(1, 0, 2, 128, 32, 93222, lengths=[130, 1, 64, 0, 300, 63]), "varlen")


def test_fwd_lowrank_weak_decay_long():
    check_lowrank(ki.make_lowrank(1, 2048, 2, 128, 32, 93223, b_mean=-5.0), "weak decay T=2048")


def test_fwd_lowrank_prefill_shape_sampled():
    """B=4, H=16, T=4096, d=128, r=32 (the prefill workload's shape with the gate in low-rank
    form); 6 sampled chains."""
    inp = ki.make_lowrank(4, 4096, 16, 128, 32, 93224, s0_std=None)
    check_lowrank(inp, "B=4 T=4096 H=16 sampled", chains=[(0, 0), (1, 7), (2, 15), (3, 3), (3, 9), (0, 12)])


@pytest.mark.parametrize("d", [64, 128])
def test_fused_equals_prologue_then_fwd_bitwise(d):
    """kda_gate(..., g) then kda_fwd(g) and kda_fwd_lowrank_gate(z) compute the same values in the
    same order: outputs and final states are bitwise equal."""
    B, T, H, r, Dm = 2, 450, 3, 32, 256
    seed = 93230 + d
    w_down, w_beta, w_up, b = ki.gate_weights(Dm, H, d, r, seed)
    x = ki.gate_hidden(B * T, Dm, seed)
    inp = ki.make_lowrank(B, T, H, d, r, seed)
    z, beta, g = kda.gate(*upload_gate(x, w_down, w_beta, w_up, b), want_g=True)
    q, k, v = (dev_io(a, "bf16") for a in (inp.q, inp.k, inp.v))
    S0 = dev_f32(inp.S0)
    o1, S1 = kda.fwd(q, k, v, g.view(B, T, H, d), beta.view(B, T, H), 1.0, S0)
    o2, S2 = kda.fwd_lowrank_gate(q, k, v, z.view(B, T, r), dev_io(w_up, "bf16"), dev_f32(b), beta.view(B, T, H),
                                  1.0, S0)
    torch.cuda.synchronize()
    print(f"fused vs prologue+fwd d={d}: o equal {torch.equal(o1, o2)}, state equal {torch.equal(S1, S2)}")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_gate_largest_rank_and_heads():
    """r = 128 (four rank blocks), H = 64 heads (four beta tiles), d = 64."""
    Ntok, Dm, H, d, r = 200, 256, 64, 64, 128
    w_down, w_beta, w_up, b = ki.gate_weights(Dm, H, d, r, 93250)
    x = ki.gate_hidden(Ntok, Dm, 93250)
    z_g, beta_g, g_g = kda.gate(*upload_gate(x, w_down, w_beta, w_up, b), want_g=True)
    torch.cuda.synchronize()
    z_ref, beta_ref, _ = oracle.gate(x, w_down, w_beta, w_up, b, H, d)
    z_st = ki.bf16_round(z_ref.astype(np.float32)).astype(np.float64)
    same = np.all(host(z_g) == z_st, axis=1)
    e_g = rel_inf(host(g_g)[same], oracle.gate_g(z_st, w_up, b, H, d)[same])
    print(f"gate r=128 H=64: z err {floored_rel(host(z_g), z_ref):.2e}, beta err {rel_inf(host(beta_g), beta_ref):.2e}, "
          f"g err {e_g:.2e} ({same.mean():.3f} identical z)")
    assert floored_rel(host(z_g), z_ref) <= 4e-3 and rel_inf(host(beta_g), beta_ref) <= 1e-5
    assert same.mean() >= 0.95 and e_g <= 1e-5


def test_gate_prologue_prefill_width():
    """The gate prologue at the width the benchmark uses (2048: the whole-line load path), 16 heads of
    128 channels, rank 32, with a ragged last workgroup (16,421 tokens); every token checked."""
    Ntok, Dm, H, d, r = 16384 + 37, 2048, 16, 128, 32
    w_down, w_beta, w_up, b = ki.gate_weights(Dm, H, d, r, 93260)
    x = ki.gate_hidden(Ntok, Dm, 93260)
    z_g, beta_g, g_g = kda.gate(*upload_gate(x, w_down, w_beta, w_up, b), want_g=True)
    torch.cuda.synchronize()
    z_g, beta_g, g_g = host(z_g), host(beta_g), host(g_g)
    z_ref, beta_ref, _ = oracle.gate(x, w_down, w_beta, w_up, b, H, d)
    z_st = ki.bf16_round(z_ref.astype(np.float32)).astype(np.float64)
    same = np.all(z_g == z_st, axis=1)
    g_ref = oracle.gate_g(z_st, w_up, b, H, d)
    e_z, e_b = floored_rel(z_g, z_ref), rel_inf(beta_g, beta_ref)
    e_g = rel_inf(g_g[same], g_ref[same])
    e_g_rest = floored_rel(g_g[~same], g_ref[~same]) if (~same).any() else 0.0
    print(f"gate Ntok={Ntok} Dm={Dm}: z err {e_z:.2e}, beta err {e_b:.2e}, g err {e_g:.2e} "
          f"({same.mean():.4f} identical z), other g err {e_g_rest:.2e}")
    assert e_z <= 4e-3 and e_b <= 1e-5
    assert same.mean() >= 0.95 and e_g <= 1e-5 and e_g_rest <= 5e-3
