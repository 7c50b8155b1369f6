"""Parity of the segment-map path (one sequence split into segments, as context parallelism
splits it over devices, here run on one GPU) with the fp64 oracle, through the C ABI.

  * kda_fwd_segment_map: (A, B) of every segment and head against oracle.segment_map, which
    writes A out as the product of the per-token maps and takes B from the recurrence.
  * kda_state_combine: A S + B against the fp64 product.
  * the whole chain (chunk records and maps of all segments, P - 1 hops, the scan from the
    incoming states): o and the final state against the oracle run over the unsplit sequence.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, err_state, host, rel_inf, tol

pytestmark = pytest.mark.gpu


def _bounds(lengths):
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def _maps(inp, cu):
    io = kda.KDA_BF16 if inp.io == "bf16" else kda.KDA_F32
    q, k, v = (dev_io(x, inp.io) for x in (inp.q, inp.k, inp.v))
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    ws = kda.fwd_chunk_local(q, k, v, dev_f32(inp.g), dev_f32(inp.beta), cu_d)
    A, B = kda.fwd_segment_map(ws, io, 1, inp.T, inp.H, inp.dk, cu_d)
    torch.cuda.synchronize()
    return host(A), host(B)


def err_A(y, r, io):
    """The error measure of the io dtype, with the denominator floored at 1e-6 as well: A is a
    product of maps of norm <= 1 (|k| = 1, 0 <= beta <= 1, alpha <= 1), so an absolute error
    below 2e-8 changes A S_in by less than 2e-8 |S_in|, and a strongly decaying segment drives A
    below the fp32 range, where the fp64 reference keeps values like 1e-100."""
    y, r = np.asarray(y, np.float64), np.asarray(r, np.float64)
    if io != "bf16":
        return float(np.max(np.abs(y - r)) / max(np.max(np.abs(r)), 1e-6))
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(y - r) / np.maximum(np.abs(r), max(rms, 1e-6))))


def check_maps(inp, cu, label, heads=None):
    A, B = _maps(inp, cu)
    worst_a = worst_b = lit_a = 0.0
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in (range(inp.H) if heads is None else heads):
            A_ref, B_ref = oracle.segment_map(inp.k[0, s:e, h], inp.v[0, s:e, h], inp.g[0, s:e, h],
                                              inp.beta[0, s:e, h])
            worst_a = max(worst_a, err_A(A[n, h], A_ref, inp.io))
            lit_a = max(lit_a, err_state(A[n, h], A_ref, inp.io)) if e > s else lit_a
            worst_b = max(worst_b, err_state(B[n, h], B_ref, inp.io) if e > s else float(np.max(np.abs(B[n, h]))))
    print(f"segment map {label}: A err {worst_a:.3e} (max|dA|/rms(A) {lit_a:.3e}), B err {worst_b:.3e}")
    assert worst_a <= tol(inp.io) and worst_b <= tol(inp.io), (label, worst_a, worst_b)


def test_segment_map_bf16_ragged_segments():
    """Segments of 320, 1, 130, 0 and 257 tokens (whole chunks, a single token, ragged tails, an
    empty one) with weak decay, so A stays far from zero over the segment."""
    lengths = [320, 1, 130, 0, 257]
    inp = ki.make_varlen(lengths, 2, 128, 128, "bf16", 93200, s0_std=None, g_shift=-5.0)
    check_maps(inp, _bounds(lengths), "bf16 d=128")


def test_segment_map_empty_segment_is_identity():
    lengths = [0, 64, 0]
    inp = ki.make_varlen(lengths, 1, 128, 128, "bf16", 93201, s0_std=None, g_shift=-5.0)
    A, B = _maps(inp, _bounds(lengths))
    for n in (0, 2):
        assert np.array_equal(A[n, 0], np.eye(128)) and not np.any(B[n, 0])


@pytest.mark.parametrize("d", [64, 128])
def test_segment_map_fp32(d):
    lengths = [200, 77]
    inp = ki.make_varlen(lengths, 2, d, d, "f32", 93202 + d, s0_std=None, g_shift=-5.0)
    check_maps(inp, _bounds(lengths), f"fp32 d={d}")


def test_segment_map_bf16_d64_strong_decay():
    lengths = [150, 64]
    inp = ki.make_varlen(lengths, 3, 64, 64, "bf16", 93203, s0_std=None)
    check_maps(inp, _bounds(lengths), "bf16 d=64 strong decay")


def test_segment_map_many_heads_uses_two_tile_workgroups():
    """16 segments x 16 heads: enough column tiles that the scan takes its two-tile form."""
    lengths = [128] * 16
    inp = ki.make_varlen(lengths, 16, 128, 128, "bf16", 93204, s0_std=None, g_shift=-5.0)
    check_maps(inp, _bounds(lengths), "16 x 16 two-tile", heads=[0, 7, 15])


@pytest.mark.parametrize("d", [64, 128])
def test_state_combine_parity(d):
    rng = np.random.default_rng(93210 + d)
    A = rng.standard_normal((3, 5, d, d)).astype(np.float32) / np.sqrt(d)
    S = rng.standard_normal((3, 5, d, d)).astype(np.float32)
    B = rng.standard_normal((3, 5, d, d)).astype(np.float32)
    out = host(kda.state_combine(dev_f32(A), dev_f32(S), dev_f32(B)))
    ref = oracle.state_combine(A, S, B)
    e = rel_inf(out, ref)
    print(f"state combine d={d}: rel err {e:.3e}")
    assert e <= 1e-5
    # the output may be the offset buffer itself
    Bd = dev_f32(B)
    kda.state_combine(dev_f32(A), dev_f32(S), Bd, out=Bd)
    assert np.array_equal(host(Bd), out)


def test_composed_maps_equal_the_map_of_the_concatenation():
    """(A2, B2) after (A1, B1) = (A2 A1, A2 B1 + B2), formed with kda_state_combine (the offset
    left out for A2 A1), against the map of the two segments as one: the step of a prefix over
    segments taken as a tree."""
    lengths = [200, 331]
    inp = ki.make_varlen(lengths, 2, 128, 128, "bf16", 93223, s0_std=None, g_shift=-5.0)
    cu = _bounds(lengths)
    io = kda.KDA_BF16
    q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
    cu_d = torch.from_numpy(cu.astype(np.int32)).to(DEV)
    ws = kda.fwd_chunk_local(q, k, v, dev_f32(inp.g), dev_f32(inp.beta), cu_d)
    A, B = kda.fwd_segment_map(ws, io, 1, inp.T, inp.H, inp.dk, cu_d)
    A12 = kda.state_combine(A[1], A[0])
    B12 = kda.state_combine(A[1], B[0], B[1])
    whole = torch.from_numpy(np.array([0, inp.T], np.int32)).to(DEV)
    ws1 = kda.fwd_chunk_local(q, k, v, dev_f32(inp.g), dev_f32(inp.beta), whole)
    Aw, Bw = kda.fwd_segment_map(ws1, io, 1, inp.T, inp.H, inp.dk, whole)
    torch.cuda.synchronize()
    direct = composed = 0.0
    for h in range(inp.H):
        A_ref, B_ref = oracle.segment_map(inp.k[0, :, h], inp.v[0, :, h], inp.g[0, :, h], inp.beta[0, :, h])
        direct = max(direct, err_A(host(Aw[0, h]), A_ref, "bf16"), err_state(host(Bw[0, h]), B_ref, "bf16"))
        composed = max(composed, err_A(host(A12[h]), A_ref, "bf16"), err_state(host(B12[h]), B_ref, "bf16"))
    print(f"map of the concatenation: err {direct:.3e}; composed from the two maps: err {composed:.3e}")
    assert direct <= tol("bf16") and composed <= tol("bf16")


def run_segmented(inp, seg_lengths):
    cu = _bounds(seg_lengths)
    assert cu[-1] == inp.T and inp.B == 1
    q, k, v = (dev_io(x, inp.io) for x in (inp.q, inp.k, inp.v))
    S0 = None if inp.S0 is None else dev_f32(inp.S0)
    o, S, _, _, _ = kda.fwd_segmented(q, k, v, dev_f32(inp.g), dev_f32(inp.beta),
                                      torch.from_numpy(cu.astype(np.int32)).to(DEV), 1.0, S0)
    torch.cuda.synchronize()
    return o, S


def check_segmented(inp, seg_lengths, label, heads=None):
    o, S = run_segmented(inp, seg_lengths)
    R = oracle.Recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, 1.0, inp.S0)
    chains = None if heads is None else [(0, h) for h in heads]
    worst_o = worst_s = 0.0
    for (n, h), (o_ref, S_ref) in R.run(chains).items():
        worst_o = max(worst_o, err(host(o[0, :, h]), o_ref, inp.io))
        worst_s = max(worst_s, err_state(host(S[0, h]), S_ref, inp.io))
    print(f"segmented {label}: o err {worst_o:.3e}, state err {worst_s:.3e}")
    assert worst_o <= tol(inp.io) and worst_s <= tol(inp.io), (label, worst_o, worst_s)
    return o, S


def test_segmented_equals_whole_sequence_weak_decay():
    """T = 4096, H = 4, S_0 given, split into 4 uneven segments (two not whole chunks)."""
    inp = ki.make_dense(1, 4096, 4, 128, 128, "bf16", 93220, s0_std=0.02, g_shift=-5.0)
    o, S = check_segmented(inp, [1024, 1000, 1100, 972], "T=4096 P=4 weak decay")
    # and against the unsplit GPU path (a different summation order of the same recurrence)
    q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o1, S1 = kda.fwd(q, k, v, dev_f32(inp.g), dev_f32(inp.beta), 1.0, dev_f32(inp.S0))
    torch.cuda.synchronize()
    e_o, e_s = err(host(o), host(o1), "bf16"), err_state(host(S), host(S1), "bf16")
    print(f"segmented vs unsplit GPU path: o {e_o:.3e}, state {e_s:.3e}")
    # each is within tol of the oracle, so they differ by at most twice that
    assert e_o <= 2 * tol("bf16") and e_s <= 2 * tol("bf16")


def test_segmented_single_segment_and_fp32():
    inp = ki.make_dense(1, 300, 2, 64, 64, "f32", 93221, s0_std=0.02, g_shift=-5.0)
    check_segmented(inp, [300], "fp32 P=1")
    check_segmented(inp, [64, 1, 100, 135], "fp32 P=4")


def test_segmented_zero_initial_state_and_empty_segments():
    """No initial state (zero), and empty segments inside the split (their map is the identity)."""
    inp = ki.make_dense(1, 700, 3, 128, 128, "bf16", 93222, s0_std=None, g_shift=-5.0)
    check_segmented(inp, [0, 256, 0, 300, 144, 0], "bf16 S_0 = 0, empty segments")


def test_segmented_long_context_p8_sampled():
    """The long-context workload (B=1, H=32, T=131072, S_0 given) split into 8 segments of 16384
    tokens, one per device of an 8-way split; sampled heads checked in full."""
    inp = ki.long_context()
    check_segmented(inp, [16384] * 8, "T=131072 P=8", heads=[0, 19, 31])


def _phases_equal_fused(kind):
    """kda_fwd_chunk_local_<kind>_gate + kda_fwd_state_scan is bitwise the fused entry point."""
    if kind == "scalar":
        inp = ki.make_scalar_gate([300], 2, 128, "bf16", 93230, dense_B=2)
        q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
        g, beta, S0 = dev_f32(inp.g), dev_f32(inp.beta), dev_f32(inp.S0)
        o1, S1 = kda.fwd_scalar_gate(q, k, v, g, beta, 1.0, S0)
        ws = kda.fwd_chunk_local(q, k, v, g, beta, gate="scalar")
        B, T, H, d = inp.q.shape
    else:
        inp = ki.make_lowrank(2, 300, 2, 128, 32, 93231)
        q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
        lr = (dev_io(inp.z, "bf16"), dev_io(inp.w_up, "bf16"), dev_f32(inp.b))
        beta, S0 = dev_f32(inp.beta), dev_f32(inp.S0)
        o1, S1 = kda.fwd_lowrank_gate(q, k, v, *lr, beta, 1.0, S0)
        ws = kda.fwd_chunk_local(q, k, v, None, beta, gate="lowrank", lowrank=lr)
        B, T, H, d = inp.q.shape
    o2, S2 = kda.fwd_state_scan(ws, kda.KDA_BF16, B, T, H, d, None, 1.0, S0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("kind", ["scalar", "lowrank"])
def test_chunk_local_phase_of_each_gate_form_is_the_fused_call(kind):
    _phases_equal_fused(kind)


def test_segmented_scalar_gate():
    """One decay per token and head, one sequence in 3 segments, against the oracle over the
    unsplit sequence (the decay copied to every key channel)."""
    inp = ki.make_scalar_gate([1500], 3, 128, "bf16", 93232, dense_B=1, g_shift=-5.0)
    q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(_bounds([512, 700, 288]).astype(np.int32)).to(DEV)
    o, S, _, _, _ = kda.fwd_segmented(q, k, v, dev_f32(inp.g), dev_f32(inp.beta), cu, 1.0, dev_f32(inp.S0),
                                      gate="scalar")
    torch.cuda.synchronize()
    gb = ki.broadcast_gate(inp.g, inp.q)
    res = oracle.Recurrence(inp.q, inp.k, inp.v, gb, inp.beta, 1.0, inp.S0).run()
    e_o = max(err(host(o[0, :, h]), o_ref, "bf16") for (_, h), (o_ref, _) in res.items())
    e_s = max(err_state(host(S[0, h]), S_ref, "bf16") for (_, h), (_, S_ref) in res.items())
    print(f"segmented scalar gate: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o <= tol("bf16") and e_s <= tol("bf16")


def test_segmented_lowrank_gate():
    """The gate in low-rank form (log alpha formed inside the chunk-local kernel), one sequence in
    4 segments, against the oracle over the unsplit sequence with g from the oracle's gate."""
    inp = ki.make_lowrank(1, 1200, 2, 128, 32, 93233, b_mean=-5.0)
    q, k, v = (dev_io(x, "bf16") for x in (inp.q, inp.k, inp.v))
    lr = (dev_io(inp.z, "bf16"), dev_io(inp.w_up, "bf16"), dev_f32(inp.b))
    cu = torch.from_numpy(_bounds([256, 333, 400, 211]).astype(np.int32)).to(DEV)
    o, S, _, _, _ = kda.fwd_segmented(q, k, v, None, dev_f32(inp.beta), cu, 1.0, dev_f32(inp.S0),
                                      gate="lowrank", lowrank=lr)
    torch.cuda.synchronize()
    B, T, H, d = inp.q.shape
    g = oracle.gate_g(inp.z.reshape(B * T, -1), inp.w_up, inp.b, H, d).reshape(B, T, H, d)
    res = oracle.Recurrence(inp.q, inp.k, inp.v, g, inp.beta, 1.0, inp.S0).run()
    e_o = max(err(host(o[0, :, h]), o_ref, "bf16") for (_, h), (o_ref, _) in res.items())
    e_s = max(err_state(host(S[0, h]), S_ref, "bf16") for (_, h), (_, S_ref) in res.items())
    print(f"segmented low-rank gate: o err {e_o:.3e}, state err {e_s:.3e}")
    assert e_o <= tol("bf16") and e_s <= tol("bf16")
