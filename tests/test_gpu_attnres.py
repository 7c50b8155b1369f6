"""Parity of Block AttnRes on the GPU with the fp64 oracle (pinned by tests/test_oracle_attnres.py).

kda_attnres (one-shot read-out of a layer over its blocks), kda_attnres_inter (phase 1 of the
two-phase inference: per layer the softmax-weighted mean over the stored blocks and the
log-sum-exp of the scores) and kda_attnres_merge (phase 2: one layer's partial block merged in).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, floored_rel, host, rel_inf, tol

pytestmark = pytest.mark.gpu
EPS = 1e-6


def blocks_dev(V):
    return [dev_io(V[b], "bf16") for b in range(V.shape[0])]


@pytest.mark.parametrize("n,T,d", [(1, 37, 512), (3, 1000, 2048), (8, 257, 1536), (16, 64, 4096), (5, 1, 1024)])
def test_attnres_one_shot(n, T, d):
    V, W = ki.attnres_inputs(n, T, d, 1, 93300 + n + d)
    h = host(kda.attnres(blocks_dev(V), dev_io(W[0], "bf16"), EPS))
    e = floored_rel(h, oracle.attnres(V, W[0], EPS))
    print(f"attnres n={n} T={T} d={d}: err {e:.3e}")
    assert e <= tol("bf16")


def test_attnres_sharp_scores():
    """Scores of size ~75: the softmax is nearly one-hot; the online form must not overflow."""
    V, W = ki.attnres_inputs(6, 300, 2048, 1, 93310, score_std=50.0)
    h = host(kda.attnres(blocks_dev(V), dev_io(W[0], "bf16"), EPS))
    e = floored_rel(h, oracle.attnres(V, W[0], EPS))
    print(f"attnres sharp scores: err {e:.3e}")
    assert e <= tol("bf16")


@pytest.mark.parametrize("n,L,T,d", [(1, 1, 100, 512), (7, 12, 500, 2048), (4, 16, 130, 1024), (16, 5, 70, 4096)])
def test_attnres_two_phase(n, L, T, d):
    """Phase 1 over n stored blocks for L layers, then phase 2 with a partial block per layer,
    against the oracle read-out over the n + 1 blocks; phase 1's outputs against the oracle too."""
    V, W = ki.attnres_inputs(n + 1, T, d, L, 93320 + n + L)
    hist, part = V[:n], V[n]
    o, lse = kda.attnres_inter(blocks_dev(hist), dev_io(W, "bf16"), EPS)
    pd = dev_io(part, "bf16")
    e_o = e_l = e_h = 0.0
    for l in range(L):
        e_o = max(e_o, floored_rel(host(o[l]), oracle.attnres(hist, W[l], EPS)))
        e_l = max(e_l, rel_inf(host(lse[l]), oracle.attnres_lse(hist, W[l], EPS)))
        h = kda.attnres_merge(pd, dev_io(W[l], "bf16"), o[l], lse[l], EPS)
        e_h = max(e_h, floored_rel(host(h), oracle.attnres(V, W[l], EPS)))
    print(f"attnres two-phase n={n} L={L} T={T} d={d}: o err {e_o:.3e}, lse err {e_l:.3e}, merged err {e_h:.3e}")
    assert e_o <= tol("bf16") and e_h <= tol("bf16") and e_l <= tol("f32")


def test_attnres_merge_without_history_returns_partial():
    V, W = ki.attnres_inputs(1, 50, 1024, 1, 93330)
    pd = dev_io(V[0], "bf16")
    lse = torch.full((50,), float("-inf"), dtype=torch.float32, device=DEV)
    o = torch.zeros((50, 1024), dtype=torch.bfloat16, device=DEV)
    h = kda.attnres_merge(pd, dev_io(W[0], "bf16"), o, lse, EPS)
    torch.cuda.synchronize()
    assert torch.equal(h, pd)


def test_attnres_two_phase_matches_one_shot_on_gpu():
    n, L, T, d = 7, 12, 333, 2048
    V, W = ki.attnres_inputs(n + 1, T, d, L, 93340)
    bl = blocks_dev(V)
    o, lse = kda.attnres_inter(bl[:n], dev_io(W, "bf16"), EPS)
    worst = 0.0
    for l in range(L):
        wl = dev_io(W[l], "bf16")
        h2 = host(kda.attnres_merge(bl[n], wl, o[l], lse[l], EPS))
        h1 = host(kda.attnres(bl, wl, EPS))
        worst = max(worst, floored_rel(h2, h1))
    print(f"attnres two-phase vs one-shot on the GPU: {worst:.3e}")
    assert worst <= tol("bf16")


def test_attnres_output_may_alias_a_block():
    """h may be one of the input blocks (each element is read before it is written)."""
    V, W = ki.attnres_inputs(4, 300, 1024, 1, 93360)
    bl = blocks_dev(V)
    wd = dev_io(W[0], "bf16")
    ref = kda.attnres(bl, wd, EPS).clone()
    kda.attnres(bl, wd, EPS, h=bl[2])
    torch.cuda.synchronize()
    assert torch.equal(bl[2], ref)


@pytest.mark.parametrize("target", ["partial", "o"])
def test_attnres_merge_output_may_alias_its_inputs(target):
    n, L, T, d = 3, 2, 200, 512
    V, W = ki.attnres_inputs(n + 1, T, d, L, 93370)
    bl = blocks_dev(V)
    o, lse = kda.attnres_inter(bl[:n], dev_io(W, "bf16"), EPS)
    wd = dev_io(W[1], "bf16")
    ref = kda.attnres_merge(bl[n], wd, o[1], lse[1], EPS).clone()
    out = bl[n] if target == "partial" else o[1]
    kda.attnres_merge(bl[n], wd, o[1], lse[1], EPS, h=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
