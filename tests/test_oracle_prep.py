"""The fp64 prologue oracle (conv -> SiLU -> L2 norm) against closed forms and library routines."""
import math

import numpy as np
import pytest
import torch

import oracle
import pins


def _golden_prep():
    r = pins._parse_golden("prep_hand_example.txt")
    ev = lambda xs: np.array([eval(x, {"log": math.log, "sqrt": math.sqrt}) for x in xs], np.float64)
    return ev(r["w"]).reshape(2, 4), ev(r["x"]).reshape(3, 2), ev(r["y"]).reshape(3, 2)


def test_hand_example():
    w, x, y_ref = _golden_prep()
    y = oracle.prep_sequence(x, w, H=1, d=2)
    assert np.max(np.abs(y - y_ref)) < 1e-15


def test_matches_numpy_convolve_and_torch_functional():
    """Special case that reduces to library routines: np.convolve per channel, and torch's
    depthwise conv1d + silu + normalize (CPU, float64)."""
    rng = np.random.default_rng(0)
    L, H, d, W = 29, 3, 8, 4
    x = rng.standard_normal((L, H * d))
    w = rng.standard_normal((H * d, W)) * 0.5
    y = oracle.prep_sequence(x, w, H, d)
    # numpy: full convolution with the reversed taps, first L outputs = causal window
    conv = np.stack([np.convolve(x[:, c], w[c, ::-1])[:L] for c in range(H * d)], axis=1)
    s = conv / (1 + np.exp(-conv))
    s = s.reshape(L, H, d)
    y_np = (s / np.maximum(np.linalg.norm(s, axis=-1, keepdims=True), 1e-12)).reshape(L, H * d)
    assert np.max(np.abs(y - y_np)) < 1e-13
    # torch.nn.functional: conv1d(groups=C, left padding W-1), silu, normalize(dim=-1)
    xt = torch.from_numpy(x.T[None])                      # [1, C, L]
    wt = torch.from_numpy(w[:, None, :])                  # [C, 1, W]
    ct = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (W - 1, 0)), wt, groups=H * d)
    st = torch.nn.functional.silu(ct)[0].T.reshape(L, H, d)
    yt = torch.nn.functional.normalize(st, dim=-1).reshape(L, H * d).numpy()
    assert np.max(np.abs(y - yt)) < 1e-13


def test_identity_taps_and_unit_norm():
    rng = np.random.default_rng(1)
    L, H, d = 17, 2, 16
    x = rng.standard_normal((L, H * d))
    w = np.zeros((H * d, 4))
    w[:, 3] = 1.0
    y = oracle.prep_sequence(x, w, H, d).reshape(L, H, d)
    s = x / (1 + np.exp(-x))
    s = s.reshape(L, H, d)
    assert np.max(np.abs(y - s / np.linalg.norm(s, axis=-1, keepdims=True))) < 1e-14
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - 1)) < 1e-14


def test_zero_input_gives_zero():
    y = oracle.prep_sequence(np.zeros((5, 8)), np.ones((8, 4)), 2, 4)
    assert np.all(y == 0)


def test_causality_and_sequence_isolation():
    rng = np.random.default_rng(2)
    lengths = [7, 3, 12]
    H, d = 2, 4
    cu = np.concatenate([[0], np.cumsum(lengths)])
    x = rng.standard_normal((cu[-1], H * d))
    w = rng.standard_normal((H * d, 4))
    base = oracle.prep(x, w, cu, H, d)
    # causality: perturbing token t of sequence 2 leaves its earlier tokens unchanged
    x2 = x.copy()
    x2[cu[2] + 6] += 3.0
    pert = oracle.prep(x2, w, cu, H, d)
    assert np.array_equal(pert[2][:6], base[2][:6]) and not np.allclose(pert[2][6:], base[2][6:])
    # isolation: the other sequences do not change; history resets at each sequence start
    assert np.array_equal(pert[0], base[0]) and np.array_equal(pert[1], base[1])
    alone = oracle.prep_sequence(x[cu[1]:cu[2]], w, H, d)
    assert np.array_equal(alone, base[1])
