"""The seeded input generator (CPU): reproducibility and the standalone gate redraw."""
import numpy as np

import kda_inputs as ki


def test_dense_gate_redraw_is_bitwise_the_full_draw():
    """dense_gate gives exactly the g that make_dense draws for the same seed and shift."""
    for shift in (2.0, -5.0):
        full = ki.make_dense(2, 70, 3, 16, 8, "bf16", 777, s0_std=0.02, g_shift=shift)
        alone = ki.dense_gate(2, 70, 3, 16, 8, 777, shift)
        assert np.array_equal(full.g, alone)


def test_draws_are_reproducible_and_distributed_as_stated():
    a = ki.make_dense(1, 4096, 4, 128, 128, "bf16", 5)
    b = ki.make_dense(1, 4096, 4, 128, 128, "bf16", 5)
    assert all(np.array_equal(x, y) for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta)))
    # q, k unit rows (up to bf16 rounding); log-decay -softplus(N(0,1) + 2): median alpha ~ 0.12
    assert np.allclose(np.linalg.norm(a.q.astype(np.float64), axis=-1), 1.0, atol=1e-2)
    assert 0.10 < np.median(np.exp(a.g)) < 0.14
    assert np.all(a.g < 0) and np.all((a.beta > 0) & (a.beta < 1))
    w = ki.make_dense(1, 4096, 4, 128, 128, "bf16", 5, g_shift=-5.0)
    assert 0.98 < np.median(np.exp(w.g)) < 0.996
