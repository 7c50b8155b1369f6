"""The fp64 oracle against the pins fixed by the pages and by mathematics (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def chain_fn():
    return pins.load_chain_fn(oracle.build(force=False))


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_pin(chain_fn, pin):
    err = pin(chain_fn)
    assert err <= pin.tol, f"{pin.__name__}: error {err:.3e} > {pin.tol:.1e}"


def test_p3_gdn_ordering_is_not_the_adopted_one(chain_fn):
    """Blog post-114 (chapter 3) reads the memory before decaying it in its Gated DeltaNet; the
    course page (section 3) decays first.  Read-before-decay is the transition
    S_t = (a_t I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, decay-first the one with
    a_t (I - beta_t k_t k_t^T).  The oracle follows the course page: with alpha != 1 the two
    orders differ; with alpha == 1 they coincide.
    """
    rng = np.random.default_rng(3)
    L, dk, dv = 6, 4, 3
    q, k, v = (rng.standard_normal((L, d)).astype(np.float32) for d in (dk, dk, dv))
    beta = np.full(L, 0.75, np.float32)
    for a, should_match in ((0.5, False), (1.0, True)):
        g = np.full((L, dk), np.log(a), np.float32)
        S = np.zeros((dk, dv))
        o_read_first = np.zeros((L, dv))
        for t in range(L):
            kt = k[t].astype(np.float64)
            A = float(np.exp(g[t, 0])) * np.eye(dk) - 0.75 * np.outer(kt, kt)
            S = A.dot(S) + 0.75 * np.outer(kt, v[t].astype(np.float64))
            o_read_first[t] = S.T.dot(q[t].astype(np.float64))
        o, _ = chain_fn(q, k, v, g, beta, 1.0, None)
        assert np.allclose(o, o_read_first, rtol=1e-12, atol=1e-12) == should_match


def test_recurrence_wrapper_matches_chain():
    """The batched wrapper (strided views of [B, T, H, d]) equals per-chain calls on copies."""
    import kda_inputs as ki
    inp = ki.make_dense(2, 70, 3, 8, 6, "f32", 5, s0_std=0.3)
    o, S = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, 0.8, inp.S0, threads=2)
    for n in range(2):
        for h in range(3):
            oc, Sc = oracle.chain(inp.q[n, :, h], inp.k[n, :, h], inp.v[n, :, h], inp.g[n, :, h],
                                  inp.beta[n, :, h], 0.8, inp.S0[n, h])
            assert np.array_equal(o[n, :, h], oc)
            assert np.array_equal(S[n, h], Sc)


def test_varlen_wrapper_isolates_sequences():
    """Packed sequences: each equals the same sequence run alone (state restarts per sequence)."""
    import kda_inputs as ki
    inp = ki.make_varlen([5, 17, 1, 9], 2, 6, 6, "bf16", 9)
    o, S = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, 1.0, inp.S0, inp.cu_seqlens)
    for n in range(4):
        s, e = inp.cu_seqlens[n], inp.cu_seqlens[n + 1]
        for h in range(2):
            oc, Sc = oracle.chain(inp.q[0, s:e, h], inp.k[0, s:e, h], inp.v[0, s:e, h],
                                  inp.g[0, s:e, h], inp.beta[0, s:e, h], 1.0, inp.S0[n, h])
            assert np.array_equal(o[0, s:e, h], oc)
            assert np.array_equal(S[n, h], Sc)


def test_nan_propagates(chain_fn):
    """No clamping: a NaN input reaches the outputs."""
    q, k, v, g, beta, S0 = pins._rand_case(1, 4, 3, 3)
    v[2, 1] = np.nan
    o, S = chain_fn(q, k, v, g, beta, 1.0, S0)
    assert np.isnan(o[2:]).any() and np.isnan(S).any() and not np.isnan(o[:2]).any()


def test_gpu_factorisation_plan_is_exact_at_workload_decay():
    """The sub-block factorisation and blocked inverse reproduce the recurrence in fp64 at the
    workload's decay strength (log-decay spans of ~140 per 64-token chunk), with a ragged tail."""
    import kda_inputs as ki
    from chunk_model import chunk_forward_gpu_plan
    inp = ki.make_dense(1, 200, 2, 32, 24, "f32", 123, s0_std=0.5)
    for h in range(2):
        args = (inp.q[0, :, h], inp.k[0, :, h], inp.v[0, :, h], inp.g[0, :, h], inp.beta[0, :, h])
        o_ref, S_ref = oracle.chain(*args, 1.0, inp.S0[0, h])
        o, S = chunk_forward_gpu_plan(*args, 1.0, inp.S0[0, h])
        assert np.max(np.abs(o - o_ref)) <= 1e-11 * np.max(np.abs(o_ref))
        assert np.max(np.abs(S - S_ref)) <= 1e-11 * np.max(np.abs(S_ref))
