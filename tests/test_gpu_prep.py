"""kda_prep (short causal conv -> SiLU -> L2 norm) against the fp64 oracle (GPU, C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_93_amd as kda
import kda_inputs as ki
import oracle
from gpu_util import DEV, dev_f32, dev_io, err, host, tol

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io,d,W", [("bf16", 128, 4), ("f32", 64, 4), ("bf16", 64, 1), ("f32", 128, 8),
                                    ("bf16", 128, 3), ("f32", 128, 2)])
def test_prep_varlen(io, d, W):
    lengths = [1, 3, 31, 32, 33, 0, 64, 100, 5, 2]
    H = 3
    x, w, cu = ki.prep_inputs(lengths, H, d, io, 17 + W, width=W)
    y = kda.prep(dev_io(x, io), dev_f32(w), cu_seqlens=torch.from_numpy(cu).to(DEV))
    ref = oracle.prep(x, w, cu, H, d)
    yh = host(y).reshape(-1, H * d)
    ref_all = np.concatenate([ref[n] for n in range(len(lengths))])
    e = err(yh, ref_all, io)
    print(f"prep {io} d={d} W={W}: err {e:.3e}")
    assert e <= tol(io)


def test_prep_dense_rows_are_sequences():
    B, T, H, d = 3, 45, 2, 128
    x, w, _ = ki.prep_inputs([T] * B, H, d, "bf16", 99)
    xb = x.reshape(B, T, H, d)
    y = host(kda.prep(dev_io(xb, "bf16"), dev_f32(w)))
    for b in range(B):
        ref = oracle.prep_sequence(xb[b].reshape(T, H * d), w, H, d)
        assert err(y[b].reshape(T, H * d), ref, "bf16") <= tol("bf16")


def test_prep_varlen_layer_shape_sampled():
    """The varlen layer packing (64 sequences, lengths U[512, 16384], H = 32, d = 128, width 4): the whole
    batch runs on the GPU, 4 sampled sequences are checked against the oracle."""
    lengths = ki.varlen_layer_lengths()
    H, d = 32, 128
    x, w, cu = ki.prep_inputs(lengths, H, d, "bf16", ki.SEED_BASE + 4)
    y = kda.prep(dev_io(x, "bf16"), dev_f32(w), cu_seqlens=torch.from_numpy(cu).to(DEV))
    for n in (0, 17, 40, 63):
        ref = oracle.prep_sequence(x[0, cu[n]:cu[n + 1]].reshape(-1, H * d), w, H, d)
        e = err(host(y[0, cu[n]:cu[n + 1]]).reshape(-1, H * d), ref, "bf16")
        assert e <= tol("bf16"), (n, e)


def test_prep_many_short_sequences():
    """Blocks of 64 tokens that cross dozens of sequence starts (lengths 0..3), a ragged last block,
    and a head count that leaves most threads of the second head group idle."""
    lengths = [(3 * i) % 4 for i in range(150)]
    H, d = 17, 128
    x, w, cu = ki.prep_inputs(lengths, H, d, "bf16", 4711, width=4)
    y = kda.prep(dev_io(x, "bf16"), dev_f32(w), cu_seqlens=torch.from_numpy(cu).to(DEV))
    ref = oracle.prep(x, w, cu, H, d)
    ref_all = np.concatenate([ref[n] for n in range(len(lengths))])
    e = err(host(y).reshape(-1, H * d), ref_all, "bf16")
    print(f"prep, 150 sequences of 0..3 tokens ({cu[-1]} tokens), H=17: err {e:.3e}")
    assert e <= tol("bf16")
