"""Benchmark of the KDA operator on one MI355X.

One step = one chunked prefill (kda_fwd) of the 4 x 4096-token, 16-head, d = 128 batch
(bf16 q/k/v, fp32 log-decay/beta/state, chunk 64): the headline "prefill tokens/s".
The same run also measures
  * the decode step (256 sequences x 32 heads, d = 128, fp32 state resident in HBM,
    100 consecutive steps): state GB/s and fraction of HBM peak;
  * the q/k prologue on the packed 64-sequence batch (lengths U[512, 16384], H = 32):
    GB/s;
  * the prefill batch with one decay per token and head, and with none (kda_fwd_scalar_gate);
  * the long-context prefill (B = 1, H = 32, T = 131072) and the varlen layer (prologue on q
    and k, then the prefill of the packed 64-sequence batch): ms and tokens/s;
  * the long-context prefill split into 8 segments of 16384 tokens (segment maps, the hop
    between segments, the scan from the incoming states): one segment's kernels, and all
    eight run on this GPU;
  * the low-rank gate prologue and the fused prefill, and Block AttnRes (one-shot and
    two-phase);
  * the fp64 CPU oracle on a bounded sample of the prefill workload (cpu_baseline).
Per-kernel times come from HIP events recorded on the stream the kernels run on.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill,decode,prep,scalar,gate,attnres,long,kcp,varlen,cpu,copy]
Prints one JSON line.  `--only copy` runs a plain 256 MiB device copy (a kernel of known size
used to calibrate the FETCH_SIZE / WRITE_SIZE counters of profiler runs).
The roofline "traffic" figure comes from profiles/traffic.json (counter runs of this same
script); it is reported only while the hash of the kernel source recorded there matches.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "KDA prefill tokens/s + MFMA %; decode-step state GB/s + % HBM peak"

# Algorithmic work per token-head of the prefill (d = 128, chunk 64): the inputs q, k, v (bf16)
# and g (fp32), beta, the output o (bf16): 3*256 + 512 + 4 + 256 bytes; flops of the chunkwise
# form (triangle-aware): 140.5 KFLOP.
PREFILL_IN_BYTES = 3 * 256 + 512 + 4
PREFILL_OUT_BYTES = 256
PREFILL_BYTES = PREFILL_IN_BYTES + PREFILL_OUT_BYTES   # 1,540 B per token-head
PREFILL_FLOP = 140.5e3
# kernel names as rocprofv3 reports them
K_LOCAL = "kda::chunk_local_kernel<true, 128, false>"
K_SCAN_2T = "kda::chunk_scan_kernel<true, 128, 2, 4, false>"   # two column tiles per workgroup
K_SCAN_1T = "kda::chunk_scan_kernel<true, 128, 1, 4, false>"   # one tile, four waves (few chains)
K_DECODE = "kda::decode_step_kernel<unsigned short, 128, 128>"
K_PREP = "kda::prep_kernel<unsigned short, 128, 4>"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bf16_dev(x, dev):
    import torch
    import kda_inputs as ki
    return torch.from_numpy(ki.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)


def time_events(fn, reps, torch):
    """Average ms of fn() over reps, with HIP events on the current stream."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / reps


def bench_prefill(args, torch, kda, dev):
    import kda_inputs as ki
    inp = ki.prefill_batch()
    B, T, H, d = inp.B, inp.T, inp.H, inp.dk
    q, k, v = (bf16_dev(x, dev) for x in (inp.q, inp.k, inp.v))
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, B, T, H, d, d, B, False)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    L = kda.lib()
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()

    def step():
        rc = L.kda_fwd(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(g), p(beta), 1.0, None, p(S),
                       p(o), p(ws), nws, stream)
        assert rc == 0, kda.status_string(rc)

    def local():
        assert L.kda_fwd_chunk_local(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(g), p(beta),
                                     p(ws), nws, stream) == 0

    def scan():
        assert L.kda_fwd_state_scan(kda.KDA_BF16, B, T, H, d, d, None, B, 1.0, None, p(S), p(o), p(ws), nws,
                                    stream) == 0

    # Untimed settle phase: the same step until ~100 ms have run.  The GPU raises its clocks
    # under sustained load, and a few warmup steps of ~0.3 ms each end before it has (the first
    # 20 steps after them measured ~15% slower than steady state).
    settle_steps = 0
    t_s = time.perf_counter()
    while time.perf_counter() - t_s < 0.1:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    # per-kernel times (events around each phase launch, same stream)
    reps = max(args.steps, 5)
    ms_local = time_events(local, reps, torch)
    ms_scan = time_events(scan, reps, torch)
    ms_fwd = time_events(step, reps, torch)
    tokens = B * T
    token_heads = B * T * H
    res = dict(tokens=tokens, token_heads=token_heads, ms_step=ms_step, ms_fwd_events=ms_fwd,
               ms_chunk_local=ms_local, ms_state_scan=ms_scan,
               ws_bytes_per_chunk_head=nws // (B * ((T + 63) // 64) * H), settle_steps=settle_steps)
    return res, inp


def bench_decode(args, torch, kda, dev):
    N, H, d, steps = 256, 32, 128, 100
    gen = torch.Generator(device=dev)
    gen.manual_seed(93003)
    state = (torch.randn((N, H, d, d), generator=gen, device=dev, dtype=torch.float32) * 0.02).contiguous()

    def unit(x):
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16).contiguous()

    toks = []
    for _ in range(steps):
        q = unit(torch.randn((N, H, d), generator=gen, device=dev))
        k = unit(torch.randn((N, H, d), generator=gen, device=dev))
        v = torch.randn((N, H, d), generator=gen, device=dev).to(torch.bfloat16)
        beta = torch.sigmoid(torch.randn((N, H), generator=gen, device=dev)).contiguous()
        g = (-torch.nn.functional.softplus(torch.randn((N, H, d), generator=gen, device=dev) + 2)).contiguous()
        toks.append((q, k, v, g, beta))
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    L = kda.lib()
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()

    def run(s):
        q, k, v, g, beta = toks[s % steps]
        assert L.kda_decode_step(kda.KDA_BF16, N, H, d, d, p(q), p(k), p(v), p(g), p(beta), 1.0, p(state),
                                 p(o), stream) == 0

    for s in range(5):
        run(s)
    torch.cuda.synchronize()
    it = iter(range(steps))
    ms = time_events(lambda: run(next(it)), steps, torch)
    state_bytes = 2 * N * H * d * d * 4
    io_bytes = N * H * (3 * d * 2 + d * 4 + 4 + d * 2)
    return dict(ms_step=ms, state_bytes=state_bytes, io_bytes=io_bytes,
                state_gbs=state_bytes / ms / 1e6, total_gbs=(state_bytes + io_bytes) / ms / 1e6)


def bench_prep(args, torch, kda, dev):
    import kda_inputs as ki
    lengths = ki.varlen_layer_lengths()
    H, d = 32, 128
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    ntok = int(cu[-1])
    gen = torch.Generator(device=dev)
    gen.manual_seed(93004)
    x = torch.randn((1, ntok, H, d), generator=gen, device=dev).to(torch.bfloat16)
    w = (torch.randn((H * d, 4), generator=gen, device=dev) * 0.5).contiguous()
    y = torch.empty_like(x)
    cu_d = torch.from_numpy(cu).to(dev)
    for _ in range(2):
        kda.prep(x, w, cu_d, y=y)
    ms = time_events(lambda: kda.prep(x, w, cu_d, y=y), 5, torch)
    nbytes = 2 * ntok * H * d * 2
    return dict(ms=ms, tokens=ntok, bytes=nbytes, gbs=nbytes / ms / 1e6)


def _unit_bf16(x):
    import torch
    return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)


def bench_long(torch, kda, dev, reps=5):
    """Long-context prefill: B=1, H=32, T=131072, d=128, S_0 ~ N(0, 0.02), one kda_fwd per rep
    (inputs drawn on the GPU with the same distributions as the parity tests)."""
    B, T, H, d = 1, 131072, 32, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(93002)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    q, k = _unit_bf16(rnd(B, T, H, d)), _unit_bf16(rnd(B, T, H, d))
    v = rnd(B, T, H, d).to(torch.bfloat16)
    beta = torch.sigmoid(rnd(B, T, H))
    g = -torch.nn.functional.softplus(rnd(B, T, H, d) + 2)
    S0 = rnd(B, H, d, d) * 0.02
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty_like(S0)
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, B, T, H, d, d, B, False)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    L = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()

    def step():
        assert L.kda_fwd(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(g), p(beta), 1.0, p(S0),
                         p(S), p(o), p(ws), nws, st) == 0

    def local():
        assert L.kda_fwd_chunk_local(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(g), p(beta),
                                     p(ws), nws, st) == 0

    def scan():
        assert L.kda_fwd_state_scan(kda.KDA_BF16, B, T, H, d, d, None, B, 1.0, p(S0), p(S), p(o), p(ws), nws,
                                    st) == 0

    step()
    torch.cuda.synchronize()
    ms = time_events(step, reps, torch)
    ms_local = time_events(local, reps, torch)
    ms_scan = time_events(scan, reps, torch)
    th = B * T * H
    return {"workload": "KDA prefill B=1 H=32 T=131072 d=128, bf16 q/k/v, S_0 ~ N(0, 0.02)",
            "ms": ms, "ms_chunk_local": ms_local, "ms_state_scan": ms_scan, "tokens_per_s": B * T / (ms / 1e3),
            "algorithmic_GBs": (PREFILL_IN_BYTES + PREFILL_OUT_BYTES) * th / ms / 1e6,
            "hbm_frac": (PREFILL_IN_BYTES + PREFILL_OUT_BYTES) * th / ms / 1e6 / HBM_PEAK_GBS}


def bench_kcp(torch, kda, dev, reps=5):
    """Segment maps (context parallelism): the long-context workload (B=1, H=32, T=131072, d=128,
    bf16, S_0 given) split into 8 segments of 16384 tokens.  (a) One segment, the share of one
    device in an 8-way split: chunk records, the segment map (A, B), one hop (kda_state_combine
    over the 32 heads) and the scan from the incoming state.  (b) All 8 segments on this GPU:
    records and maps of every segment in one launch each, the 7 serial hops, one scan."""
    P, Ts, H, d = 8, 16384, 32, 128
    T = P * Ts
    gen = torch.Generator(device=dev)
    gen.manual_seed(93007)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    q, k = _unit_bf16(rnd(1, T, H, d)), _unit_bf16(rnd(1, T, H, d))
    v = rnd(1, T, H, d).to(torch.bfloat16)
    beta = torch.sigmoid(rnd(1, T, H))
    g = -torch.nn.functional.softplus(rnd(1, T, H, d) + 2)
    S0 = rnd(1, H, d, d) * 0.02
    L = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    B16 = kda.KDA_BF16

    # (a) one device's share: the first segment's tokens as a dense batch of one sequence
    qs, ks, vs, gs, bs = (x[:, :Ts].contiguous() for x in (q, k, v, g, beta))
    nws1 = kda.fwd_workspace_bytes(B16, 1, Ts, H, d, d, 1, False)
    ws1 = torch.empty(nws1, dtype=torch.uint8, device=dev)
    A1 = torch.empty((1, H, d, d), dtype=torch.float32, device=dev)
    B1 = torch.empty_like(A1)
    S_next = torch.empty_like(A1)
    S_end = torch.empty_like(A1)
    o1 = torch.empty((1, Ts, H, d), dtype=torch.bfloat16, device=dev)

    def local1():
        assert L.kda_fwd_chunk_local(B16, 1, Ts, H, d, d, None, 1, p(qs), p(ks), p(vs), p(gs), p(bs), p(ws1),
                                     nws1, st) == 0

    def map1():
        assert L.kda_fwd_segment_map(B16, 1, Ts, H, d, d, None, 1, p(A1), p(B1), p(ws1), nws1, st) == 0

    def hop1():
        assert L.kda_state_combine(H, d, d, p(A1), p(S0), p(B1), p(S_next), st) == 0

    def scan1():
        assert L.kda_fwd_state_scan(B16, 1, Ts, H, d, d, None, 1, 1.0, p(S0), p(S_end), p(o1), p(ws1), nws1,
                                    st) == 0

    # (b) all segments on this GPU
    cu = torch.arange(0, T + 1, Ts, dtype=torch.int32, device=dev)
    nws = kda.fwd_workspace_bytes(B16, 1, T, H, d, d, P, True)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    A = torch.empty((P, H, d, d), dtype=torch.float32, device=dev)
    Bm = torch.empty_like(A)
    S_in = torch.empty_like(A)
    S_out = torch.empty_like(A)
    o = torch.empty((1, T, H, d), dtype=torch.bfloat16, device=dev)
    seg = H * d * d * 4  # bytes of one segment's maps or states

    def whole():
        assert L.kda_fwd_chunk_local(B16, 1, T, H, d, d, p(cu), P, p(q), p(k), p(v), p(g), p(beta), p(ws), nws,
                                     st) == 0
        assert L.kda_fwd_segment_map(B16, 1, T, H, d, d, p(cu), P, p(A), p(Bm), p(ws), nws, st) == 0
        S_in[0].copy_(S0[0])
        for j in range(P - 1):
            assert L.kda_state_combine(H, d, d, p(A) + j * seg, p(S_in) + j * seg, p(Bm) + j * seg,
                                       p(S_in) + (j + 1) * seg, st) == 0
        assert L.kda_fwd_state_scan(B16, 1, T, H, d, d, p(cu), P, 1.0, p(S_in), p(S_out), p(o), p(ws), nws,
                                    st) == 0

    local1(); map1(); hop1(); scan1(); whole()
    torch.cuda.synchronize()
    ms_l, ms_m = time_events(local1, reps, torch), time_events(map1, reps, torch)
    ms_h, ms_s = time_events(hop1, 20, torch), time_events(scan1, reps, torch)
    ms_w = time_events(whole, reps, torch)
    return {"workload": "KDA prefill B=1 H=32 T=131072 d=128 bf16, S_0 given, in 8 segments of 16384",
            "segment_ms": {"chunk_local": ms_l, "segment_map": ms_m, "hop": ms_h, "state_scan": ms_s},
            "segment_map_overhead": (ms_m + ms_h) / (ms_l + ms_s),
            "all_segments_one_gpu_ms": ms_w, "all_segments_tokens_per_s": T / (ms_w / 1e3)}


def bench_scalar_gate(torch, kda, dev, reps=20):
    """The prefill batch (B=4, H=16, T=4096, d=128, bf16) with one log-decay per token and head
    (kda_fwd_scalar_gate), and with none (alpha = 1)."""
    B, T, H, d = 4, 4096, 16, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(93106)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    q, k = _unit_bf16(rnd(B, T, H, d)), _unit_bf16(rnd(B, T, H, d))
    v = rnd(B, T, H, d).to(torch.bfloat16)
    beta = torch.sigmoid(rnd(B, T, H))
    g = -torch.nn.functional.softplus(rnd(B, T, H) + 2)
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, B, T, H, d, d, B, False)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    L = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: None if t is None else t.data_ptr()

    def run(gp):
        assert L.kda_fwd_scalar_gate(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), gp, p(beta), 1.0,
                                     None, p(S), p(o), p(ws), nws, st) == 0

    out = {"workload": "KDA prefill B=4 H=16 T=4096 d=128 bf16, one log-decay per token and head "
                       "(Gated DeltaNet case) and alpha = 1 (DeltaNet case)"}
    for label, gp in (("per_head_decay", p(g)), ("alpha_one", None)):
        for _ in range(3):
            run(gp)
        torch.cuda.synchronize()
        ms = time_events(lambda: run(gp), reps, torch)
        out[label] = {"ms": ms, "tokens_per_s": B * T / (ms / 1e3)}
    return out


def bench_lowrank_gate(torch, kda, dev, reps=20):
    """The prefill batch (B=4, H=16, T=4096, d=128, bf16) with the gate in low-rank form: hidden
    width 2048, rank 32.  Times the gate prologue (z and beta; and with log alpha written out), the
    operator fed with that log alpha (kda_fwd) and the fused operator (kda_fwd_lowrank_gate), and
    the two layer totals: prologue(g) + kda_fwd versus prologue(z) + fused."""
    B, T, H, d, r, Dm = 4, 4096, 16, 128, 32, 2048
    n = B * T
    gen = torch.Generator(device=dev)
    gen.manual_seed(93240)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    x = rnd(n, Dm).to(torch.bfloat16)
    w_down = (rnd(r, Dm) / Dm ** 0.5).to(torch.bfloat16)
    w_beta = (rnd(H, Dm) / Dm ** 0.5).to(torch.bfloat16)
    w_up = (rnd(H * d, r) / r ** 0.5).to(torch.bfloat16)
    b = (2.0 + 0.5 * rnd(H * d)).contiguous()
    q, k = _unit_bf16(rnd(B, T, H, d)), _unit_bf16(rnd(B, T, H, d))
    v = rnd(B, T, H, d).to(torch.bfloat16)
    z = torch.empty((n, r), dtype=torch.bfloat16, device=dev)
    beta = torch.empty((n, H), dtype=torch.float32, device=dev)
    g = torch.empty((n, H, d), dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=dev)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, B, T, H, d, d, B, False)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    L = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: None if t is None else t.data_ptr()

    def prologue(gp):
        assert L.kda_gate(kda.KDA_BF16, n, Dm, H, d, r, p(x), p(w_down), p(w_beta), p(w_up), p(b), p(z), p(beta),
                          gp, st) == 0

    def fwd_g():
        assert L.kda_fwd(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(g), p(beta), 1.0, None, p(S),
                         p(o), p(ws), nws, st) == 0

    def fwd_fused():
        assert L.kda_fwd_lowrank_gate(kda.KDA_BF16, B, T, H, d, d, None, B, p(q), p(k), p(v), p(z), r, p(w_up), p(b),
                                      p(beta), 1.0, None, p(S), p(o), p(ws), nws, st) == 0

    prologue(p(g))
    fns = {"prologue_z_beta": lambda: prologue(None), "prologue_with_log_alpha": lambda: prologue(p(g)),
           "fwd_with_log_alpha": fwd_g, "fwd_fused": fwd_fused,
           "layer_unfused": lambda: (prologue(p(g)), fwd_g()), "layer_fused": lambda: (prologue(None), fwd_fused())}
    out = {"workload": "KDA prefill B=4 H=16 T=4096 d=128 bf16 with the gate from hidden states of width 2048 "
                       "through rank 32 (log alpha = -softplus(z W_up^T + b), beta = sigmoid(x w_beta^T))"}
    for label, fn in fns.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        out[label + "_ms"] = time_events(fn, reps, torch)
    x_bytes, zb_bytes, g_bytes = n * Dm * 2, n * (r * 2 + H * 4), n * H * d * 4
    out["prologue_z_beta_GBs"] = (x_bytes + zb_bytes) / out["prologue_z_beta_ms"] / 1e6
    out["prologue_z_beta_hbm_frac"] = out["prologue_z_beta_GBs"] / HBM_PEAK_GBS
    out["prologue_with_log_alpha_GBs"] = (x_bytes + zb_bytes + g_bytes) / out["prologue_with_log_alpha_ms"] / 1e6
    out["layer_fused_tokens_per_s"] = n / (out["layer_fused_ms"] / 1e3)
    out["layer_unfused_tokens_per_s"] = n / (out["layer_unfused_ms"] / 1e3)
    return out


def bench_attnres(torch, kda, dev, reps=20):
    """Block AttnRes over 16,384 tokens of width 2048 (the prefill batch's tokens, width H*d):
    8 blocks (7 stored + the partial one) and 12 layers per block.  Times the one-shot read-out of
    one layer over the 8 blocks, phase 1 of the two-phase inference (the 7 stored blocks scored and
    mixed for all 12 layers), and one layer's phase-2 merge; a block's total either way."""
    T, d, n, L, eps = 16384, 2048, 8, 12, 1e-6
    gen = torch.Generator(device=dev)
    gen.manual_seed(93350)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    blocks = [(rnd(T, d) * (1.0 + 0.5 * b)).to(torch.bfloat16) for b in range(n)]
    W = (rnd(L, d) * (1.5 / d ** 0.5)).to(torch.bfloat16)
    o = torch.empty((L, T, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((L, T), dtype=torch.float32, device=dev)
    h = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    L_ = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    arr_all = (ctypes.c_void_p * n)(*[b.data_ptr() for b in blocks])
    arr_hist = (ctypes.c_void_p * (n - 1))(*[b.data_ptr() for b in blocks[:-1]])
    nws = int(L_.kda_attnres_inter_workspace_bytes(n - 1, L, T))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    one = lambda: L_.kda_attnres(kda.KDA_BF16, n, T, d, arr_all, W.data_ptr(), eps, h.data_ptr(), st)
    inter = lambda: L_.kda_attnres_inter(kda.KDA_BF16, n - 1, L, T, d, arr_hist, W.data_ptr(), eps, o.data_ptr(),
                                         lse.data_ptr(), ws.data_ptr(), nws, st)
    merge = lambda: L_.kda_attnres_merge(kda.KDA_BF16, T, d, blocks[-1].data_ptr(), W.data_ptr(), eps,
                                         o.data_ptr(), lse.data_ptr(), h.data_ptr(), st)
    out = {"workload": "Block AttnRes, 16384 tokens, width 2048, bf16: 8 blocks (7 stored + partial), "
                       "12 layers per block"}
    for label, fn in (("one_shot_layer", one), ("phase1_all_layers", inter), ("phase2_merge_layer", merge)):
        for _ in range(3):
            assert fn() == 0
        torch.cuda.synchronize()
        out[label + "_ms"] = time_events(lambda: fn(), reps, torch)
    row = T * d * 2
    one_b, p1_b, p2_b = (n + 1) * row, (n - 1) * row + L * row + L * T * 4, 3 * row + T * 4
    out["one_shot_layer_GBs"] = one_b / out["one_shot_layer_ms"] / 1e6
    out["one_shot_layer_hbm_frac"] = out["one_shot_layer_GBs"] / HBM_PEAK_GBS
    out["phase1_algorithmic_GBs"] = p1_b / out["phase1_all_layers_ms"] / 1e6
    out["phase1_hbm_frac"] = out["phase1_algorithmic_GBs"] / HBM_PEAK_GBS
    out["phase2_merge_GBs"] = p2_b / out["phase2_merge_layer_ms"] / 1e6
    out["phase2_hbm_frac"] = out["phase2_merge_GBs"] / HBM_PEAK_GBS
    out["block_one_shot_ms"] = L * out["one_shot_layer_ms"]
    out["block_two_phase_ms"] = out["phase1_all_layers_ms"] + L * out["phase2_merge_layer_ms"]
    return out


def bench_varlen_layer(torch, kda, dev, reps=5):
    """Varlen layer: 64 packed sequences (lengths U[512, 16384] from the workload seed), H=32, d=128:
    prologue on raw q and k (width 4), then the chunked prefill with per-sequence S_0 ~ N(0, 0.02)."""
    import kda_inputs as ki
    lengths = ki.varlen_layer_lengths()
    H, d = 32, 128
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T, N = int(cu[-1]), len(lengths)
    gen = torch.Generator(device=dev)
    gen.manual_seed(93004)
    rnd = lambda *shape: torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    qr, kr = rnd(1, T, H, d).to(torch.bfloat16), rnd(1, T, H, d).to(torch.bfloat16)
    v = rnd(1, T, H, d).to(torch.bfloat16)
    beta = torch.sigmoid(rnd(1, T, H))
    g = -torch.nn.functional.softplus(rnd(1, T, H, d) + 2)
    wq, wk = (rnd(H * d, 4) * 0.5).contiguous(), (rnd(H * d, 4) * 0.5).contiguous()
    S0 = rnd(N, H, d, d) * 0.02
    cu_d = torch.from_numpy(cu).to(dev)
    q, k = torch.empty_like(qr), torch.empty_like(kr)
    o = torch.empty_like(v)
    S = torch.empty_like(S0)
    nws = kda.fwd_workspace_bytes(kda.KDA_BF16, 1, T, H, d, d, N, True)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    L = kda.lib()
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()

    def layer():
        assert L.kda_prep(kda.KDA_BF16, 1, T, H, d, p(cu_d), N, p(qr), p(wq), 4, p(q), st) == 0
        assert L.kda_prep(kda.KDA_BF16, 1, T, H, d, p(cu_d), N, p(kr), p(wk), 4, p(k), st) == 0
        assert L.kda_fwd(kda.KDA_BF16, 1, T, H, d, d, p(cu_d), N, p(q), p(k), p(v), p(g), p(beta), 1.0, p(S0),
                         p(S), p(o), p(ws), nws, st) == 0

    def fwd():
        assert L.kda_fwd(kda.KDA_BF16, 1, T, H, d, d, p(cu_d), N, p(q), p(k), p(v), p(g), p(beta), 1.0, p(S0),
                         p(S), p(o), p(ws), nws, st) == 0

    def local():
        assert L.kda_fwd_chunk_local(kda.KDA_BF16, 1, T, H, d, d, p(cu_d), N, p(q), p(k), p(v), p(g), p(beta),
                                     p(ws), nws, st) == 0

    def scan():
        assert L.kda_fwd_state_scan(kda.KDA_BF16, 1, T, H, d, d, p(cu_d), N, 1.0, p(S0), p(S), p(o), p(ws), nws,
                                    st) == 0

    layer()
    torch.cuda.synchronize()
    ms = time_events(layer, reps, torch)
    ms_fwd = time_events(fwd, reps, torch)
    ms_local = time_events(local, reps, torch)
    ms_scan = time_events(scan, reps, torch)
    th = T * H
    return {"workload": f"{T} packed tokens (64 sequences, lengths U[512, 16384]), H=32, d=128: 2 prologue "
                        "launches (q, k) + chunked prefill with per-sequence S_0",
            "ms_layer": ms, "ms_fwd": ms_fwd, "ms_chunk_local": ms_local, "ms_state_scan": ms_scan,
            "tokens_per_s": T / (ms / 1e3), "token_heads": th,
            "fwd_algorithmic_GBs": PREFILL_BYTES * th / ms_fwd / 1e6}


def cpu_info():
    """The host CPU as /proc/cpuinfo describes it (every identifying field, not only the model name)."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            first = f.read().split("\n\n")[0]
        fields = dict(l.split(":", 1) for l in first.splitlines() if ":" in l)
        fields = {k.strip(): v.strip() for k, v in fields.items()}
        for k in ("vendor_id", "model name", "cpu family", "model", "stepping", "cpu MHz", "cache size"):
            if k in fields:
                info[k.replace(" ", "_")] = fields[k]
    except OSError:
        pass
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def _time_oracle(fn, min_seconds):
    """Repeat fn() until min_seconds of wall time; returns (passes, seconds)."""
    passes = 0
    t0 = time.perf_counter()
    while True:
        fn()
        passes += 1
        wall = time.perf_counter() - t0
        if wall >= min_seconds or passes >= 200:
            return passes, wall


def cpu_baseline(inp, min_seconds=10.0):
    """The fp64 oracle (the plain token recurrence, one thread per (sequence, head) chain) timed on
    this host on bounded samples of every workload; the headline figure is the prefill batch on all
    threads.  Token throughput of the oracle is linear in the chains and tokens it runs (7 d_k d_v
    fp64 flops per token-head), so a sample of chains stands for its whole workload: tokens/s of a
    workload = token-heads/s / H."""
    import oracle
    import kda_inputs as ki
    threads = oracle.default_threads()
    R = oracle.Recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta)
    passes, wall = _time_oracle(lambda: R.run(threads=threads), min_seconds)
    th_rate = inp.B * inp.T * inp.H * passes / wall
    per = {}

    def sample(name, q, k, v, g, beta, S0, H_workload, desc, nthreads, budget=1.5):
        Rs = oracle.Recurrence(q, k, v, g, beta, 1.0, S0)
        chains = [(n, h) for n in range(Rs.N) for h in range(Rs.H)]
        n_, w_ = _time_oracle(lambda: Rs.run(chains, threads=nthreads), budget)
        ths = sum(Rs.bounds(n)[2] for n, _ in chains) * n_ / w_
        per[name] = {"token_heads_per_s": ths, "tokens_per_s": ths / H_workload, "threads": nthreads,
                     "sample": desc, "passes": n_, "seconds": round(w_, 2)}

    # small fp32 recurrence (B=1, H=2, T=256, d=64): the whole workload, one thread
    s0 = ki.small_fp32()
    sample("small_fp32_1thread", s0.q, s0.k, s0.v, s0.g, s0.beta, None, 2, "whole workload, 2 chains", 1, 1.0)
    # prefill batch: 2 of its 64 chains on one thread (B=4 H=16 T=4096 shape, its distributions)
    s1 = ki.make_dense(1, 4096, 2, 128, 128, "bf16", 93101)
    sample("prefill_batch_1thread", s1.q, s1.k, s1.v, s1.g, s1.beta, None, 16,
           "2 chains of 4096 tokens (d=128)", 1)
    # long context: 2 chains of 32768 tokens (1/4 of T) on two threads
    s2 = ki.make_dense(1, 32768, 2, 128, 128, "bf16", 93102, s0_std=0.02)
    sample("long_context", s2.q, s2.k, s2.v, s2.g, s2.beta, s2.S0, 32,
           "2 chains of 32768 tokens of the T=131072, H=32 shape", 2)
    # decode pool: 100 steps of 8 (sequence, head) chains, one thread (a chain of 100 tokens each)
    s3 = ki.make_dense(8, 100, 1, 128, 128, "bf16", 93103, s0_std=0.02)
    sample("decode_pool_1thread", s3.q, s3.k, s3.v, s3.g, s3.beta, s3.S0, 32,
           "8 of the 8192 chains over 100 steps; tokens/s = decode steps x sequences / s", 1)
    # varlen layer: 2 heads of 2 of its sequences (lengths from the workload), two threads
    lengths = ki.varlen_layer_lengths()[:2]
    s4 = ki.make_varlen(lengths, 2, 128, 128, "bf16", 93104)
    sample("varlen_layer", s4.q, s4.k, s4.v, s4.g, s4.beta, s4.S0, 32,
           f"2 heads of sequences 0-1 (lengths {int(lengths[0])}, {int(lengths[1])})", 2)
    return {"value": th_rate / inp.H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_info(),
            "sample": f"{passes} whole passes over the prefill batch (all {inp.B * inp.H} (sequence, head) "
                      f"chains of {inp.T} tokens), fp64 token recurrence, {wall:.1f} s wall on {threads} threads",
            "per_workload": per}


def bench_copy(torch, dev, nbytes=1 << 28):
    """Device-to-device copy of nbytes (the runtime's copy kernel), 256 MiB by default: the reference
    kernel for counter calibration, and the copy the decode step is set against in the same run
    (every large copy of a run has this one size, which the calibration relies on)."""
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    ms = time_events(lambda: y.copy_(x), 5, torch)
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms, "GBs": 2 * nbytes / ms / 1e6}


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank space removed, so a comment-only edit
    does not mark the counter profiles as taken on other code."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "gated_delta_rule_93_amd", "csrc"))):
        with open(os.path.join(ROOT, "gated_delta_rule_93_amd", "csrc", f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        code = "\n".join(line.strip() for line in src.splitlines() if line.strip())
        h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def _traffic_table():
    try:
        with open(TRAFFIC_JSON) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    return t if t.get("source_hash") == kernel_source_hash() else None


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` in the leg `workload` from profiles/traffic.json, if the
    counters were taken on the current kernel source (None otherwise)."""
    t = _traffic_table()
    k = None if t is None else t.get("workloads", {}).get(workload, {}).get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def measured_mfma(workload, kernel):
    """rocprofv3 MfmaUtil (%) and issued bf16 MFMA flops per launch of `kernel` in leg `workload`."""
    t = _traffic_table()
    return None if t is None else t.get("workloads", {}).get(workload, {}).get("mfma", {}).get(kernel)


def measured_insts(workload, kernel):
    """rocprofv3 instructions issued per wave (VALU, MFMA, LDS, SALU, VMEM) and the share of wave
    cycles spent waiting to issue LDS instructions, for `kernel` in leg `workload`."""
    t = _traffic_table()
    return None if t is None else t.get("workloads", {}).get(workload, {}).get("insts", {}).get(kernel)


# ----------------------------------------------------------------------------- profile summaries
# `python bench.py --summarize DIR` turns rocprofv3 csv output into profiles/traffic.json and the
# text summaries under profiles/.  DIR/<leg>/ holds the output of three runs of one bench leg
# (<leg> is a name of --only, e.g. prefill, long, varlen, decode, prep):
#   rocprofv3 --kernel-trace --stats -f csv -d DIR/<leg>/trace -o trace -- python3 bench.py --only <leg>,copy --steps 5 --warmup 2
#   rocprofv3 --pmc FETCH_SIZE       -f csv -d DIR/<leg>/fetch -o fetch -- python3 bench.py --only <leg>,copy --steps 5 --warmup 2
#   rocprofv3 --pmc WRITE_SIZE       -f csv -d DIR/<leg>/write -o write -- python3 bench.py --only <leg>,copy --steps 5 --warmup 2
# and optionally DIR/<leg>/mfma (--pmc MfmaUtil MfmaFlopsBF16) and DIR/<leg>/insts (--pmc with the
# INSTS_COUNTERS below: instructions issued per wave, and the share of wave cycles spent waiting to
# issue LDS instructions) and DIR/<leg>/stall (--pmc with the STALL_COUNTERS: where the waves' cycles
# go).  The copy leg runs a 256 MiB
# device copy in the same process: its FETCH_SIZE / WRITE_SIZE (KiB) against the 268,435,456 bytes
# it reads and writes give the scale factors applied to every kernel of the leg.
def _short_kernel(name):
    name = name.replace("void ", "")
    m = re.match(r"(kda::[a-z_]+(?:<[^>]*>)?|__amd_rocclr_copyBuffer)", name)
    return m.group(1) if m else name[:60]


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def _counters(path):
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = _short_kernel(r["Kernel_Name"])
            if name.startswith("kda::") or name == "__amd_rocclr_copyBuffer":
                per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return per


PROFILE_STEPS = "--steps 5 --warmup 2"
INSTS_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM SQ_WAIT_INST_LDS "
                  "SQ_WAVE_CYCLES")
STALL_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
                  "SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA")


def summarize_profiles(top, cmd_prefix="rocprofv3"):
    import csv
    copy_name, nb = "__amd_rocclr_copyBuffer", 1 << 28
    table = {"source_hash": kernel_source_hash(), "workloads": {}}
    for leg in sorted(os.listdir(top)):
        d = os.path.join(top, leg)
        if not os.path.isdir(d):
            continue
        entry = {"kernels": {}, "mfma": {}, "kernel_avg_us": {}}
        md = [f"# rocprofv3 summary: bench leg `{leg}`", "",
              f"Commands (run from /tmp on one MI355X with TMPDIR=/tmp; `<repo>` is this repository):", "", "```",
              f"{cmd_prefix} --kernel-trace --stats -f csv -d <out>/{leg}/trace -o trace -- python3 <repo>/bench.py --only {leg},copy {PROFILE_STEPS}",
              f"{cmd_prefix} --pmc FETCH_SIZE -f csv -d <out>/{leg}/fetch -o fetch -- python3 <repo>/bench.py --only {leg},copy {PROFILE_STEPS}",
              f"{cmd_prefix} --pmc WRITE_SIZE -f csv -d <out>/{leg}/write -o write -- python3 <repo>/bench.py --only {leg},copy {PROFILE_STEPS}",
              f"{cmd_prefix} --pmc MfmaUtil MfmaFlopsBF16 -f csv -d <out>/{leg}/mfma -o mfma -- python3 <repo>/bench.py --only {leg} {PROFILE_STEPS}   (prefill, long, varlen)",
              f"{cmd_prefix} --pmc {INSTS_COUNTERS} -f csv -d <out>/{leg}/insts -o insts -- python3 <repo>/bench.py --only {leg} {PROFILE_STEPS}   (prefill, long, varlen)",
              f"{cmd_prefix} --pmc {STALL_COUNTERS} -f csv -d <out>/{leg}/stall -o stall -- python3 <repo>/bench.py --only {leg} {PROFILE_STEPS}   (prefill, long, varlen)",
              f"python3 <repo>/bench.py --summarize <out>", "```", ""]
        stats = _find_csv(os.path.join(d, "trace"), "kernel_stats.csv")
        if stats:
            md += ["Kernel durations (`kernel_stats.csv`; torch's input-generation kernels omitted):", "",
                   "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
            with open(stats) as fh:
                for r in csv.DictReader(fh):
                    k = _short_kernel(r["Name"])
                    if k.startswith("kda::") or k == copy_name:
                        avg = float(r["AverageNs"]) / 1e3
                        entry["kernel_avg_us"][k] = avg
                        md.append(f"| `{k}` | {r['Calls']} | {avg:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                                  f"{float(r['MaxNs']) / 1e3:.1f} |")
            md.append("")
        fpath, wpath = _find_csv(os.path.join(d, "fetch"), "counter_collection.csv"), \
            _find_csv(os.path.join(d, "write"), "counter_collection.csv")
        if fpath and wpath:
            fe, wr = _counters(fpath), _counters(wpath)
            fcal, wcal = max(fe[copy_name]["FETCH_SIZE"]), max(wr[copy_name]["WRITE_SIZE"])
            fs, ws = nb / (fcal * 1024), nb / (wcal * 1024)
            entry.update(fetch_scale=fs, write_scale=ws)
            md += [f"HBM traffic per launch: FETCH_SIZE x {fs:.3f} + WRITE_SIZE x {ws:.3f} (the 256 MiB runtime copy of "
                   f"the same run reads {fcal:.0f} KiB by FETCH_SIZE and writes {wcal:.0f} KiB by WRITE_SIZE).", "",
                   "| kernel | launches | read (MB) | written (MB) | total (MB) |", "|---|---|---|---|---|"]
            for k in sorted(set(fe) & set(wr)):
                f, w = fe[k].get("FETCH_SIZE"), wr[k].get("WRITE_SIZE")
                if not f or not w:
                    continue
                if k == copy_name:
                    f = [x for x in f if x > 0.99 * fcal]
                    w = [x for x in w if x > 0.99 * wcal]
                rd, wt = sum(f) / len(f) * 1024 * fs, sum(w) / len(w) * 1024 * ws
                entry["kernels"][k] = {"bytes_read": rd, "bytes_written": wt, "bytes_per_launch": rd + wt,
                                       "launches": len(f)}
                md.append(f"| `{k}` | {len(f)} | {rd / 1e6:.1f} | {wt / 1e6:.1f} | {(rd + wt) / 1e6:.1f} |")
            md.append("")
        mpath = _find_csv(os.path.join(d, "mfma"), "counter_collection.csv")
        if mpath:
            mf = _counters(mpath)
            md += ["MFMA counters (MfmaUtil %, issued bf16 MFMA flops per launch):", "",
                   "| kernel | launches | MfmaUtil (%) | MfmaFlopsBF16 (GFLOP) |", "|---|---|---|---|"]
            for k, c in sorted(mf.items()):
                u, fl = c.get("MfmaUtil"), c.get("MfmaFlopsBF16")
                if u and fl:
                    entry["mfma"][k] = {"util_pct": sum(u) / len(u), "bf16_flops_issued": sum(fl) / len(fl)}
                    md.append(f"| `{k}` | {len(u)} | {sum(u) / len(u):.1f} | {sum(fl) / len(fl) / 1e9:.2f} |")
            md.append("")
        ipath = _find_csv(os.path.join(d, "insts"), "counter_collection.csv")
        if ipath:
            ic = _counters(ipath)
            md += ["Instructions issued per wave (SQ_INSTS_* / SQ_WAVES, averaged over launches) and the share of "
                   "wave cycles spent waiting to issue an LDS instruction (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES, both in "
                   "units of 4 cycles):", "",
                   "| kernel | launches | waves | VALU | MFMA | LDS | SALU | VMEM | LDS issue wait (%) |",
                   "|---|---|---|---|---|---|---|---|---|"]
            entry["insts"] = {}
            for k, c in sorted(ic.items()):
                if k == copy_name or not c.get("SQ_WAVES"):
                    continue
                mean = {n: sum(v) / len(v) for n, v in c.items()}
                w = mean["SQ_WAVES"]
                per = {n: mean.get(f"SQ_INSTS_{n}", 0.0) / w for n in ("VALU", "MFMA", "LDS", "SALU", "VMEM")}
                wait = 100.0 * mean.get("SQ_WAIT_INST_LDS", 0.0) / max(mean.get("SQ_WAVE_CYCLES", 0.0), 1.0)
                entry["insts"][k] = dict(waves=w, lds_issue_wait_pct=wait, **{f"{n.lower()}_per_wave": x for n, x in per.items()})
                md.append(f"| `{k}` | {len(c['SQ_WAVES'])} | {w:.0f} | {per['VALU']:.0f} | {per['MFMA']:.0f} | "
                          f"{per['LDS']:.0f} | {per['SALU']:.0f} | {per['VMEM']:.0f} | {wait:.1f} |")
            md.append("")
        spath = _find_csv(os.path.join(d, "stall"), "counter_collection.csv")
        if spath:
            sc = _counters(spath)
            md += ["Where the waves' cycles go, as shares of SQ_WAVE_CYCLES (the cycles waves are resident; "
                   "the wait counters count in the same 4-cycle units; the ACTIVE_INST counters are taken as "
                   "reported, so their shares are indicative): waiting for anything (dependencies, "
                   "`s_waitcnt`, barriers), waiting to issue, and working on any, vector ALU, vector memory, "
                   "LDS and scalar instructions:", "",
                   "| kernel | launches | wait any (%) | wait issue (%) | active any (%) | VALU (%) | VMEM (%) | LDS (%) | scalar (%) |",
                   "|---|---|---|---|---|---|---|---|---|"]
            entry["stall"] = {}
            for k, c in sorted(sc.items()):
                if k == copy_name or not c.get("SQ_WAVE_CYCLES"):
                    continue
                mean = {n: sum(v) / len(v) for n, v in c.items()}
                wc = max(mean["SQ_WAVE_CYCLES"], 1.0)
                sh = {n: 100.0 * mean.get(n, 0.0) / wc for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                                                                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VMEM",
                                                                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA")}
                entry["stall"][k] = {n.replace("SQ_", "").lower() + "_pct": x for n, x in sh.items()}
                md.append(f"| `{k}` | {len(c['SQ_WAVE_CYCLES'])} | {sh['SQ_WAIT_ANY']:.1f} | {sh['SQ_WAIT_INST_ANY']:.1f} | "
                          f"{sh['SQ_ACTIVE_INST_ANY']:.1f} | {sh['SQ_ACTIVE_INST_VALU']:.1f} | {sh['SQ_ACTIVE_INST_VMEM']:.1f} | "
                          f"{sh['SQ_ACTIVE_INST_LDS']:.1f} | {sh['SQ_ACTIVE_INST_SCA']:.1f} |")
            md.append("")
        table["workloads"][leg] = entry
        with open(os.path.join(ROOT, "profiles", f"kda_{leg}_rocprof_summary.md"), "w") as fh:
            fh.write("\n".join(md))
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(table, fh, indent=1)
    return table


def roofline_block(leg, th, ms_whole, kernels):
    """Roofline figures of one prefill leg: the dominant kernel by the survey's algorithmic bytes
    per token-head (1,540 B: q, k, v bf16, g fp32, beta, o bf16) over its own duration, the whole
    prefill by the same bytes over the whole call, and each kernel's measured traffic."""
    alg = PREFILL_BYTES * th
    dom = max(kernels, key=lambda k: kernels[k][1])
    dom_name, dom_ms = kernels[dom]
    r = {"bound": "hbm", "kernel": dom_name, "algorithmic_bytes_per_launch": alg,
         "achieved": alg / (dom_ms / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = measured_traffic(leg, dom_name)
    r["ms_per_launch"] = dom_ms
    whole = {"bound": "hbm", "algorithmic_bytes": alg, "ms": ms_whole, "achieved": alg / (ms_whole / 1e3) / 1e9,
             "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    whole["frac"] = whole["achieved"] / HBM_PEAK_GBS
    tr = {k: measured_traffic(leg, name) for k, (name, _) in kernels.items()}
    whole["traffic"] = None if any(v is None for v in tr.values()) else sum(tr.values())
    per_kernel = {k: {"kernel": name, "ms": ms, "traffic": tr[k], "mfma": measured_mfma(leg, name),
                      "insts_per_wave": measured_insts(leg, name)}
                  for k, (name, ms) in kernels.items()}
    return r, whole, per_kernel


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="write profiles/traffic.json and profiles/kda_<leg>_rocprof_summary.md from rocprofv3 "
                         "csv output under DIR/<leg>/{trace,fetch,write,mfma,insts,stall} (no GPU needed)")
    ap.add_argument("--only", default="prefill,decode,prep,scalar,gate,attnres,long,kcp,varlen,cpu",
                    help="comma list of prefill, decode, prep, scalar, gate, attnres, long, kcp, varlen, cpu, "
                         "copy")
    args = ap.parse_args()
    if args.summarize:
        t = summarize_profiles(args.summarize)
        print(json.dumps({k: list(v["kernels"]) for k, v in t["workloads"].items()}))
        return
    only = set(x.strip() for x in args.only.split(",") if x.strip())
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operator shards by head and sequence with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_delta_rule_93_amd as kda
    dev = torch.device("cuda:0")
    kda.lib()

    def long_block(lc):
        th = 131072 * 32
        r, whole, per = roofline_block("long", th, lc["ms"], {
            "chunk_local": (K_LOCAL, lc["ms_chunk_local"]), "state_scan": (K_SCAN_1T, lc["ms_state_scan"])})
        lc.update(roofline=r, roofline_whole=whole, kernels=per)
        return lc

    def varlen_block(vl):
        r, whole, per = roofline_block("varlen", vl["token_heads"], vl["ms_fwd"], {
            "chunk_local": (K_LOCAL, vl["ms_chunk_local"]), "state_scan": (K_SCAN_2T, vl["ms_state_scan"])})
        vl.update(roofline=r, roofline_whole=whole, kernels=per)
        return vl

    if "prefill" not in only:  # single legs (profiling runs)
        out = {}
        if "decode" in only:
            out["decode"] = bench_decode(args, torch, kda, dev)
        if "prep" in only:
            out["prep"] = bench_prep(args, torch, kda, dev)
        if "scalar" in only:
            out["scalar_gate"] = bench_scalar_gate(torch, kda, dev)
        if "gate" in only:
            out["lowrank_gate"] = bench_lowrank_gate(torch, kda, dev)
        if "attnres" in only:
            out["attnres"] = bench_attnres(torch, kda, dev)
        if "long" in only:
            out["long_context"] = long_block(bench_long(torch, kda, dev))
        if "kcp" in only:
            out["segment_maps"] = bench_kcp(torch, kda, dev)
        if "varlen" in only:
            out["varlen_layer"] = varlen_block(bench_varlen_layer(torch, kda, dev))
        if "copy" in only:
            out["copy"] = bench_copy(torch, dev)
        if "cpu" in only:
            import kda_inputs as ki
            out["cpu_baseline"] = cpu_baseline(ki.prefill_batch())
        print(json.dumps(out), flush=True)
        return
    log("prefill ...")
    pf, inp = bench_prefill(args, torch, kda, dev)
    token_heads = pf["token_heads"]
    value = pf["tokens"] / (pf["ms_step"] / 1e3)
    flops = PREFILL_FLOP * token_heads
    roof, whole, per = roofline_block("prefill", token_heads, pf["ms_step"], {
        "chunk_local": (K_LOCAL, pf["ms_chunk_local"]), "state_scan": (K_SCAN_2T, pf["ms_state_scan"])})
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": pf["ms_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "KDA chunked prefill B=4 H=16 T=4096 d_k=d_v=128 chunk=64, bf16 q/k/v, "
                               "fp32 log-decay/beta/state", "global_batch": 4, "seq_len": 4096, "heads": 16,
                   "head_dim": 128, "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_whole_prefill": whole,
        "prefill": {"ms_fwd": pf["ms_fwd_events"], "ms_chunk_local": pf["ms_chunk_local"],
                    "ms_state_scan": pf["ms_state_scan"], "kernels": per,
                    "algorithmic_GBs": PREFILL_BYTES * token_heads / pf["ms_fwd_events"] / 1e6,
                    "algorithmic_TFLOPs": flops / pf["ms_fwd_events"] / 1e9,
                    "mfma_frac_of_bf16_peak": flops / pf["ms_fwd_events"] / 1e9 / BF16_PEAK_TFLOPS,
                    "workspace_bytes_per_chunk_head": pf["ws_bytes_per_chunk_head"],
                    "untimed_settle_steps": pf["settle_steps"]},
    }
    if "decode" in only:
        log("decode ...")
        dc = bench_decode(args, torch, kda, dev)
        out["decode"] = {"workload": "256 sequences x 32 heads, d=128, fp32 state, bf16 tokens, 100 steps",
                         "ms_per_step": dc["ms_step"], "state_GBs": dc["state_gbs"], "total_GBs": dc["total_gbs"],
                         "roofline": {"bound": "hbm", "kernel": K_DECODE, "achieved": dc["total_gbs"],
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": dc["total_gbs"] / HBM_PEAK_GBS,
                                      "traffic": measured_traffic("decode", K_DECODE),
                                      "algorithmic_bytes_per_launch": dc["state_bytes"] + dc["io_bytes"]}}
        cp = bench_copy(torch, dev)
        out["decode"]["copy_same_run"] = {"what": "runtime device copy of 256 MiB (read + write)",
                                          "GBs": cp["GBs"], "decode_over_copy": dc["total_gbs"] / cp["GBs"]}
    if "prep" in only:
        log("prep ...")
        pr = bench_prep(args, torch, kda, dev)
        out["prep"] = {"workload": f"{pr['tokens']} packed tokens (64 sequences), H=32, d=128, width 4, bf16",
                       "ms": pr["ms"], "GBs": pr["gbs"], "frac": pr["gbs"] / HBM_PEAK_GBS,
                       "roofline": {"bound": "hbm", "kernel": K_PREP, "achieved": pr["gbs"], "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": pr["gbs"] / HBM_PEAK_GBS,
                                    "algorithmic_bytes_per_launch": pr["bytes"],
                                    "traffic": measured_traffic("prep", K_PREP)}}
    if "scalar" in only:
        log("scalar gate ...")
        out["scalar_gate"] = bench_scalar_gate(torch, kda, dev)
    if "gate" in only:
        log("low-rank gate ...")
        out["lowrank_gate"] = bench_lowrank_gate(torch, kda, dev)
    if "attnres" in only:
        log("block attnres ...")
        out["attnres"] = bench_attnres(torch, kda, dev)
    if "long" in only:
        log("long context ...")
        out["long_context"] = long_block(bench_long(torch, kda, dev))
    if "kcp" in only:
        log("segment maps ...")
        out["segment_maps"] = bench_kcp(torch, kda, dev)
    if "varlen" in only:
        log("varlen layer ...")
        out["varlen_layer"] = varlen_block(bench_varlen_layer(torch, kda, dev))
    if "copy" in only:
        out["copy"] = bench_copy(torch, dev)
    if "cpu" in only:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
