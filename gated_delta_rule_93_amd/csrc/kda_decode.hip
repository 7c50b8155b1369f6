// kda_decode.hip -- single-token KDA update with the state resident in HBM.
//
// Per (sequence n, head h), in place (course page "线性注意力与 KDA", section 3 update;
// section 2 read-out):
//   alpha = exp(g);  S~ = Diag(alpha) S
//   p = S~^T k;  r = S~^T q;  u = beta (v - p)
//   S <- S~ + k u^T;   o = scale (S_new^T q) = scale (r + (q . k) u)
// The last identity lets one pass over the state produce both the update and the read-out:
// the state is read once and written once (2 * d_k * d_v * 4 bytes per head and step).
//
// Mapping: one workgroup of NT = DK * DV / 16 threads per (n, h) (1024 at d = 128), so every
// thread holds four 16-byte pieces of the state.  Thread t owns value columns 4 * (t % (DV/4))
// .. +3 and key rows i = t / (DV/4) + RG * m (m = 0 .. 3), where RG = NT / (DV/4) row groups.
// A wave reads whole 16-byte column quads of consecutive rows, so every state access is a fully
// coalesced dwordx4.  The column reductions p and r are a per-thread partial sum over its rows
// followed by a fixed-order LDS reduction across the RG row groups (deterministic).  Measured on
// the 256 x 32-head, d = 128 step: 16 rows per thread (256 threads) ran at 5.5 TB/s, 8 rows at
// 5.5, 4 rows (1024 threads) at 5.8: each head's state then arrives with more requests in flight.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV> constexpr int decode_threads() { return DK * DV / 16; }

template <typename TIO, int DK, int DV>
__global__ void __launch_bounds__((decode_threads<DK, DV>()))
decode_step_kernel(const TIO *__restrict__ q, const TIO *__restrict__ k, const TIO *__restrict__ v,
                   const float *__restrict__ g, const float *__restrict__ beta, float scale,
                   float *__restrict__ state, TIO *__restrict__ o) {
    constexpr int NT = decode_threads<DK, DV>();
    constexpr int TPR = DV / 4;          // threads per state row (one float4 each)
    constexpr int RG = NT / TPR;         // row groups
    constexpr int RPT = DK / RG;         // rows per thread (4)
    static_assert(RG * TPR == NT && RPT * RG == DK && NT <= 1024 && NT >= kWave, "tile");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f32x4 s_p[RG][TPR], s_r[RG][TPR];
    __shared__ float s_qk;

    const long head = blockIdx.x;  // n * H + h
    const int t = threadIdx.x;
    const int cq = t % TPR;
    const int rg = t / TPR;

    float *S = state + head * (long)(DK * DV);
    // issue the state loads first: RPT independent 16-byte loads per thread
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (long)i * DV) + cq);
    }
    for (int i = t; i < DK; i += NT) {
        s_k[i] = IO<TIO>::load(k, head * DK + i);
        s_q[i] = IO<TIO>::load(q, head * DK + i);
        s_a[i] = __expf(g[head * DK + i]);
    }
    __syncthreads();
    if (t < kWave) {  // q . k, fixed-order wave reduction
        float acc = 0.f;
        for (int i = t; i < DK; i += kWave) acc += s_q[i] * s_k[i];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (t == 0) s_qk = acc;
    }
    f32x4 p = zero4(), r = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const float a = s_a[i];
        s[m] *= a;                       // S~ rows
        p += s[m] * s_k[i];
        r += s[m] * s_q[i];
    }
    s_p[rg][cq] = p;
    s_r[rg][cq] = r;
    __syncthreads();
    f32x4 pt = s_p[0][cq], rt = s_r[0][cq];
#pragma unroll
    for (int j = 1; j < RG; ++j) {
        pt += s_p[j][cq];
        rt += s_r[j][cq];
    }
    const float b = beta[head];
    const f32x4 vv = load4(v + head * DV + 4 * cq);
    const f32x4 u = b * (vv - pt);
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const f32x4 sn = s[m] + s_k[i] * u;
        __builtin_nontemporal_store(sn, reinterpret_cast<f32x4 *>(S + (long)i * DV) + cq);
    }
    if (rg == 0) {
        const f32x4 ov = scale * (rt + s_qk * u);
        const long ob = head * DV + 4 * cq;
        IO<TIO>::store(o, ob + 0, ov.x);
        IO<TIO>::store(o, ob + 1, ov.y);
        IO<TIO>::store(o, ob + 2, ov.z);
        IO<TIO>::store(o, ob + 3, ov.w);
    }
}

template <typename TIO, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st) {
    const long heads = (long)a.N * a.H;
    return launch_kernel(decode_step_kernel<TIO, DK, DV>, dim3((unsigned)heads), dim3(decode_threads<DK, DV>()), st,
                         a.q, a.k, a.v, a.g, a.beta, a.scale, a.state, a.o);
}

template <typename TIO>
static hipError_t launch_decode_io(const DecodeArgs &a, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) return launch_decode_t<TIO, 128, 128>(a, st);
    if (a.dk == 64 && a.dv == 64) return launch_decode_t<TIO, 64, 64>(a, st);
    if (a.dk == 128 && a.dv == 64) return launch_decode_t<TIO, 128, 64>(a, st);
    return launch_decode_t<TIO, 64, 128>(a, st);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
    return a.bf16 ? launch_decode_io<uint16_t>(a, st) : launch_decode_io<float>(a, st);
}

}  // namespace kda
