// kda_prep.hip -- q/k prologue: short causal depthwise conv -> SiLU -> L2 norm per head.
//
// Page "Kimi K3 注意力三件套" (yeyulingfeng.com), KDA section: q and k pass a short causal
// convolution (a local sliding window) and are then L2-normalised, which bounds the write
// magnitude; blog post-114, chapter 3: normalize(silu(.)) in the DeltaNet code.
//   c'_t[c] = sum_{tau=0}^{W-1} w[c, tau] x_{t-(W-1)+tau}[c]   (zero before the sequence start)
//   y_t     = silu(c'_t) / max(||silu(c'_t)||_2 over the head's d channels, 1e-12)
//
// HBM-bound stencil.  Each thread owns 8 consecutive channels (one 16-byte bf16 vector) of one
// head and walks TT consecutive tokens, keeping the W-1 previous inputs in registers, so the
// input is read once plus a (W-1)/TT halo.  The rows of the next kPrepPF tokens are always in
// flight (a ring of raw 16-byte vectors): with one row per wave in flight the kernel was bound
// by load latency.  The d/8 lanes of a head reduce the sum of squares
// with xor shuffles inside their aligned lane group (fixed order, deterministic).  SiLU and the
// norm use the hardware reciprocal and reciprocal square root (about 1 ulp each): the division
// and square root of IEEE fp32 made the kernel issue-bound at 3.7 TB/s.  The taps are scaled by
// log2(e) once, so the convolution yields c log2(e) and SiLU's exponential needs no multiply: the
// factor log2(e) it leaves on silu(c) cancels in the L2 norm (the 1e-12 floor is scaled with it).
// Heads past H (the last workgroup's spare lanes) compute on head 0's rows and store nothing.
// bf16 rows are read and written with non-temporal accesses (each byte is touched once here).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr int kPrepTT = 64;
constexpr int kPrepPF = 4;  // token rows in flight per thread
static_assert(kPrepTT % kPrepPF == 0, "whole prefetch groups per block");

template <typename TIO> struct Vec8;
template <> struct Vec8<uint16_t> {
    typedef __attribute__((ext_vector_type(4))) unsigned int Raw;
    static __device__ __forceinline__ Raw load_raw(const uint16_t *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw *>(p));
    }
    static __device__ __forceinline__ void unpack(const Raw &w, float *x) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t *p, const float *x) {
        Raw w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        w.z = pack_bf16x2(x[4], x[5]);
        w.w = pack_bf16x2(x[6], x[7]);
        __builtin_nontemporal_store(w, reinterpret_cast<Raw *>(p));
    }
};
template <> struct Vec8<float> {
    struct Raw { f32x4 a, b; };
    static __device__ __forceinline__ Raw load_raw(const float *p) {
        return Raw{reinterpret_cast<const f32x4 *>(p)[0], reinterpret_cast<const f32x4 *>(p)[1]};
    }
    static __device__ __forceinline__ void unpack(const Raw &w, float *x) {
        x[0] = w.a.x; x[1] = w.a.y; x[2] = w.a.z; x[3] = w.a.w;
        x[4] = w.b.x; x[5] = w.b.y; x[6] = w.b.z; x[7] = w.b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *x) {
        reinterpret_cast<f32x4 *>(p)[0] = f32x4{x[0], x[1], x[2], x[3]};
        reinterpret_cast<f32x4 *>(p)[1] = f32x4{x[4], x[5], x[6], x[7]};
    }
};

// Largest n in [0, N) with cu[n] <= t (cu non-decreasing, cu[0] = 0 <= t).
__device__ __forceinline__ int find_seq(const int32_t *cu, int N, long t) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <typename TIO, int D, int W>
__global__ void __launch_bounds__(256)
prep_kernel(const TIO *__restrict__ x, const float *__restrict__ w, TIO *__restrict__ y,
            const int32_t *__restrict__ cu, int N, int T, long ntok, int H) {
    constexpr int LPH = D / 8;              // lanes per head
    constexpr int HPB = 256 / LPH;          // heads per block
    const int lane_in_head = threadIdx.x % LPH;
    const int h = blockIdx.y * HPB + threadIdx.x / LPH;
    const bool active = h < H;
    const int hh = active ? h : 0;
    const long t0 = (long)blockIdx.x * kPrepTT;
    const long t1 = min(t0 + kPrepTT, ntok);
    const long row = (long)H * D;           // elements per token
    const int c0 = hh * D + lane_in_head * 8;  // first channel of this thread

    float wt[8][W];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int tau = 0; tau < W; ++tau) wt[j][tau] = w[(long)(c0 + j) * W + tau] * kLog2e;

    // sequence containing t0 and its end
    long seq_start, seq_end;
    int n = 0;
    if (cu) {
        n = find_seq(cu, N, t0);
        seq_start = cu[n];
        seq_end = cu[n + 1];
    } else {
        seq_start = (t0 / T) * T;
        seq_end = seq_start + T;
    }
    // history: hist[m] holds token t - (W-1) + m for the next t.  Every load below reads a valid
    // row (tokens before 0 or past t1 - 1 are clamped into [0, t1 - 1] and the values then
    // replaced or never used; threads of a head past H read head 0), so all of them are issued
    // without branches and stay in flight together.
    using Raw = typename Vec8<TIO>::Raw;
    const TIO *xc0 = x + c0;
    float hist[W > 1 ? W - 1 : 1][8];
    {
        Raw hr[W > 1 ? W - 1 : 1];
#pragma unroll
        for (int m = 0; m < W - 1; ++m) {
            const long ts = t0 - (W - 1) + m;
            hr[m] = Vec8<TIO>::load_raw(xc0 + (ts >= 0 ? ts : t0) * row);
        }
#pragma unroll
        for (int m = 0; m < W - 1; ++m) {
            const long ts = t0 - (W - 1) + m;
            const bool live = active && ts >= seq_start;
            Vec8<TIO>::unpack(hr[m], hist[m]);
#pragma unroll
            for (int j = 0; j < 8; ++j) hist[m][j] = live ? hist[m][j] : 0.f;
        }
    }
    Raw pend[kPrepPF];  // pend[j]: the row of token tb + j of the current group
#pragma unroll
    for (int j = 0; j < kPrepPF; ++j) pend[j] = Vec8<TIO>::load_raw(xc0 + min(t0 + j, t1 - 1) * row);
    for (long tb = t0; tb < t1; tb += kPrepPF) {
#pragma unroll
        for (int j = 0; j < kPrepPF; ++j) {
            // tokens past t1 - 1 (only in a block's last group, for the last block) are computed
            // from clamped rows and not stored: no branch around the ring, whose registers then
            // stay fixed and are never copied while a load into them is in flight
            const long t = tb + j;
            float xc[8];
            Vec8<TIO>::unpack(pend[j], xc);
            pend[j] = Vec8<TIO>::load_raw(xc0 + min(t + kPrepPF, t1 - 1) * row);  // token t + kPrepPF
            while (t >= seq_end && (!cu || n + 1 < N)) {  // crossed into the next sequence: zero history
                if (cu) {
                    ++n;
                    seq_start = cu[n];
                    seq_end = cu[n + 1];
                } else {
                    seq_start = seq_end;
                    seq_end = seq_start + T;
                }
#pragma unroll
                for (int m = 0; m < W - 1; ++m)
#pragma unroll
                    for (int i = 0; i < 8; ++i) hist[m][i] = 0.f;
            }
            float yv[8];
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float c = wt[i][W - 1] * xc[i];
#pragma unroll
                for (int m = 0; m < W - 1; ++m) c = fmaf(wt[i][m], hist[m][i], c);
                const float s = c * __builtin_amdgcn_rcpf(1.f + fast_exp2(-c));
                yv[i] = s;
                ss = fmaf(s, s, ss);
            }
#pragma unroll
            for (int off = LPH / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
            const float inv = ss > 1e-24f * kLog2e * kLog2e ? __builtin_amdgcn_rsqf(ss) : 1e12f / kLog2e;
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] *= inv;
            if (active && t < t1) Vec8<TIO>::store(y + t * row + c0, yv);
#pragma unroll
            for (int m = 0; m + 1 < W - 1; ++m)
#pragma unroll
                for (int i = 0; i < 8; ++i) hist[m][i] = hist[m + 1][i];
            if (W > 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) hist[W > 1 ? W - 2 : 0][i] = xc[i];
            }
        }
    }
}

template <typename TIO, int D>
static hipError_t launch_prep_d(const PrepArgs &a, hipStream_t st) {
    constexpr int HPB = 256 / (D / 8);
    const long ntok = (long)a.B * a.T;
    dim3 grid((unsigned)((ntok + kPrepTT - 1) / kPrepTT), (unsigned)((a.H + HPB - 1) / HPB));
    const TIO *x = (const TIO *)a.x;
    TIO *y = (TIO *)a.y;
    switch (a.W) {
#define KDA_PREP_W(WW)                                                                                \
    case WW:                                                                                          \
        return launch_kernel(prep_kernel<TIO, D, WW>, grid, dim3(256), st, x, a.w, y, a.cu_seqlens, a.N, a.T, \
                             ntok, a.H);
        KDA_PREP_W(1) KDA_PREP_W(2) KDA_PREP_W(3) KDA_PREP_W(4)
        KDA_PREP_W(5) KDA_PREP_W(6) KDA_PREP_W(7) KDA_PREP_W(8)
#undef KDA_PREP_W
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t st) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    if (a.bf16) return a.d == 128 ? launch_prep_d<uint16_t, 128>(a, st) : launch_prep_d<uint16_t, 64>(a, st);
    return a.d == 128 ? launch_prep_d<float, 128>(a, st) : launch_prep_d<float, 64>(a, st);
}

}  // namespace kda
