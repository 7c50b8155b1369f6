// kda_attnres.hip -- Block AttnRes read-out over stored block outputs (bf16 hidden states).
//
// For one layer with query w (blog post-114, chapter 6, the block AttnRes listing; page "Kimi K3
// 注意力三件套", AttnRes section):  h[t] = sum_n softmax_n(w . norm(V_n[t])) V_n[t], where norm is an
// RMS norm over the hidden width.  Two-phase inference (same page): for the L layers of a block
// the stored blocks are scored and mixed once for all layers (phase 1: per layer the
// softmax-weighted mean o and the log-sum-exp of the scores), then each layer merges its partial
// block with an online-softmax step (phase 2).
//
// Kernels
//   attnres_online_kernel  one wave per token: a single pass over the blocks with an online
//                          softmax (running max, rescaled sum); serves the one-shot read-out and,
//                          seeded with (o, lse), the phase-2 merge.
//   attnres_scores_kernel  phase 1a: the scores' dot products w_l . V_n[t] and sum V_n[t]^2 as one
//                          bf16 MFMA product over the width, rows = 16 tokens of one block, the
//                          operands staged in LDS as whole lines.
//   attnres_mix_kernel     phase 1b: per token, the softmax over the blocks for every layer and the
//                          weighted sums o_l = sum_n a_ln V_n (the blocks are read once for all L).
#include <utility>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ void unpack8(const u32x4 &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 pack8(const float *x) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)x[2 * i]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)x[2 * i + 1]);
        r[i] = lo | (hi << 16);
    }
    return r;
}

// Sum over the 64 lanes of a wave (butterfly; every lane ends with the same value, in the same
// order on every lane, so results are reproducible).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace

// ---------------------------------------------------------------- one-shot read-out / merge
// J = d / 512: lane l holds channels 512 j + 8 l .. + 7 of every row, j < J.
template <int J>
__global__ void __launch_bounds__(256) attnres_online_kernel(AttnResArgs a) {
    const int lane = threadIdx.x & 63;
    const long t = (long)blockIdx.x * 4 + wave_id();
    if (t >= a.T) return;  // whole wave
    const float inv_d = 1.f / (float)(512 * J);
    const long row = t * (512 * J) + 8 * lane;
    u32x4 wq[J], xb[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        wq[j] = *reinterpret_cast<const u32x4 *>(a.w + 512 * j + 8 * lane);
        xb[j] = *reinterpret_cast<const u32x4 *>(a.blk[0] + row + 512 * j);
    }
    float acc[J][8];
    float m = -INFINITY, s = 0.f;
    if (a.prior_o) {  // earlier blocks, summarised by their softmax-weighted mean and log-sum-exp
        m = a.prior_lse[t];
        s = 1.f;
#pragma unroll
        for (int j = 0; j < J; ++j) unpack8(*reinterpret_cast<const u32x4 *>(a.prior_o + row + 512 * j), acc[j]);
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
    }
    for (int b = 0; b < a.n; ++b) {
        float ss = 0.f, dw = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            float x[8], wf[8];
            unpack8(xb[j], x);
            unpack8(wq[j], wf);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ss += x[i] * x[i];
                dw += wf[i] * x[i];
            }
        }
        u32x4 xn[J];  // next block's row, in flight while this one is folded in
        const uint16_t *nb = a.blk[b + 1 < a.n ? b + 1 : b];
#pragma unroll
        for (int j = 0; j < J; ++j) xn[j] = *reinterpret_cast<const u32x4 *>(nb + row + 512 * j);
        ss = wave_sum(ss);
        dw = wave_sum(dw);
        const float l = dw / sqrtf(ss * inv_d + a.eps);  // w . (x / rms(x))
        const float mn = fmaxf(m, l);
        const float c = fast_exp2((m - mn) * kLog2e), p = fast_exp2((l - mn) * kLog2e);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            float x[8];
            unpack8(xb[j], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] * c + p * x[i];
            xb[j] = xn[j];
        }
        s = s * c + p;
        m = mn;
    }
    const float inv_s = 1.f / s;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = acc[j][i] * inv_s;
        *reinterpret_cast<u32x4 *>(a.h + row + 512 * j) = pack8(y);
    }
}

// ---------------------------------------------------------------- phase 1a: score dot products
// Workgroup (block b, 64 tokens), wave w: rows = the 16 tokens 16 w .., columns = layers (<= 16),
// k = width in blocks of 32 with lane (grp, r16) holding the 8 consecutive width indices
// 32 kb + 8 grp .. (A and B alike).  A second MFMA of the tile with itself gives sum x^2 of each
// token row on its diagonal.  The operands reach the MFMAs through LDS, 256 widths per step: a
// wave loads its 16 token rows, and the four waves together the 16 query rows (rows past L read
// row 0 and are zeroed), as whole 128-byte lines (half a wave per 512-byte row segment); loaded
// directly in the fragment layout every load held 16 rows x 64 bytes and the kernel waited on
// issuing its loads.  The next step's loads are in flight while the current one is multiplied.
constexpr int kScoreStep = 256;                  // widths per step
constexpr int kScoreRow = kScoreStep + 8;        // LDS row (bf16), padded against bank conflicts
__global__ void __launch_bounds__(256) attnres_scores_kernel(AttnScoreArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[4][16][kScoreRow];
    __shared__ __attribute__((aligned(16))) uint16_t ws[16][kScoreRow];
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    const int b = blockIdx.y;
    const long t0 = ((long)blockIdx.x * 4 + wave) * 16;
    // load j (< 8) of this wave: token row 2 j + (lane >> 5); query load j (< 2): row 4 wave + 2 j +
    // (lane >> 5); lane & 31 picks the 16-byte piece of the row's 512-byte step.  Rows past the
    // end are read from a valid row (tokens: the last one; queries: row 0, then zeroed).
    const int half = lane >> 5, piece = 8 * (lane & 31);
    const uint16_t *xl[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const long t = t0 + 2 * j + half;
        xl[j] = a.blk[b] + (t < a.T ? t : a.T - 1) * a.d + piece;
    }
    const uint16_t *wl[2];
    bool wok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 4 * wave + 2 * j + half;
        wok[j] = row < a.L;
        wl[j] = a.W + (long)(wok[j] ? row : 0) * a.d + piece;
    }
    const int nsteps = a.d / kScoreStep;
    auto issue = [&](int st, u32x4 (&xr)[8], u32x4 (&wr)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) xr[j] = *reinterpret_cast<const u32x4 *>(xl[j] + (long)kScoreStep * st);
#pragma unroll
        for (int j = 0; j < 2; ++j) wr[j] = *reinterpret_cast<const u32x4 *>(wl[j] + (long)kScoreStep * st);
    };
    f32x4 dots = zero4(), sq = zero4();
    // one step: the registers to LDS, the next step's loads issued, then the 16 MFMAs from LDS
    auto step = [&](int st, u32x4 (&xr)[8], u32x4 (&wr)[2], u32x4 (&xn)[8], u32x4 (&wn)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(&xs[wave][2 * j + half][piece]) = xr[j];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<u32x4 *>(&ws[4 * wave + 2 * j + half][piece]) = wok[j] ? wr[j] : u32x4{0u, 0u, 0u, 0u};
        if (st + 1 < nsteps) issue(st + 1, xn, wn);
        __syncthreads();  // the step's query rows (written by all four waves) are in LDS
#pragma unroll
        for (int kb = 0; kb < kScoreStep / 32; ++kb) {
            const FragB xa{__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&xs[wave][r16][32 * kb + 8 * grp]))};
            const FragB wb{__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ws[r16][32 * kb + 8 * grp]))};
            dots = mfma(xa, wb, dots);
            sq = mfma(xa, xa, sq);
        }
        __syncthreads();  // every wave is done with the step's rows before they are overwritten
    };
    u32x4 xA[8], wA[2], xB[8], wB[2];
    issue(0, xA, wA);
    for (int st = 0; st < nsteps; st += 2) {  // nsteps is even (d is a multiple of 512)
        step(st, xA, wA, xB, wB);
        step(st + 1, xB, wB, xA, wA);
    }
    // lane (grp, r16) holds rows 4 grp + e, column r16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const long t = t0 + 4 * grp + e;
        if (t >= a.T) continue;
        if (r16 < a.L) a.dots[((long)b * a.T + t) * 16 + r16] = dots[e];
        if (r16 == 4 * grp + e) a.sumsq[(long)b * a.T + t] = sq[e];
    }
}

// ---------------------------------------------------------------- phase 1b: softmax and mix
// One wave per token; NB = number of blocks.  Lane l < L forms layer l's softmax over the blocks
// and its log-sum-exp; the weights go through LDS to every lane, which then mixes its 8-channel
// slices of the blocks (loaded once per slice) for the layers, four at a time.
template <int NB>
__global__ void __launch_bounds__(256) attnres_mix_kernel(AttnMixArgs a) {
    __shared__ float wts[4][kAttnResMaxLayers][NB];  // [wave][layer][block]
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const long t = (long)blockIdx.x * 4 + wave;
    if (t >= a.T) return;  // whole wave; no workgroup barrier below
    const float inv_d = 1.f / (float)a.d;
    if (lane < a.L) {
        float lg[NB];
        float m = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float ssq = a.sumsq[(long)b * a.T + t];
            lg[b] = a.dots[((long)b * a.T + t) * 16 + lane] / sqrtf(ssq * inv_d + a.eps);
            m = fmaxf(m, lg[b]);
        }
        float sum = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            lg[b] = fast_exp2((lg[b] - m) * kLog2e);
            sum += lg[b];
        }
        const float inv = 1.f / sum;
#pragma unroll
        for (int b = 0; b < NB; ++b) wts[wave][lane][b] = lg[b] * inv;
        if (a.lse) a.lse[(long)lane * a.T + t] = m + __builtin_amdgcn_logf(sum) * kLn2;
    } else if (lane < kAttnResMaxLayers) {  // layers past L: zero weights (read, never stored)
#pragma unroll
        for (int b = 0; b < NB; ++b) wts[wave][lane][b] = 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int J = a.d / 512;
    for (int j = 0; j < J; ++j) {
        const long off = t * a.d + 512 * j + 8 * lane;
        u32x4 xb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) xb[b] = *reinterpret_cast<const u32x4 *>(a.blk[b] + off);
        for (int l0 = 0; l0 < a.L; l0 += 4) {
            float acc[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float x[8];
                unpack8(xb[b], x);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float wl = wts[wave][(l0 + u) & (kAttnResMaxLayers - 1)][b];  // l0 + u < 16
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[u][i] += wl * x[i];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (l0 + u < a.L) *reinterpret_cast<u32x4 *>(a.o + (long)(l0 + u) * a.T * a.d + off) = pack8(acc[u]);
        }
    }
}

hipError_t launch_attnres(const AttnResArgs &a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.T + 3) / 4)), block(256);
    switch (a.d / 512) {
        case 1: return launch_kernel(attnres_online_kernel<1>, grid, block, st, a);
        case 2: return launch_kernel(attnres_online_kernel<2>, grid, block, st, a);
        case 3: return launch_kernel(attnres_online_kernel<3>, grid, block, st, a);
        case 4: return launch_kernel(attnres_online_kernel<4>, grid, block, st, a);
        case 5: return launch_kernel(attnres_online_kernel<5>, grid, block, st, a);
        case 6: return launch_kernel(attnres_online_kernel<6>, grid, block, st, a);
        case 7: return launch_kernel(attnres_online_kernel<7>, grid, block, st, a);
        case 8: return launch_kernel(attnres_online_kernel<8>, grid, block, st, a);
        default: return hipErrorInvalidValue;
    }
}

template <int NB>
static hipError_t launch_mix(const AttnMixArgs &m, hipStream_t st) {
    return launch_kernel(attnres_mix_kernel<NB>, dim3((unsigned)((m.T + 3) / 4)), dim3(256), st, m);
}

// The mix kernel instance for m.n blocks; hipErrorInvalidValue when m.n is out of range.
template <int... NBs>
static hipError_t launch_mix_n(const AttnMixArgs &m, hipStream_t st, std::integer_sequence<int, NBs...>) {
    hipError_t e = hipErrorInvalidValue;
    ((void)(m.n == NBs + 1 && ((e = launch_mix<NBs + 1>(m, st)), true)), ...);
    return e;
}

hipError_t launch_attnres_inter(const AttnScoreArgs &s, const AttnMixArgs &m, hipStream_t st) {
    if (s.T <= 0) return hipSuccess;
    const hipError_t e =
        launch_kernel(attnres_scores_kernel, dim3((unsigned)((s.T + 63) / 64), (unsigned)s.n), dim3(256), st, s);
    if (e != hipSuccess) return e;
    return launch_mix_n(m, st, std::make_integer_sequence<int, kAttnResMaxBlocks>{});
}

}  // namespace kda
