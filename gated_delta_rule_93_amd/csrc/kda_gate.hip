// kda_gate.hip -- the gate prologue: the low-rank down projection z = x W_down^T (stored bf16),
// beta = sigmoid(x w_beta^T), and, when asked, log(alpha) = -softplus(z W_up^T + b) written out.
//
// The page "Kimi K3 注意力三件套" (KDA section) says alpha is produced by a low-rank down-up
// projection of the input and beta is one scalar; blog post-114, chapter 3 has beta as the
// sigmoid of a linear map of x and chapter 4 a gate per head and channel computed from x.
//
// One 512-thread workgroup per 64 tokens.  The down projection and the beta projection are one
// skinny bf16 MFMA product over the model width (x rows as A fragments, the stacked weight rows
// [W_down; w_beta] as B fragments), four column tiles at a time, the width split over two waves
// per 16-token row tile.  When the width is a multiple of 256 the operands reach the MFMAs through
// LDS: x rows and weight rows are loaded as whole 128-byte lines, and the weight rows of a step
// once per workgroup for its four row-tile waves.  z is rounded to bf16 once; the optional
// log(alpha) is formed from those rounded values by the same MFMA and the same nonlinearity as
// the fused chunk-local kernel, so the two paths agree bit for bit, and leaves through LDS as
// 512-byte row segments.
#include <utility>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kGateTokens = 64;

// Operands of the projections over the model width: lane (grp, r16) supplies row r16 and the 8
// consecutive width indices 32 kb + 8 grp .. + 7 (one 16-byte load).  A and B use the same map,
// so the MFMA sums over all 32 indices of the block; this is not the k-slot map of the other
// kernels, which only matters for fragments shared with them (z below is not loaded this way).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + fast_exp2(-x * kLog2e)); }

}  // namespace

// Waves (tt, kh): row tile tt = w & 3 (16 tokens), half kh = w >> 2 of the model width for the
// projections and of the log-alpha columns.  The width loop works in steps of four k blocks; on
// the direct path a wave issues a step's 20 loads before its MFMAs, on the whole-line path the
// next step's 8 loads are in flight while the current step is formed from LDS.
__global__ void __launch_bounds__(512) gate_kernel(GateArgs a) {
    __shared__ uint16_t zs[kGateTokens][128 + 8];  // the block's rounded z rows (for log(alpha))
    __shared__ f32x4 red[4][4][64];                // upper-half partial sums of four column tiles
    // whole-line path: each wave's 16 x rows and, shared by the four waves of a width half, the
    // weight rows of the column group, 128 widths per step (+ 8 of padding against bank conflicts)
    __shared__ __attribute__((aligned(16))) uint16_t xs[8][16][136];
    // [step parity][half][tile] weight rows; afterwards, per wave, 16 rows x 128 columns of log(alpha)
    __shared__ __attribute__((aligned(16))) union {
        uint16_t w[2][2][4][16][136];
        float g[8][16][132];
    } stg;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    const int tt = wave & 3, kh = wave >> 2;
    const long tok0 = (long)blockIdx.x * kGateTokens;
    const long arow = tok0 + 16 * tt + r16;                      // this lane's A row (token)
    const int xrow = (int)(arow < a.Ntok ? arow : a.Ntok - 1);
    const int nzt = a.r / 16, nbt = (a.H + 15) / 16, nct = nzt + nbt;
    const int nkb = a.Dm / 32, kb0 = kh * (nkb / 2), kb1 = kh ? nkb : nkb / 2;

    // ---- z and beta: column tiles ct < nzt are rank indices, the rest heads.  The loop over the
    // width is branch-free (every tile of the group is loaded from a valid row and masked), so
    // the unrolled iterations keep their loads in flight together.
    const uint16_t *xp = a.x + (long)xrow * a.Dm + 8 * grp;
    // Whole-line path (the width a multiple of 256, so both halves have the same whole steps): load j
    // of a wave covers rows 8 (j >> 1) + (l >> 3) and bytes 128 (j & 1) + 16 (l & 7) of each row's
    // 256-byte step, so every request is a whole 128-byte line; the operands are then read from LDS
    // in the fragment layout.  Loaded directly in the fragment layout, every load holds 16 rows x
    // 64 bytes (each line fetched as two halves) and the four row-tile waves each fetch the same
    // weight rows; the L1 then bounded the kernel (35 us on 16384 tokens of width 2048, 16 us
    // this way).
    const bool lines = (nkb & 7) == 0;  // uniform over the workgroup
    const long lrow0 = tok0 + 16 * tt + (lane >> 3), lrow1 = lrow0 + 8;
    const uint16_t *xl[2] = {a.x + (lrow0 < a.Ntok ? lrow0 : a.Ntok - 1) * (long)a.Dm + 8 * (lane & 7),
                             a.x + (lrow1 < a.Ntok ? lrow1 : a.Ntok - 1) * (long)a.Dm + 8 * (lane & 7)};
    for (int cg = 0; cg < nct; cg += 4) {
        const uint16_t *wp[4];  // this lane's weight row of each tile of the group
        bool wvalid[4];         // false for rows past H (and tiles past the last): zero operand
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ct = cg + u;
            const bool zt = ct < nzt;
            const int row = zt ? 16 * ct + r16 : 16 * (ct - nzt) + r16;
            wvalid[u] = zt || (ct < nct && row < a.H);
            wp[u] = (wvalid[u] ? (zt ? a.w_down : a.w_beta) + (long)row * a.Dm : a.w_down) + 8 * grp;
        }
        f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
        if (lines) {
            // wave (tt, kh) stages weight tile cg + tt of half kh; rows past the valid ones read
            // row 0 of w_down and are masked by the consumer (wvalid)
            const int ctw = cg + tt;
            const bool ztw = ctw < nzt;
            const uint16_t *wl[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int rr = 8 * h2 + (lane >> 3);
                const int row = ztw ? 16 * ctw + rr : 16 * (ctw - nzt) + rr;
                const bool ok = ztw || (ctw < nct && row < a.H);
                wl[h2] = (ok ? (ztw ? a.w_down : a.w_beta) + (long)row * a.Dm : a.w_down) + 8 * (lane & 7);
            }
            auto issue = [&](int kb, u32x4 (&xr)[4], u32x4 (&wr)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xr[j] = ld16(xl[j >> 1] + 32 * kb + 64 * (j & 1));
                    wr[j] = ld16(wl[j >> 1] + 32 * kb + 64 * (j & 1));
                }
            };
            // one step: the loads of the next step are already in flight (other register set)
            auto consume = [&](auto bufc, u32x4 (&xr)[4], u32x4 (&wr)[4]) __attribute__((always_inline)) {
                constexpr int buf = decltype(bufc)::value;
                asm volatile("" : "+v"(xr[0]), "+v"(xr[1]), "+v"(xr[2]), "+v"(xr[3]),
                                  "+v"(wr[0]), "+v"(wr[1]), "+v"(wr[2]), "+v"(wr[3]));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 8 * (j >> 1) + (lane >> 3), cc = 64 * (j & 1) + 8 * (lane & 7);
                    *reinterpret_cast<u32x4 *>(&xs[wave][rr][cc]) = xr[j];
                    *reinterpret_cast<u32x4 *>(&stg.w[buf][kh][tt][rr][cc]) = wr[j];
                }
                __syncthreads();  // the half's four weight tiles of this step are in LDS
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const FragB xa{__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&xs[wave][r16][32 * i + 8 * grp]))};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const u32x4 w = *reinterpret_cast<const u32x4 *>(&stg.w[buf][kh][u][r16][32 * i + 8 * grp]);
                        acc[u] = mfma(xa, FragB{__builtin_bit_cast(bf16x8, wvalid[u] ? w : u32x4{0u, 0u, 0u, 0u})}, acc[u]);
                    }
                }
            };
            // Every load is unconditional (a step past the end reloads the last one), so the wait
            // before each step counts exactly the loads of the step after it.
            u32x4 xa0[4], wa0[4], xa1[4], wa1[4];
            issue(kb0, xa0, wa0);
            for (int kb = kb0; kb < kb1; kb += 8) {
                issue(min(kb + 4, kb1 - 4), xa1, wa1);
                consume(std::integral_constant<int, 0>{}, xa0, wa0);
                issue(min(kb + 8, kb1 - 4), xa0, wa0);
                if (kb + 4 < kb1) consume(std::integral_constant<int, 1>{}, xa1, wa1);
            }
        } else {
        // four k blocks per step: all 20 loads are issued before the 16 MFMAs that use them
        for (int kb = kb0; kb < kb1; kb += 4) {
            u32x4 xv[4], wv4[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = min(kb + i, kb1 - 1);  // past the end: a valid block, zeroed below
                xv[i] = ld16(xp + 32 * kk);
#pragma unroll
                for (int u = 0; u < 4; ++u) wv4[i][u] = ld16(wp[u] + 32 * kk);
            }
            // The loaded values pass through an empty asm statement: every load is issued before it
            // and no MFMA moves above it, so all 20 loads are in flight together (left alone, the
            // scheduler issues each load just before its MFMA).
            asm volatile("" : "+v"(xv[0]), "+v"(xv[1]), "+v"(xv[2]), "+v"(xv[3]),
                              "+v"(wv4[0][0]), "+v"(wv4[0][1]), "+v"(wv4[0][2]), "+v"(wv4[0][3]),
                              "+v"(wv4[1][0]), "+v"(wv4[1][1]), "+v"(wv4[1][2]), "+v"(wv4[1][3]),
                              "+v"(wv4[2][0]), "+v"(wv4[2][1]), "+v"(wv4[2][2]), "+v"(wv4[2][3]),
                              "+v"(wv4[3][0]), "+v"(wv4[3][1]), "+v"(wv4[3][2]), "+v"(wv4[3][3]));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (kb + i >= kb1) xv[i] = u32x4{0u, 0u, 0u, 0u};
                const FragB xa{__builtin_bit_cast(bf16x8, xv[i])};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const u32x4 w = wvalid[u] ? wv4[i][u] : u32x4{0u, 0u, 0u, 0u};
                    acc[u] = mfma(xa, FragB{__builtin_bit_cast(bf16x8, w)}, acc[u]);
                }
            }
        }
        }
        // add the two halves in a fixed order (lower + upper), so the result is deterministic
        if (kh == 1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) red[tt][u][lane] = acc[u];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ct = cg + u;
                if (ct >= nct) break;
                acc[u] += red[tt][u][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int trow = 16 * tt + 4 * grp + e;  // token row within the block
                    const long tok = tok0 + trow;
                    if (ct < nzt) {
                        const int j = 16 * ct + r16;
                        const uint16_t zb = __builtin_bit_cast(uint16_t, (__bf16)acc[u][e]);  // round to nearest even
                        zs[trow][j] = zb;
                        if (tok < a.Ntok) a.z[tok * a.r + j] = zb;
                    } else {
                        const int hh = 16 * (ct - nzt) + r16;
                        if (tok < a.Ntok && hh < a.H) a.beta[tok * a.H + hh] = sigmoidf_(acc[u][e]);
                    }
                }
            }
        }
        __syncthreads();  // red is reused by the next column group; zs is complete after the last
    }
    if (!a.g) return;  // uniform over the grid

    // ---- log(alpha) = -softplus(z W_up^T + b) from the rounded z (A fragments read back from LDS);
    // wave (tt, kh) forms row tile tt for half kh of the columns
    const int nrk = a.r / 32;
    FragB za[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (kb >= nrk) break;
        const uint16_t *p = &zs[16 * tt + r16][32 * kb + 4 * grp];
        za[kb] = frag_bits(*reinterpret_cast<const uint2 *>(p), *reinterpret_cast<const uint2 *>(p + 16));
    }
    const int ncols = a.H * a.d, nt = ncols / 16, ct0 = kh * (nt / 2), ct1 = kh ? nt : nt / 2;
    auto tile = [&](int ct) __attribute__((always_inline)) {  // z W_up^T + b of column tile ct
        const int c = 16 * ct + r16;
        const uint16_t *wr = a.w_up + (long)c * a.r + 4 * grp;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb >= nrk) break;
            acc = mfma(za[kb], frag_bits(*reinterpret_cast<const uint2 *>(wr + 32 * kb),
                                         *reinterpret_cast<const uint2 *>(wr + 32 * kb + 16)), acc);
        }
        const float bc = a.b[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += bc;
        return acc;
    };
    if ((nt & 15) == 0) {
        // Eight column tiles at a time go through the wave's LDS tile, and each token row then
        // leaves as 512 contiguous bytes (two rows per store instruction); stored straight from
        // the MFMA layout, every store wrote 64-byte pieces of four rows.
        for (int cg8 = ct0; cg8 < ct1; cg8 += 8) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const f32x4 acc = tile(cg8 + u);
#pragma unroll
                for (int e = 0; e < 4; ++e) stg.g[wave][4 * grp + e][16 * u + r16] = gate_log_alpha(acc[e]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int rr = 2 * j + (lane >> 5);
                const long tok = tok0 + 16 * tt + rr;
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&stg.g[wave][rr][4 * (lane & 31)]);
                if (tok < a.Ntok) *reinterpret_cast<f32x4 *>(a.g + tok * ncols + 16 * cg8 + 4 * (lane & 31)) = v;
            }
        }
    } else {
#pragma unroll 4
        for (int ct = ct0; ct < ct1; ++ct) {
            const f32x4 acc = tile(ct);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long tok = tok0 + 16 * tt + 4 * grp + e;
                if (tok < a.Ntok) a.g[tok * ncols + 16 * ct + r16] = gate_log_alpha(acc[e]);
            }
        }
    }
}

hipError_t launch_gate(const GateArgs &a, hipStream_t st) {
    if (a.Ntok <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.Ntok + kGateTokens - 1) / kGateTokens);
    return launch_kernel(gate_kernel, dim3(blocks), dim3(512), st, a);
}

}  // namespace kda
