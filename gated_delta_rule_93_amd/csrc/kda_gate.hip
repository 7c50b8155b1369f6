// kda_gate.hip -- the gate prologue: the low-rank down projection z = x W_down^T (stored bf16),
// beta = sigmoid(x w_beta^T), and, when asked, log(alpha) = -softplus(z W_up^T + b) written out.
//
// The page "Kimi K3 注意力三件套" (KDA section) says alpha is produced by a low-rank down-up
// projection of the input and beta is one scalar; blog post-114, chapter 3 has beta as the
// sigmoid of a linear map of x and chapter 4 a gate per head and channel computed from x.
//
// One 256-thread workgroup per 64 tokens; wave w owns tokens 16w .. 16w+15 of the block.  The
// down projection and the beta projection are one skinny bf16 MFMA product over the model width
// (x rows as A fragments, the stacked weight rows [W_down; w_beta] as B fragments), four column
// tiles at a time.  z is rounded to bf16 once; the optional log(alpha) is formed from those
// rounded values by the same MFMA and the same nonlinearity as the fused chunk-local kernel, so
// the two paths agree bit for bit.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kGateTokens = 64;

// B fragment of row `row` of a [rows, ld] bf16 matrix, k block kb (zero past `rows`).
__device__ __forceinline__ FragB row_frag(const uint16_t *w, int rows, long ld, int row, int kb, int grp) {
    if (row >= rows) return frag_bits(make_uint2(0u, 0u), make_uint2(0u, 0u));
    const uint16_t *p = w + (long)row * ld + 32 * kb + 4 * grp;
    return frag_bits(*reinterpret_cast<const uint2 *>(p), *reinterpret_cast<const uint2 *>(p + 16));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + fast_exp2(-x * kLog2e)); }

}  // namespace

__global__ void __launch_bounds__(256) gate_kernel(GateArgs a) {
    __shared__ uint16_t zs[kGateTokens][128 + 8];  // the block's rounded z rows (for log(alpha))
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    const long tok0 = (long)blockIdx.x * kGateTokens;
    const long arow = tok0 + 16 * wave + r16;                      // this lane's A row (token)
    const uint16_t *xr = a.x + (arow < a.Ntok ? arow : a.Ntok - 1) * (long)a.Dm + 4 * grp;
    const int nzt = a.r / 16, nbt = (a.H + 15) / 16, nct = nzt + nbt;
    const int nkb = a.Dm / 32;

    // ---- z and beta: column tiles ct < nzt are rank indices, the rest heads
    for (int cg = 0; cg < nct; cg += 4) {
        f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
        for (int kb = 0; kb < nkb; ++kb) {
            const FragB xa = frag_bits(*reinterpret_cast<const uint2 *>(xr + 32 * kb),
                                       *reinterpret_cast<const uint2 *>(xr + 32 * kb + 16));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ct = cg + u;
                if (ct >= nct) break;
                const FragB wb = ct < nzt ? row_frag(a.w_down, a.r, a.Dm, 16 * ct + r16, kb, grp)
                                          : row_frag(a.w_beta, a.H, a.Dm, 16 * (ct - nzt) + r16, kb, grp);
                acc[u] = mfma(xa, wb, acc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ct = cg + u;
            if (ct >= nct) break;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int trow = 16 * wave + 4 * grp + e;  // token row within the block
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
    if (!a.g) return;  // uniform over the grid

    // ---- log(alpha) = -softplus(z W_up^T + b) from the rounded z (A fragments read back from LDS)
    __syncthreads();
    const int nrk = a.r / 32;
    FragB za[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (kb >= nrk) break;
        const uint16_t *p = &zs[16 * wave + r16][32 * kb + 4 * grp];
        za[kb] = frag_bits(*reinterpret_cast<const uint2 *>(p), *reinterpret_cast<const uint2 *>(p + 16));
    }
    const int ncols = a.H * a.d;
    for (int ct = 0; ct < ncols / 16; ++ct) {
        const int c = 16 * ct + r16;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb >= nrk) break;
            acc = mfma(za[kb], row_frag(a.w_up, ncols, a.r, c, kb, grp), acc);
        }
        const float bc = a.b[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long tok = tok0 + 16 * wave + 4 * grp + e;
            if (tok < a.Ntok) a.g[tok * ncols + c] = gate_log_alpha(acc[e] + bc);
        }
    }
}

hipError_t launch_gate(const GateArgs &a, hipStream_t st) {
    if (a.Ntok <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.Ntok + kGateTokens - 1) / kGateTokens);
    hipLaunchKernelGGL(gate_kernel, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace kda
