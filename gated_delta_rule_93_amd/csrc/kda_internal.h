// kda_internal.h -- launcher interface between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "../../include/kda.h"

namespace kda {

// The argument checks of kda_fwd (sizes, pointers, alignment, workspace against the windowed
// minimum), without launching anything.
kda_status_t fwd_check_args(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                            int N, const void *q, const void *k, const void *v, const float *g, const float *beta,
                            const float *initial_state, const float *final_state, const void *o,
                            const void *workspace, size_t workspace_bytes);

// Launch `kern` on `st` and return the runtime's status for this launch itself (hipLaunchKernel
// reports it directly; no sticky error left on the thread by an earlier, unrelated call is read
// or cleared).  Each argument is converted to the kernel's parameter type.
template <typename... P, size_t... I>
inline hipError_t launch_kernel_impl(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t st,
                                     std::tuple<P...> &vals, std::index_sequence<I...>) {
    void *ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1] = {static_cast<void *>(&std::get<I>(vals))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block, ptrs, 0, st);
}
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t st, A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals{static_cast<P>(args)...};
    return launch_kernel_impl(kern, grid, block, st, vals, std::index_sequence_for<P...>{});
}

struct DecodeArgs {
    bool bf16;
    int N, H, dk, dv;
    const void *q, *k, *v;
    const float *g, *beta;
    float scale;
    float *state;
    void *o;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);

struct PrepArgs {
    bool bf16;
    int B, T, H, d, W, N;
    const int32_t *cu_seqlens;  // NULL: dense rows
    const void *x;
    const float *w;
    void *y;
};
hipError_t launch_prep(const PrepArgs &a, hipStream_t st);

struct FwdArgs {
    bool bf16;
    int B, T, H, dk, dv, N;
    const int32_t *cu_seqlens;  // NULL: dense
    const void *q, *k, *v;
    const float *g, *beta;
    bool scalar_gate;           // g is [B, T, H] (one log-decay per token and head), or NULL (alpha = 1)
    // Low-rank gate (g == NULL, bf16 only): log(alpha) = -softplus(z W_up^T + b), formed in the
    // chunk-local kernel; z [tokens, r], w_up [H*dk, r] (bf16 bits), b [H*dk]; r % 32 == 0, r <= 128.
    const uint16_t *gate_z, *gate_w_up;
    const float *gate_b;
    int gate_r;
    float scale;
    const float *s0;
    float *sN;
    void *o;
    void *ws;
    float *map_A;               // segment map only: the linear part A [N, H, dk, dk] (sN receives B)
};
// Bytes of workspace for one (chunk, head) and the number of chunk slots.
size_t fwd_bytes_per_chunk_head(bool bf16, int d);
long fwd_chunk_slots(int B, int T, int N, bool varlen);
// How kda_fwd splits the chunks into windows for a workspace of ws_bytes: Wc chunk indices per
// window, nwin windows; with carry, the state travels between windows in the workspace at
// carry_off (no final_state given).  False when the workspace is too small for one chunk per
// window.  fwd_min_workspace is the smallest workspace plan_fwd_windows accepts.
struct WindowPlan {
    long Wc, nwin;
    size_t carry_off;
    bool carry;
};
bool plan_fwd_windows(bool bf16, int d, int B, int T, int H, int N, bool varlen, bool have_final_state,
                      size_t ws_bytes, WindowPlan &p);
size_t fwd_min_workspace(bool bf16, int d, int B, int T, int H, int N, bool varlen, bool have_final_state);
// Both phases over the windows that a workspace of ws_bytes allows.
hipError_t launch_fwd(const FwdArgs &a, size_t ws_bytes, hipStream_t st);
hipError_t launch_fwd_local(const FwdArgs &a, hipStream_t st);    // chunk-local phase
hipError_t launch_fwd_scan(const FwdArgs &a, hipStream_t st);     // state-scan phase
// The affine map S_out = A S_in + B of every (sequence, head) chain, from the chunk-local records
// (a.map_A receives A, a.sN receives B; s0 and o are not used).
hipError_t launch_fwd_segment_map(const FwdArgs &a, hipStream_t st);

// out[c] = A[c] S[c] + B[c] for c < count; A [count, d, d], S, B, out [count, d, d] fp32.
hipError_t launch_state_combine(int count, int d, const float *A, const float *S, const float *B, float *out,
                                hipStream_t st);

struct GateArgs {
    int Ntok, Dm, H, d, r;
    const uint16_t *x, *w_down, *w_beta, *w_up;  // bf16 bits: [Ntok, Dm], [r, Dm], [H, Dm], [H*d, r]
    const float *b;                              // [H*d]
    uint16_t *z;                                 // [Ntok, r] bf16
    float *beta;                                 // [Ntok, H]
    float *g;                                    // [Ntok, H, d] or NULL
};
hipError_t launch_gate(const GateArgs &a, hipStream_t st);

constexpr int kAttnResMaxBlocks = 16, kAttnResMaxLayers = 16;
struct AttnResArgs {             // one-shot read-out, or the merge when prior_o != NULL
    int n, T, d;
    const uint16_t *blk[kAttnResMaxBlocks];  // block outputs, each [T, d] bf16
    const uint16_t *w;                       // [d] bf16 query
    float eps;
    const uint16_t *prior_o;                 // [T, d] bf16 or NULL
    const float *prior_lse;                  // [T] (with prior_o)
    uint16_t *h;                             // [T, d] bf16
};
struct AttnScoreArgs {
    int n, L, T, d;
    const uint16_t *blk[kAttnResMaxBlocks];
    const uint16_t *W;                       // [L, d] bf16 queries
    float *dots;                             // [n, T, 16] workspace
    float *sumsq;                            // [n, T] workspace
};
struct AttnMixArgs {
    int n, L, T, d;
    const uint16_t *blk[kAttnResMaxBlocks];
    float eps;
    const float *dots, *sumsq;
    uint16_t *o;                             // [L, T, d] bf16
    float *lse;                              // [L, T] or NULL
};
hipError_t launch_attnres(const AttnResArgs &a, hipStream_t st);
hipError_t launch_attnres_inter(const AttnScoreArgs &s, const AttnMixArgs &m, hipStream_t st);

}  // namespace kda
