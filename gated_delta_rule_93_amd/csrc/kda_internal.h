// kda_internal.h -- launcher interface between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

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
hipError_t launch_fwd(const FwdArgs &a, hipStream_t st);          // both phases
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
