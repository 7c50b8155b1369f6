// kda_api.hip -- extern "C" entry points of libkda.so: argument validation and launches.
// Semantics, layouts and error behaviour are documented in include/kda.h.
#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool supported_d(int d) { return d == 64 || d == 128; }
bool valid_dtype(kda_dtype_t io) { return io == KDA_F32 || io == KDA_BF16; }
// true when the byte ranges [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK: success";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT: null pointer, bad size, misaligned buffer or bad dtype";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: valid arguments that the library does not implement";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case KDA_ERR_TOO_LARGE:
            return "KDA_ERR_TOO_LARGE: the sizes need more than the library's fixed device scratch "
                   "(KDA_NOALLOC_SCRATCH_BYTES; kda_fwd_noalloc)";
    }
    return "KDA: unknown status";
}

size_t kda_fwd_workspace_bytes(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, int N, int varlen) {
    if (!valid_dtype(io) || B < 0 || T < 0 || H < 0 || N < 0) return 0;
    if (d_k != d_v || !supported_d(d_k)) return 0;
    if (varlen && B != 1) return 0;
    const long slots = kda::fwd_chunk_slots(B, T, N, varlen != 0);
    return (size_t)slots * (size_t)H * kda::fwd_bytes_per_chunk_head(io == KDA_BF16, d_k);
}

size_t kda_fwd_workspace_min_bytes(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, int N, int varlen,
                                   int have_final_state) {
    if (!valid_dtype(io) || B < 0 || T < 0 || H < 0 || N < 0) return 0;
    if (d_k != d_v || !supported_d(d_k)) return 0;
    if (varlen && B != 1) return 0;
    return kda::fwd_min_workspace(io == KDA_BF16, d_k, B, T, H, N, varlen != 0, have_final_state != 0);
}

size_t kda_attnres_inter_workspace_bytes(int n, int L, int T) {
    if (n < 1 || n > kda::kAttnResMaxBlocks || L < 1 || L > kda::kAttnResMaxLayers || T < 0) return 0;
    return (size_t)n * (size_t)T * (16 + 1) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by kda_fwd and its two phases.  Pointers passed as `nullptr_ok` sentinels
// are not required by the calling phase.
enum FwdPart { kLocal = 1, kScan = 2, kBoth = 3 };

kda_status_t check_fwd(int part, kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                       const int32_t *cu_seqlens, int N, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const float *s0, const float *sN, const void *o,
                       const void *workspace, size_t workspace_bytes, bool g_optional = false) {
    if (!valid_dtype(io) || B < 0 || T < 0 || H < 0 || N < 0 || d_k <= 0 || d_v <= 0)
        return KDA_ERR_INVALID_ARGUMENT;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned4(cu_seqlens)) return KDA_ERR_INVALID_ARGUMENT;  // read as int32 scalars
    } else if (N != B) {
        return KDA_ERR_INVALID_ARGUMENT;
    }
    if (d_k != d_v || !supported_d(d_k)) return KDA_ERR_UNSUPPORTED;
    const long tokens = (long)B * T;
    if (tokens > 0 && H > 0) {
        if (part & kLocal) {
            if (!q || !k || !v || (!g && !g_optional) || !beta) return KDA_ERR_INVALID_ARGUMENT;
            if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (g && !aligned16(g)))
                return KDA_ERR_INVALID_ARGUMENT;
        }
        if (part & kScan) {
            if (!o || !aligned16(o)) return KDA_ERR_INVALID_ARGUMENT;
        }
    }
    if ((part & kScan) && ((s0 && !aligned16(s0)) || (sN && !aligned16(sN)))) return KDA_ERR_INVALID_ARGUMENT;
    // the whole prefill runs in windows when the workspace does not hold every chunk's record;
    // its two phases called on their own need the whole workspace
    const size_t need = part == kBoth
                            ? kda::fwd_min_workspace(io == KDA_BF16, d_k, B, T, H, N, cu_seqlens != nullptr, sN != nullptr)
                            : kda_fwd_workspace_bytes(io, B, T, H, d_k, d_v, N, cu_seqlens != nullptr);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return KDA_ERR_WORKSPACE;
    return KDA_OK;
}

// Checks of the low-rank gate operands shared by the fused forward and its chunk-local phase
// (after check_fwd).
kda_status_t check_lowrank(kda_dtype_t io, int B, int T, int N, int H, const void *z, int r, const void *w_up,
                           const float *b_gate) {
    if (r <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (io != KDA_BF16 || r % 32 != 0 || r > 128) return KDA_ERR_UNSUPPORTED;
    if ((long)N * H == 0) return KDA_OK;
    if ((long)B * T > 0) {
        if (!z || !w_up || !b_gate) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned16(z) || !aligned16(w_up) || !aligned16(b_gate)) return KDA_ERR_INVALID_ARGUMENT;
    }
    return KDA_OK;
}

kda::FwdArgs fwd_args(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens, int N,
                      const void *q, const void *k, const void *v, const float *g, const float *beta, float scale,
                      const float *s0, float *sN, void *o, void *workspace) {
    kda::FwdArgs a;
    a.bf16 = io == KDA_BF16;
    a.B = B; a.T = T; a.H = H; a.dk = d_k; a.dv = d_v; a.N = N;
    a.cu_seqlens = cu_seqlens;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.scalar_gate = false; a.scale = scale;
    a.s0 = s0; a.sN = sN; a.o = o; a.ws = workspace;
    a.gate_z = nullptr; a.gate_w_up = nullptr; a.gate_b = nullptr; a.gate_r = 0;
    a.map_A = nullptr;
    return a;
}

}  // namespace

kda_status_t kda::fwd_check_args(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                                 int N, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *initial_state, const float *final_state,
                                 const void *o, const void *workspace, size_t workspace_bytes) {
    return check_fwd(kBoth, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, initial_state, final_state, o,
                     workspace, workspace_bytes);
}

extern "C" {

kda_status_t kda_fwd(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens, int N,
                     const void *q, const void *k, const void *v, const float *g, const float *beta, float scale,
                     const float *initial_state, float *final_state, void *o, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kBoth, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, initial_state,
                                final_state, o, workspace, workspace_bytes);
    if (st != KDA_OK || (long)N * H == 0) return st;
    const kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, scale, initial_state,
                                    final_state, o, workspace);
    return kda::launch_fwd(a, workspace_bytes, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_scalar_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                                 int N, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, float scale, const float *initial_state, float *final_state,
                                 void *o, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kBoth, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, initial_state,
                                final_state, o, workspace, workspace_bytes, true);
    if (st != KDA_OK || (long)N * H == 0) return st;
    kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, scale, initial_state,
                              final_state, o, workspace);
    a.scalar_gate = true;
    return kda::launch_fwd(a, workspace_bytes, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_lowrank_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                  const int32_t *cu_seqlens, int N, const void *q, const void *k, const void *v,
                                  const void *z, int r, const void *w_up, const float *b_gate, const float *beta,
                                  float scale, const float *initial_state, float *final_state, void *o,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kBoth, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, nullptr, beta, initial_state,
                                final_state, o, workspace, workspace_bytes, true);
    if (st != KDA_OK) return st;
    st = check_lowrank(io, B, T, N, H, z, r, w_up, b_gate);
    if (st != KDA_OK || (long)N * H == 0) return st;
    kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, nullptr, beta, scale, initial_state,
                              final_state, o, workspace);
    a.gate_z = static_cast<const uint16_t *>(z);
    a.gate_w_up = static_cast<const uint16_t *>(w_up);
    a.gate_b = b_gate;
    a.gate_r = r;
    return kda::launch_fwd(a, workspace_bytes, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_gate(kda_dtype_t io, int Ntok, int Dm, int H, int d_k, int r, const void *x, const void *w_down,
                      const void *w_beta, const void *w_up, const float *b_gate, void *z, float *beta, float *g,
                      hipStream_t stream) {
    if (!valid_dtype(io) || Ntok < 0 || Dm <= 0 || H <= 0 || d_k <= 0 || r <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (io != KDA_BF16 || r % 32 != 0 || r > 128 || Dm % 32 != 0 || !supported_d(d_k)) return KDA_ERR_UNSUPPORTED;
    if (Ntok == 0) return KDA_OK;
    if (!x || !w_down || !w_beta || !z || !beta) return KDA_ERR_INVALID_ARGUMENT;
    if (g && (!w_up || !b_gate)) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_down) || !aligned16(w_beta) || !aligned16(z) || !aligned16(beta))
        return KDA_ERR_INVALID_ARGUMENT;
    if (g && (!aligned16(g) || !aligned16(w_up) || !aligned16(b_gate))) return KDA_ERR_INVALID_ARGUMENT;
    kda::GateArgs a;
    a.Ntok = Ntok; a.Dm = Dm; a.H = H; a.d = d_k; a.r = r;
    a.x = static_cast<const uint16_t *>(x);
    a.w_down = static_cast<const uint16_t *>(w_down);
    a.w_beta = static_cast<const uint16_t *>(w_beta);
    a.w_up = static_cast<const uint16_t *>(w_up);
    a.b = b_gate;
    a.z = static_cast<uint16_t *>(z);
    a.beta = beta;
    a.g = g;
    return kda::launch_gate(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Checks shared by the AttnRes entry points: dtype, sizes, the host array of block pointers.
kda_status_t check_attnres(kda_dtype_t io, int n, int T, int d, float eps, const void *const *blocks) {
    if (!valid_dtype(io) || n < 1 || T < 0 || d <= 0 || !(eps >= 0.f)) return KDA_ERR_INVALID_ARGUMENT;
    if (io != KDA_BF16 || n > kda::kAttnResMaxBlocks || d % 512 != 0 || d > 4096) return KDA_ERR_UNSUPPORTED;
    if (T == 0) return KDA_OK;
    if (!blocks) return KDA_ERR_INVALID_ARGUMENT;
    for (int b = 0; b < n; ++b)
        if (!blocks[b] || !aligned16(blocks[b])) return KDA_ERR_INVALID_ARGUMENT;
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_attnres(kda_dtype_t io, int n, int T, int d, const void *const *blocks, const void *w, float eps,
                         void *h, hipStream_t stream) {
    kda_status_t st = check_attnres(io, n, T, d, eps, blocks);
    if (st != KDA_OK || T == 0) return st;
    if (!w || !h || !aligned16(w) || !aligned16(h)) return KDA_ERR_INVALID_ARGUMENT;
    kda::AttnResArgs a{};
    a.n = n; a.T = T; a.d = d; a.eps = eps;
    for (int b = 0; b < n; ++b) a.blk[b] = static_cast<const uint16_t *>(blocks[b]);
    a.w = static_cast<const uint16_t *>(w);
    a.prior_o = nullptr; a.prior_lse = nullptr;
    a.h = static_cast<uint16_t *>(h);
    return kda::launch_attnres(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_attnres_inter(kda_dtype_t io, int n, int L, int T, int d, const void *const *blocks, const void *W,
                               float eps, void *o_bar, float *lse, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (L < 1) return KDA_ERR_INVALID_ARGUMENT;
    kda_status_t st = check_attnres(io, n, T, d, eps, blocks);
    if (st != KDA_OK) return st;
    if (L > kda::kAttnResMaxLayers) return KDA_ERR_UNSUPPORTED;
    if (T == 0) return KDA_OK;
    if (!W || !o_bar || !aligned16(W) || !aligned16(o_bar) || (lse && !aligned4(lse))) return KDA_ERR_INVALID_ARGUMENT;
    const size_t need = kda_attnres_inter_workspace_bytes(n, L, T);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KDA_ERR_WORKSPACE;
    kda::AttnScoreArgs s{};
    kda::AttnMixArgs m{};
    s.n = m.n = n; s.L = m.L = L; s.T = m.T = T; s.d = m.d = d;
    for (int b = 0; b < n; ++b) s.blk[b] = m.blk[b] = static_cast<const uint16_t *>(blocks[b]);
    float *dots = static_cast<float *>(workspace);
    float *sumsq = dots + (size_t)n * T * 16;
    s.W = static_cast<const uint16_t *>(W); s.dots = dots; s.sumsq = sumsq;
    m.eps = eps; m.dots = dots; m.sumsq = sumsq; m.o = static_cast<uint16_t *>(o_bar); m.lse = lse;
    return kda::launch_attnres_inter(s, m, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_attnres_merge(kda_dtype_t io, int T, int d, const void *partial, const void *w, float eps,
                               const void *o_bar, const float *lse, void *h, hipStream_t stream) {
    const void *blocks[1] = {partial};
    kda_status_t st = check_attnres(io, 1, T, d, eps, blocks);
    if (st != KDA_OK || T == 0) return st;
    if (!w || !o_bar || !lse || !h || !aligned16(w) || !aligned16(o_bar) || !aligned4(lse) || !aligned16(h))
        return KDA_ERR_INVALID_ARGUMENT;
    kda::AttnResArgs a{};
    a.n = 1; a.T = T; a.d = d; a.eps = eps;
    a.blk[0] = static_cast<const uint16_t *>(partial);
    a.w = static_cast<const uint16_t *>(w);
    a.prior_o = static_cast<const uint16_t *>(o_bar);
    a.prior_lse = lse;
    a.h = static_cast<uint16_t *>(h);
    return kda::launch_attnres(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_chunk_local(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                                 int N, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kLocal, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, nullptr, nullptr,
                                nullptr, workspace, workspace_bytes);
    if (st != KDA_OK || (long)N * H == 0) return st;
    const kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, 1.f, nullptr, nullptr,
                                    nullptr, workspace);
    return kda::launch_fwd_local(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_state_scan(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                                int N, float scale, const float *initial_state, float *final_state, void *o,
                                void *workspace, size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kScan, io, B, T, H, d_k, d_v, cu_seqlens, N, nullptr, nullptr, nullptr, nullptr,
                                nullptr, initial_state, final_state, o, workspace, workspace_bytes);
    if (st != KDA_OK || (long)N * H == 0) return st;
    const kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, scale, initial_state, final_state, o, workspace);
    return kda::launch_fwd_scan(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_chunk_local_scalar_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                             const int32_t *cu_seqlens, int N, const void *q, const void *k,
                                             const void *v, const float *g, const float *beta, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kLocal, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, nullptr, nullptr,
                                nullptr, workspace, workspace_bytes, true);
    if (st != KDA_OK || (long)N * H == 0) return st;
    kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, g, beta, 1.f, nullptr, nullptr,
                              nullptr, workspace);
    a.scalar_gate = true;
    return kda::launch_fwd_local(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_chunk_local_lowrank_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                              const int32_t *cu_seqlens, int N, const void *q, const void *k,
                                              const void *v, const void *z, int r, const void *w_up,
                                              const float *b_gate, const float *beta, void *workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
    kda_status_t st = check_fwd(kLocal, io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, nullptr, beta, nullptr,
                                nullptr, nullptr, workspace, workspace_bytes, true);
    if (st != KDA_OK) return st;
    st = check_lowrank(io, B, T, N, H, z, r, w_up, b_gate);
    if (st != KDA_OK || (long)N * H == 0) return st;
    kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, q, k, v, nullptr, beta, 1.f, nullptr, nullptr,
                              nullptr, workspace);
    a.gate_z = static_cast<const uint16_t *>(z);
    a.gate_w_up = static_cast<const uint16_t *>(w_up);
    a.gate_b = b_gate;
    a.gate_r = r;
    return kda::launch_fwd_local(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_fwd_segment_map(kda_dtype_t io, int B, int T, int H, int d_k, int d_v, const int32_t *cu_seqlens,
                                 int N, float *transition, float *offset, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    kda_status_t st = check_fwd(0, io, B, T, H, d_k, d_v, cu_seqlens, N, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes);
    if (st != KDA_OK || (long)N * H == 0) return st;
    if (!transition || !offset || !aligned16(transition) || !aligned16(offset)) return KDA_ERR_INVALID_ARGUMENT;
    const size_t bytes = (size_t)N * H * d_k * d_v * sizeof(float);
    if (overlaps(transition, bytes, offset, bytes)) return KDA_ERR_INVALID_ARGUMENT;
    kda::FwdArgs a = fwd_args(io, B, T, H, d_k, d_v, cu_seqlens, N, nullptr, nullptr, nullptr, nullptr, nullptr,
                              1.f, nullptr, offset, nullptr, workspace);
    a.map_A = transition;
    return kda::launch_fwd_segment_map(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_state_combine(int count, int d_k, int d_v, const float *transition, const float *state_in,
                               const float *offset, float *state_out, hipStream_t stream) {
    if (count < 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (d_k != d_v || !supported_d(d_k)) return KDA_ERR_UNSUPPORTED;
    if (count > (1 << 26)) return KDA_ERR_UNSUPPORTED;  // grid size
    if (count == 0) return KDA_OK;
    if (!transition || !state_in || !state_out) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(transition) || !aligned16(state_in) || (offset && !aligned16(offset)) || !aligned16(state_out))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t bytes = (size_t)count * d_k * d_v * sizeof(float);
    if (overlaps(state_out, bytes, transition, bytes) || overlaps(state_out, bytes, state_in, bytes))
        return KDA_ERR_INVALID_ARGUMENT;
    if (offset && offset != state_out && overlaps(state_out, bytes, offset, bytes)) return KDA_ERR_INVALID_ARGUMENT;
    return kda::launch_state_combine(count, d_k, transition, state_in, offset, state_out, stream) == hipSuccess
               ? KDA_OK
               : KDA_ERR_LAUNCH;
}

kda_status_t kda_decode_step(kda_dtype_t io, int N, int H, int d_k, int d_v, const void *q, const void *k,
                             const void *v, const float *g, const float *beta, float scale, float *state, void *o,
                             hipStream_t stream) {
    if (!valid_dtype(io) || N < 0 || H < 0 || d_k <= 0 || d_v <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (!supported_d(d_k) || !supported_d(d_v)) return KDA_ERR_UNSUPPORTED;
    if ((long)N * H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(state) || !aligned16(o))
        return KDA_ERR_INVALID_ARGUMENT;
    kda::DecodeArgs a;
    a.bf16 = io == KDA_BF16;
    a.N = N; a.H = H; a.dk = d_k; a.dv = d_v;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.scale = scale; a.state = state; a.o = o;
    return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status_t kda_prep(kda_dtype_t io, int B, int T, int H, int d, const int32_t *cu_seqlens, int N, const void *x,
                      const float *conv_w, int W, void *y, hipStream_t stream) {
    if (!valid_dtype(io) || B < 0 || T < 0 || H < 0 || d <= 0 || N < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (W < 1 || W > 8) return W < 1 ? KDA_ERR_INVALID_ARGUMENT : KDA_ERR_UNSUPPORTED;
    if (cu_seqlens) {
        if (B != 1 || N < 1) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned4(cu_seqlens)) return KDA_ERR_INVALID_ARGUMENT;  // read as int32 scalars
    }
    if (!supported_d(d)) return KDA_ERR_UNSUPPORTED;
    if ((long)B * T * H == 0) return KDA_OK;
    if (!x || !conv_w || !y) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(y) || !aligned16(conv_w)) return KDA_ERR_INVALID_ARGUMENT;
    if (x == y) return KDA_ERR_INVALID_ARGUMENT;
    kda::PrepArgs a;
    a.bf16 = io == KDA_BF16;
    a.B = B; a.T = T; a.H = H; a.d = d; a.W = W; a.N = cu_seqlens ? N : B;
    a.cu_seqlens = cu_seqlens; a.x = x; a.w = conv_w; a.y = y;
    return kda::launch_prep(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"
