/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator library (libkda.so).
 *
 * The operator (one sequence n, one head h, tokens t = 1..L):
 *     S~  = Diag(alpha_t) S_{t-1},            alpha_t = exp(g_t) in (0,1]^{d_k}
 *     S_t = S~ + beta_t k_t (v_t - S~^T k_t)^T
 *     o_t = scale * S_t^T q_t
 * Sources: course page "线性注意力与 KDA" (ai.air7.fun, Day 19), section 3 (decay per
 * channel, then the delta write of the prediction error) and section 2 (read-out
 * o_t = q_t S_t with a fixed d_k x d_v state); page "Kimi K3 注意力三件套"
 * (yeyulingfeng.com), KDA section (alpha_t is a vector over the d_k channels; q and k
 * pass a short causal convolution and an L2 norm; deployment uses a chunkwise form);
 * blog post ciyuanerhao.com post-114, chapter 3 (state passed in as a cache that
 * defaults to zero; DeltaNet code in [d_k, d_v] orientation) and chapter 4
 * (alpha of shape (B, T, C) multiplying the rows of S).
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers to contiguous row-major buffers,
 *     16-byte aligned.  The caller owns all memory, including the workspace; the
 *     library never allocates, frees or keeps device memory, keeps no global
 *     state and may be called concurrently on different streams.
 *   - io dtype (KDA_F32 or KDA_BF16) applies to q, k, v, o and to x, y of kda_prep.
 *     g (= log alpha), beta, conv weights and states are always fp32.
 *   - State layout [N, H, d_k, d_v] fp32, K-major: element (i, j) couples key
 *     channel i with value channel j, so o = S^T q.
 *   - Host-checkable arguments are validated before anything is launched; on
 *     error a status is returned and no output is touched.  Device contents
 *     (finite inputs, monotone cu_seqlens) are the caller's contract; NaN and Inf
 *     propagate.  g must be finite (g = -inf, a hard reset, is not supported).
 *   - Work is enqueued on `stream` and the call returns without synchronising.
 *     Kernel faults surface at the caller's next synchronisation.  No float
 *     atomics are used: results are bitwise reproducible on one device.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes and element types are plain ints across the ABI, so a caller may pass any value
 * (an unknown dtype or status code is reported, never undefined behaviour). */
typedef int32_t kda_status_t;
enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned buffer, bad dtype */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. d_k not in {64, 128}) */
    KDA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than kda_fwd_workspace_bytes */
    KDA_ERR_LAUNCH = 4,           /* the HIP runtime rejected a kernel launch */
    KDA_ERR_TOO_LARGE = 5         /* kda_fwd_noalloc: sizes need more than its fixed scratch */
};

typedef int32_t kda_dtype_t;
enum { KDA_F32 = 0, KDA_BF16 = 1 };

/* Static, NUL-terminated description of a status code (never NULL). */
const char *kda_status_string(kda_status_t status);

/*
 * Workspace for kda_fwd to run every chunk in one pass (bytes, a multiple of 256); the two phases
 * kda_fwd_chunk_local / kda_fwd_state_scan and kda_fwd_segment_map always need this much.
 * It is one record per (chunk, head): 92,160 bytes at d = 128 in bf16 (1,440 bytes per
 * token-head), i.e. it grows with T * H (about 377 MB for 4 x 4096 tokens x 16 heads, 6.0 GB for
 * 131,072 tokens x 32 heads).  A packed batch has N extra chunk slots (sequences need not start
 * on a chunk boundary).
 * varlen != 0 means cu_seqlens will be passed; then B must be 1 and T is the packed
 * token count.  Returns 0 for unsupported or invalid sizes.
 */
size_t kda_fwd_workspace_bytes(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                               int N, int varlen);

/*
 * Smallest workspace kda_fwd, kda_fwd_scalar_gate and kda_fwd_lowrank_gate accept for these
 * sizes (bytes).  Given less than kda_fwd_workspace_bytes, they run the chunks in windows: the
 * chunk-local phase and the state scan of one window, then the next (see kda_fwd), so the
 * workspace holds one window's records, plus the running state of every (sequence, head) when
 * no final_state buffer carries it (have_final_state == 0).  The minimum is one chunk per window.
 * Returns 0 for unsupported or invalid sizes.
 */
size_t kda_fwd_workspace_min_bytes(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                   int N, int varlen, int have_final_state);

/*
 * kda_fwd -- chunked prefill over a dense batch or a packed (varlen) batch.
 * Computes exactly the recurrence above for every sequence and head, with the chunkwise
 * parallel form (chunks of 64 tokens restarting at each sequence start) that the
 * yeyulingfeng page's KDA section names and the post-114 blog's chapter 3 describes
 * (parallel inside a chunk, serial across chunks).
 *
 *   io            KDA_F32 or KDA_BF16 (dtype of q, k, v, o)
 *   B, T, H       dense: B sequences of T tokens each; varlen: B = 1, T = cu_seqlens[N]
 *   d_k, d_v      head sizes; supported: d_k == d_v in {64, 128}
 *   cu_seqlens    NULL for dense; else device int32 [N + 1], cu_seqlens[0] = 0,
 *                 non-decreasing, cu_seqlens[N] = T (zero-length sequences allowed)
 *   N             number of sequences (dense: must equal B)
 *   q, k          [B, T, H, d_k] io dtype (q and k are expected L2-normalised per head)
 *   v             [B, T, H, d_v] io dtype
 *   g             [B, T, H, d_k] fp32, log of the per-channel forget gate (finite, <= 0)
 *   beta          [B, T, H] fp32, write strength
 *   scale         multiplies the read-out
 *   initial_state [N, H, d_k, d_v] fp32 or NULL (zero state)
 *   final_state   [N, H, d_k, d_v] fp32 or NULL (not written); may alias initial_state
 *   o             [B, T, H, d_v] io dtype, written for every token; must not alias inputs
 *   workspace     device buffer of at least kda_fwd_workspace_min_bytes(...) bytes (16-byte
 *                 aligned), reused freely by the library during the call.  The chunks run in
 *                 windows of Wc chunk indices: a dense batch takes chunks [w Wc, (w + 1) Wc) of
 *                 every sequence in window w, a packed batch the chunks whose first token lies in
 *                 [64 w Wc, 64 (w + 1) Wc).  With kda_fwd_workspace_bytes(...) bytes or more
 *                 all chunks run in one window; with less, Wc is as large as the workspace
 *                 allows.  Results are bitwise the same for any window size on one device (the
 *                 chunks and their arithmetic do not change, only when each is formed), and equal
 *                 to kda_fwd_chunk_local + kda_fwd_state_scan.
 *   Returns KDA_ERR_WORKSPACE when workspace is NULL or smaller than the minimum.
 */
kda_status_t kda_fwd(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                     const int32_t *cu_seqlens, int N,
                     const void *q, const void *k, const void *v,
                     const float *g, const float *beta, float scale,
                     const float *initial_state, float *final_state,
                     void *o, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * The two phases of kda_fwd, for callers that schedule or time them separately.
 * kda_fwd(...) is exactly kda_fwd_chunk_local(...) followed by kda_fwd_state_scan(...) on the
 * same stream with the same workspace; arguments have the meaning given for kda_fwd.
 *   kda_fwd_chunk_local: per (chunk, head), fully parallel -- cumulative log-decay, decayed
 *     Gram matrices, the UT transform of the chunk and the WY factors; results go to the
 *     workspace only.
 *   kda_fwd_state_scan: per (sequence, head), serial over the chunks -- propagates the state,
 *     writes o and final_state.  Reads what kda_fwd_chunk_local left in the workspace.
 */
kda_status_t kda_fwd_chunk_local(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                 const int32_t *cu_seqlens, int N,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);
kda_status_t kda_fwd_state_scan(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                const int32_t *cu_seqlens, int N, float scale,
                                const float *initial_state, float *final_state, void *o,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_fwd_scalar_gate -- kda_fwd for a forget gate shared by all key channels of a head:
 * alpha_t = exp(g_t) * (1, ..., 1) with one g per token and head (the Gated DeltaNet case,
 * blog post-114 chapter 3, where the gate is one scalar for all channels; chapter 4 contrasts
 * it with the per-channel gate of KDA), or alpha_t = 1 (DeltaNet, chapter 3) when g is NULL.
 * The recurrence is the operator's above with that alpha, decay first (the course page's
 * section 3 order; the chapter's Gated DeltaNet listing reads the memory before the decay,
 * which this library does not follow).  Equal to kda_fwd with g broadcast over d_k, and
 * faster: the decay leaves the channel sums of the chunk's Gram matrices.
 *
 *   g     [B, T, H] fp32 (log alpha per token and head, finite, <= 0), or NULL (alpha = 1)
 *   all other arguments, layouts, the workspace (kda_fwd_workspace_bytes) and the error
 *   behaviour are those of kda_fwd.
 */
kda_status_t kda_fwd_scalar_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                 const int32_t *cu_seqlens, int N,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, float scale,
                                 const float *initial_state, float *final_state,
                                 void *o, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * kda_fwd_chunk_local_scalar_gate -- the chunk-local phase of kda_fwd_scalar_gate alone (same
 * arguments, g [B, T, H] or NULL).  Its workspace records have the layout of kda_fwd_chunk_local's,
 * so kda_fwd_state_scan and kda_fwd_segment_map take them: kda_fwd_scalar_gate(...) is exactly
 * this call followed by kda_fwd_state_scan(...) on the same stream and workspace.
 */
kda_status_t kda_fwd_chunk_local_scalar_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                             const int32_t *cu_seqlens, int N,
                                             const void *q, const void *k, const void *v,
                                             const float *g, const float *beta,
                                             void *workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/*
 * Low-rank gate.  The page "Kimi K3 注意力三件套" (KDA section) says the per-channel alpha comes
 * from a low-rank down-up projection of the layer input x, and beta is one scalar; blog post-114
 * has beta = sigmoid(w_beta(x)) (chapter 3) and a gate per head and channel computed from x
 * (chapter 4).  The pages give no nonlinearity for alpha; the one used here is
 *     z      = x W_down^T                         rank r, shared by all heads
 *     log a  = g = -softplus(z W_up^T + b)        per (token, head, key channel), so 0 < alpha < 1
 *     beta   = sigmoid(x w_beta^T)                per (token, head)
 * Weights use the [out, in] layout.  bf16 operands, fp32 arithmetic; z is stored in bf16.
 */

/*
 * kda_gate -- the gate prologue for Ntok tokens: writes z and beta, and g when g != NULL.
 * The g it writes is bitwise the one kda_fwd_lowrank_gate forms internally from the same z.
 *
 *   io      KDA_BF16 (x, weights and z); anything else returns KDA_ERR_UNSUPPORTED
 *   x       [Ntok, Dm] bf16 (Dm a multiple of 32)
 *   w_down  [r, Dm] bf16 (r a multiple of 32, at most 128);  w_beta [H, Dm] bf16
 *   w_up    [H * d_k, r] bf16 and b_gate [H * d_k] fp32: required only when g != NULL
 *   z       [Ntok, r] bf16 out;  beta [Ntok, H] fp32 out;  g [Ntok, H, d_k] fp32 out or NULL
 *   Supported: d_k in {64, 128}.  All buffers device, 16-byte aligned, caller-owned.
 */
kda_status_t kda_gate(kda_dtype_t io, int Ntok, int Dm, int H, int d_k, int r,
                      const void *x, const void *w_down, const void *w_beta,
                      const void *w_up, const float *b_gate,
                      void *z, float *beta, float *g, hipStream_t stream);

/*
 * kda_fwd_lowrank_gate -- kda_fwd with the gate given by its low-rank form instead of g:
 * log(alpha) = -softplus(z W_up^T + b) is formed inside the chunk-local kernel, so the fp32 g
 * (d_k floats per token and head) is never written to or read from HBM.  Bitwise equal to
 * kda_gate(..., g) followed by kda_fwd(..., g, ...).
 *
 *   io      KDA_BF16 only (q, k, v, o, z, w_up); KDA_F32 returns KDA_ERR_UNSUPPORTED
 *   z       [B, T, r] bf16 (tokens laid out as q's);  r a multiple of 32, at most 128
 *   w_up    [H * d_k, r] bf16;  b_gate [H * d_k] fp32
 *   all other arguments, layouts, the workspace (kda_fwd_workspace_bytes) and the error
 *   behaviour are those of kda_fwd.
 */
kda_status_t kda_fwd_lowrank_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                  const int32_t *cu_seqlens, int N,
                                  const void *q, const void *k, const void *v,
                                  const void *z, int r, const void *w_up, const float *b_gate,
                                  const float *beta, float scale,
                                  const float *initial_state, float *final_state,
                                  void *o, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * kda_fwd_chunk_local_lowrank_gate -- the chunk-local phase of kda_fwd_lowrank_gate alone (same
 * arguments and checks).  As for kda_fwd_chunk_local_scalar_gate, its records feed
 * kda_fwd_state_scan and kda_fwd_segment_map, and kda_fwd_lowrank_gate(...) is exactly this call
 * followed by kda_fwd_state_scan(...).
 */
kda_status_t kda_fwd_chunk_local_lowrank_gate(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                              const int32_t *cu_seqlens, int N,
                                              const void *q, const void *k, const void *v,
                                              const void *z, int r, const void *w_up, const float *b_gate,
                                              const float *beta, void *workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/*
 * Segment maps (context parallelism).  Blog post-114, chapter 3: the chunked form computes
 * each block's contribution in parallel and merges the blocks into the state one after the
 * other; K3's KCP carries this across devices.  Taking a device's segment of a sequence as one
 * block, its contribution is the affine map the recurrence applies to the state entering it:
 *     S_out = A S_in + B,   A = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t)   (latest on the left)
 *                           B = the state reached from S_in = 0.
 * A caller that splits one sequence into P segments (packed as the sequences of a varlen batch,
 * cu_seqlens = the segment boundaries) runs kda_fwd_chunk_local and kda_fwd_segment_map on all
 * segments at once, chains the incoming states with kda_state_combine (S_in of segment j + 1 =
 * A_j S_in(j) + B_j, P - 1 serial hops), and finishes with kda_fwd_state_scan from those
 * incoming states, which writes every o and the final state.  The result equals kda_fwd over
 * the whole sequence up to fp32 rounding of the states at the segment boundaries.
 */

/*
 * kda_fwd_segment_map -- the affine map (A, B) of every (sequence, head) chain of a batch, from
 * the records kda_fwd_chunk_local left in the workspace (same sizes, cu_seqlens and workspace).
 *
 *   transition  [N, H, d_k, d_k] fp32 out: A, element (i, j) maps key channel j of S_in to i
 *   offset      [N, H, d_k, d_v] fp32 out: B, in the state layout
 *   The two must not overlap.  A zero-length sequence gives A = I, B = 0.  Other arguments,
 *   the workspace (kda_fwd_workspace_bytes) and the error behaviour are those of kda_fwd.
 */
kda_status_t kda_fwd_segment_map(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                                 const int32_t *cu_seqlens, int N,
                                 float *transition, float *offset,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_state_combine -- one hop between segments, for `count` maps at once (fp32, fixed order):
 *     state_out[c] = transition[c] state_in[c] + offset[c]
 *   transition  [count, d_k, d_k] fp32;  state_in, offset, state_out [count, d_k, d_v] fp32
 *   offset may be NULL (taken as zero): with state_in = the transition of an earlier segment this
 *   composes two maps, (A2, B2) after (A1, B1) = (A2 A1, A2 B1 + B2), the step of a prefix over
 *   segments taken as a tree (log2 P rounds) instead of a chain.
 *   Supported: d_k == d_v in {64, 128}.  state_out must not overlap transition or state_in; it
 *   may be offset itself (exactly, not a shifted overlap).  count == 0 does nothing.
 */
kda_status_t kda_state_combine(int count, int d_k, int d_v, const float *transition,
                               const float *state_in, const float *offset, float *state_out,
                               hipStream_t stream);

/*
 * Block AttnRes.  Blog post-114, chapter 6 (the block AttnRes listing): the outputs of the
 * earlier blocks of layers (and the current, partial block) are stacked, normalised into keys,
 * scored against the layer's projection weight w, and mixed with the softmax of the scores over
 * the blocks; the page "Kimi K3 注意力三件套" (AttnRes section) adds that the weights sum to one,
 * and that at inference the scoring of the stored blocks is done once for all layers of a block
 * (phase 1), each layer then merging its partial block by an online-softmax step (phase 2):
 *     h[t] = sum_n softmax_n( w . norm(V_n[t]) ) V_n[t],   norm(x) = x / sqrt(mean(x^2) + eps)
 * (an RMS norm without learned scale: a scale would only multiply w element-wise).
 * Block outputs, queries and results are bf16 ([T, d] each, row-major); arithmetic is fp32.
 * `blocks` is a HOST array of n device pointers.  Device buffers are 16-byte aligned, except the
 * fp32 lse arrays (4-byte aligned, so a layer's row of a [L, T] array can be passed).  Supported: n <= 16 blocks, L <= 16 layers,
 * d a multiple of 512 up to 4096; io = KDA_BF16 only.  eps >= 0.
 */

/*
 * kda_attnres -- one-shot read-out of one layer over n blocks (the last may be the partial
 * block): h [T, d].  h may alias one of the blocks (each element is read before it is written).
 */
kda_status_t kda_attnres(kda_dtype_t io, int n, int T, int d, const void *const *blocks,
                         const void *w, float eps, void *h, hipStream_t stream);

/*
 * kda_attnres_inter -- phase 1 for L layers over n stored blocks, each block read once:
 *   o_bar  [L, T, d] bf16 out: per layer the softmax-weighted mean over the blocks
 *   lse    [L, T] fp32 out or NULL: per layer the log-sum-exp of the scores
 *   W      [L, d] bf16: the layers' queries
 *   workspace: device, kda_attnres_inter_workspace_bytes(n, L, T) bytes, caller-owned.
 * o_bar must not overlap the blocks.
 */
size_t kda_attnres_inter_workspace_bytes(int n, int L, int T);
kda_status_t kda_attnres_inter(kda_dtype_t io, int n, int L, int T, int d, const void *const *blocks,
                               const void *W, float eps, void *o_bar, float *lse,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_attnres_merge -- phase 2 for one layer: merges the partial block [T, d] into that layer's
 * phase-1 result (o_bar [T, d], lse [T]: one layer's slices of kda_attnres_inter's outputs):
 *     m = max(lse, s),  s = w . norm(partial),
 *     h = (e^{lse-m} o_bar + e^{s-m} partial) / (e^{lse-m} + e^{s-m}),
 * equal to kda_attnres over the stored blocks and the partial block.  lse = -inf (no stored
 * block) gives h = partial.  h may alias partial or o_bar.
 */
kda_status_t kda_attnres_merge(kda_dtype_t io, int T, int d, const void *partial, const void *w,
                               float eps, const void *o_bar, const float *lse, void *h,
                               hipStream_t stream);

/*
 * kda_decode_step -- one token of the recurrence for N independent sequences, in place.
 * The state stays resident in HBM; each call reads and rewrites it once
 * (the fixed-size state of the course page's section 2 makes each step O(1) in the
 * context length).
 *
 *   q, k   [N, H, d_k] io dtype;  v [N, H, d_v] io dtype
 *   g      [N, H, d_k] fp32 (log alpha);  beta [N, H] fp32
 *   state  [N, H, d_k, d_v] fp32, read then overwritten with the updated state
 *   o      [N, H, d_v] io dtype (read-out with the updated state)
 *   Supported: d_k, d_v in {64, 128}.
 */
kda_status_t kda_decode_step(kda_dtype_t io, int N, int H, int d_k, int d_v,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float scale,
                             float *state, void *o, hipStream_t stream);

/*
 * kda_prep -- q/k prologue: short causal depthwise convolution, SiLU, L2 norm per head.
 * (yeyulingfeng page, KDA section: short causal convolution then L2 normalisation;
 * post-114 blog chapter 3: normalize(silu(.)).)  Called once for q and once for k.
 *     c' = sum_{tau=0}^{W-1} conv_w[c, tau] * x_{t-(W-1)+tau}[c]   (x = 0 before the
 *          first token of the sequence; tap W-1 is the current token; no bias)
 *     y  = silu(c') / max(||silu(c')||_2 over the d channels of the head, 1e-12)
 *
 *   x, y        [B, T, H, d] io dtype (y must not alias x)
 *   cu_seqlens  NULL (each of the B rows is one sequence) or device int32 [N + 1] with B = 1
 *   conv_w      [H * d, W] fp32 device buffer;  W in 1..8
 *   Supported: d in {64, 128}.
 */
kda_status_t kda_prep(kda_dtype_t io, int B, int T, int H, int d,
                      const int32_t *cu_seqlens, int N,
                      const void *x, const float *conv_w, int W, void *y,
                      hipStream_t stream);

/*
 * kda_fwd_noalloc -- kda_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments as kda_fwd,
 * without the workspace: the library uses its own fixed device scratch of
 * KDA_NOALLOC_SCRATCH_BYTES per GPU instead (a device array that each GPU the library runs on
 * holds until the process ends), running the chunks in windows as large as that scratch allows.
 * Nothing is allocated or freed.  Returns KDA_ERR_TOO_LARGE, before launching anything, when
 * even one chunk per window (plus the running states, if final_state is NULL) does not fit,
 * i.e. when kda_fwd_workspace_min_bytes(...) > KDA_NOALLOC_SCRATCH_BYTES.  All calls on one GPU
 * share that GPU's scratch: calls that overlap on one GPU (different streams without ordering
 * between them, or different host threads) race and must not be issued.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
kda_status_t kda_fwd_noalloc(kda_dtype_t io, int B, int T, int H, int d_k, int d_v,
                             const int32_t *cu_seqlens, int N,
                             const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float scale,
                             const float *initial_state, float *final_state,
                             void *o, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
