// kda_chunk.hip -- chunked KDA prefill: a chunk-local kernel and a serial state-scan kernel.
//
// The pages state that deployment uses a chunkwise parallel form, the WY representation with
// a UT transform (page "Kimi K3 注意力三件套", KDA section), i.e. parallel work inside a chunk
// and a serial pass across chunks (blog post-114, chapter 3).  They leave out the algebra; the
// form used here follows from unrolling the course page's section-3 update over one chunk of
// C <= 64 tokens with incoming state S (per channel G_t = sum_{s<=t} g_s, gamma = G_last):
//
//   Akk[t,j] = beta_t sum_c k_tc k_jc e^{G_tc - G_jc}   (j < t)      Tm = (I + Akk)^-1
//   Aqk[t,j] =        sum_c q_tc k_jc e^{G_tc - G_jc}   (j <= t)     T' = Tm Diag(beta)
//   W = T' (K * e^G),  U = T' V,  Qh = Q * e^G,  Kh = K * e^{gamma - G}
//   Ud = U - W S;   O = scale (Qh S + Aqk Ud);   S <- Diag(e^gamma) S + Kh^T Ud
//
// Kernel 1 (chunk_local_kernel): one 256-thread workgroup per (chunk, head), fully parallel.
//   It builds the cumulative log-decay in LDS, the two decayed Gram matrices, the UT
//   transform Tm by blocked forward substitution, and writes W, U, Qh, Kh^T, Aqk and
//   e^gamma to the workspace, laid out as ready-to-load MFMA operand fragments.
// Kernel 2 (chunk_scan_kernel): per (sequence, head, 16 value columns) a set of 2 or 4 waves, each
//   keeping a slice of the d_k x 16 fp32 state in MFMA accumulator registers, walks the chunks.
//
// Exponent safety.  Every e^{x} is evaluated with x <= 0 or with |x| bounded by a checked
// half-span: the Gram matrices use 16-token sub-blocks with the sub-block's middle row m as
// reference (row factor e^{G_i - G_m}, column factor e^{G_m - G_j}, and for blocks I > J the
// per-channel bridge e^{G_mI - G_mJ} <= 1).  If some |G_i - G_m| exceeds 115 (log2 units) the
// chunk takes an exact element-wise fallback instead.
//
// Precision (bf16 inputs).  The Gram operands, Tm, S and Ud enter the MFMAs as hi + lo bf16
// pairs (about 16 significant bits); U is kept at 24 bits (see pack_u24); Kh^T and Aqk enter the
// state update and the read-out as their bf16 plane plus the remainder in fp8 with a scale per
// channel or per token row (see split_bf16_fp8), the remainder times Ud in bf8 under a
// power-of-two scale per value column (see ut_and_outputs).  q, k, v are used as stored (exact).
// The fp32 path uses fp32 MFMAs and fp32 U throughout.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// ------------------------------------------------------------------ operand precision
template <bool BF16> struct Prec;
template <> struct Prec<true> {
    using Plain = FragB;
    using Split = Frag2;
    static constexpr int kPlainPlanes = 1;
    static constexpr int kSplitPlanes = 2;
    static __device__ __forceinline__ Plain plain(const float *x) { return make_fragB(x); }
    static __device__ __forceinline__ Split split(const float *x) { return make_frag2(x); }
    static __device__ __forceinline__ void st_plain(char *base, int, int f, int lane, const Plain &p) {
        reinterpret_cast<bf16x8 *>(base)[f * 64 + lane] = p.h;
    }
    static __device__ __forceinline__ Plain ld_plain(const char *base, int, int f, int lane) {
        return FragB{reinterpret_cast<const bf16x8 *>(base)[f * 64 + lane]};
    }
    static __device__ __forceinline__ void st_split(char *base, int nf, int f, int lane, const Split &p) {
        reinterpret_cast<bf16x8 *>(base)[f * 64 + lane] = p.h;
        reinterpret_cast<bf16x8 *>(base + (size_t)nf * 1024)[f * 64 + lane] = p.l;
    }
    static __device__ __forceinline__ Split ld_split(const char *base, int nf, int f, int lane) {
        Frag2 r;
        r.h = reinterpret_cast<const bf16x8 *>(base)[f * 64 + lane];
        r.l = reinterpret_cast<const bf16x8 *>(base + (size_t)nf * 1024)[f * 64 + lane];
        return r;
    }
};
template <> struct Prec<false> {
    using Plain = FragF;
    using Split = FragF;
    static constexpr int kPlainPlanes = 2;
    static constexpr int kSplitPlanes = 2;
    static __device__ __forceinline__ Plain plain(const float *x) { return make_fragF(x); }
    static __device__ __forceinline__ Split split(const float *x) { return make_fragF(x); }
    static __device__ __forceinline__ void st_plain(char *base, int nf, int f, int lane, const FragF &p) {
        reinterpret_cast<f32x4 *>(base)[f * 64 + lane] = f32x4{p.v[0], p.v[1], p.v[2], p.v[3]};
        reinterpret_cast<f32x4 *>(base + (size_t)nf * 1024)[f * 64 + lane] = f32x4{p.v[4], p.v[5], p.v[6], p.v[7]};
    }
    static __device__ __forceinline__ FragF ld_plain(const char *base, int nf, int f, int lane) {
        const f32x4 a = reinterpret_cast<const f32x4 *>(base)[f * 64 + lane];
        const f32x4 b = reinterpret_cast<const f32x4 *>(base + (size_t)nf * 1024)[f * 64 + lane];
        return FragF{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
    }
    static __device__ __forceinline__ void st_split(char *base, int nf, int f, int lane, const FragF &p) {
        st_plain(base, nf, f, lane, p);
    }
    static __device__ __forceinline__ FragF ld_split(const char *base, int nf, int f, int lane) {
        return ld_plain(base, nf, f, lane);
    }
};

// ------------------------------------------------------------------ workspace layout
// Per (chunk slot, head): W, Qh fragments [tt][kb]; Kh^T fragments [rt][kb2]; Aqk fragments
// (6 lower ones; for bf16 the bf16 plane, then the low part in fp8 e4m3, 8 bytes per lane and
// fragment, scaled by 2^a per row, see split_bf16_fp8); e^gamma [D] and, for bf16, the scales 2^-a
// of the Kh^T low plane [D] and of the Aqk low plane [64] as bf16 and the exponents of the bf8 scale
// of Ud per value column [D] as int8 (see ut_and_outputs; together padded to 1 KB); U as
// accumulator tiles [jt][tt][lane] (f32x4; for bf16 the four values as 24-bit floats in three
// dwords, see pack_u24); for bf16, the low part of Kh^T [rt][kb2] (Kh^T minus its bf16 plane
// above) as fp8 e4m3 scaled by 2^a per channel, 8 bytes per lane.  Everything before U is read by
// every column tile of the chain and is staged in LDS by the state scan; U tile jt is read by
// column tile jt, the Kh^T low plane by each wave for its own state rows.
template <bool BF16, int D> struct WsLayout {
    static constexpr int NT = 4;           // 16-token tiles per chunk
    static constexpr int NKB = D / 32;     // 32-channel k-blocks
    static constexpr int NRT = D / 16;     // 16-channel tiles
    static constexpr int nW = NT * NKB, nQ = NT * NKB, nK = NRT * 2, nA = 6;
    static constexpr int PP = Prec<BF16>::kPlainPlanes, SP = Prec<BF16>::kSplitPlanes;
    static constexpr size_t offW = 0;
    static constexpr size_t offQ = offW + (size_t)nW * PP * 1024;
    static constexpr size_t offK = offQ + (size_t)nQ * PP * 1024;
    static constexpr size_t offA = offK + (size_t)nK * PP * 1024;
    static constexpr size_t offAl = offA + (size_t)nA * 1024;  // Aqk low plane (bf16)
    static constexpr size_t offE = offA + (size_t)nA * (BF16 ? 1024 + 512 : SP * 1024);
    static constexpr size_t offU = offE + 1024;
    static constexpr size_t offEl = offE + (size_t)D * 4;   // scales of the Kh^T low plane (bf16)
    static constexpr size_t offEa = offEl + (size_t)D * 2;  // scales of the Aqk low plane (bf16)
    static constexpr size_t offEs = offEa + (size_t)kChunk * 2;  // bf8 scale exponents of Ud's columns (bf16)
    static constexpr size_t uTile = BF16 ? 768 : 1024;   // bytes of one U accumulator tile
    static constexpr size_t offKl = offU + (size_t)NRT * NT * uTile;
    static constexpr size_t bytes = offKl + (BF16 ? (size_t)nK * 512 : 0);
    static_assert(D * 7 + kChunk * 2 <= 1024, "e^gamma and the low-plane scales fit their 1 KB slot");
};

// The bf16 plane of nf fragments (8 values per lane each) and the remainder lo = x - bf16(x) in
// fp8 e4m3, scaled by 2^a, where a is shared by the lanes r16 + 16 g (one row of an A operand: a
// channel of Kh^T, a token of Aqk) and chosen so that the largest |lo| of those lanes' fragments
// lands in [64, 128), within the e4m3 range whichever e4m3 variant the hardware uses.  Returns the
// scale 2^-a by which a product with the fp8 plane is multiplied back.  A product then takes x as
// bf16 plane x (the other operand's hi + lo) plus fp8 plane x (the other operand in bf8): a single
// bf16 rounding puts a relative error of 2^-9 on every term, the two planes about 2^-13.
template <int NF>
__device__ __forceinline__ float split_bf16_fp8(const float (&x)[NF][8], uint4 (&hi)[NF], uint2 (&lo8)[NF]) {
    float lo[NF][8], m = 0.f;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        uint32_t hw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t h = pk_bf16(x[f][2 * p], x[f][2 * p + 1]);
            hw[p] = h;
            lo[f][2 * p] = x[f][2 * p] - __uint_as_float(h << 16);
            lo[f][2 * p + 1] = x[f][2 * p + 1] - __uint_as_float(h & 0xffff0000u);
            m = fmaxf(m, fmaxf(fabsf(lo[f][2 * p]), fabsf(lo[f][2 * p + 1])));
        }
        hi[f] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    // a = 6 - floor(log2 m), within [-126, 126] (m = 0 or tiny: the low part is zero or negligible)
    const int em = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;
    const int a = m > 0.f ? min(126, max(-126, 6 - em)) : 0;
    const float up = __uint_as_float((uint32_t)(a + 127) << 23);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[f][0] * up, lo[f][1] * up, 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[f][2] * up, lo[f][3] * up, w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[f][4] * up, lo[f][5] * up, 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(lo[f][6] * up, lo[f][7] * up, w1, true);
        lo8[f] = make_uint2((uint32_t)w0, (uint32_t)w1);
    }
    return __uint_as_float((uint32_t)(127 - a) << 23);
}
// a power of two (or any value whose low 16 bits are zero) as bf16 bits
__device__ __forceinline__ uint16_t bf16_exact(float x) { return (uint16_t)(__float_as_uint(x) >> 16); }

// The two Kh^T fragments (row tile rt, token k-blocks 0 and 1) of a record.  fp32: as they are.
// bf16: the bf16 plane and the fp8 low plane of split_bf16_fp8 with one scale per channel; the
// state update takes Kh^T as bf16 plane x Ud (hi + lo) plus low plane x Ud in bf8 (Kh^T
// single-rounded to bf16 puts a relative error of 2^-9 on every term of Kh^T Ud, which the
// state carries from chunk to chunk).  A channel's 64 tokens sit in this lane's two fragments and
// in the lanes r16 + 16 g of the other lane groups.
template <bool BF16, int D>
__device__ __forceinline__ void st_kh(char *wsb, int rt, int lane, const float (&kh)[2][8]) {
    using L = WsLayout<BF16, D>;
    if constexpr (BF16) {
        uint4 hi[2];
        uint2 lo8[2];
        const float down = split_bf16_fp8<2>(kh, hi, lo8);
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            reinterpret_cast<uint4 *>(wsb + L::offK)[(rt * 2 + kb2) * 64 + lane] = hi[kb2];
            reinterpret_cast<uint2 *>(wsb + L::offKl)[(rt * 2 + kb2) * 64 + lane] = lo8[kb2];
        }
        if (lane < 16) reinterpret_cast<uint16_t *>(wsb + L::offEl)[16 * rt + lane] = bf16_exact(down);
    } else {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) Prec<false>::st_plain(wsb + L::offK, L::nK, rt * 2 + kb2, lane, make_fragF(kh[kb2]));
    }
}

// U of the bf16 path in 24-bit floats: fp32 rounded to nearest even at 15 stored mantissa bits
// (relative error 2^-16, far below what the bf16 W of U - W S brings), four values in the three
// high bytes of each, three dwords per lane.  v_perm_b32 takes bytes 0-3 from its second operand
// and 4-7 from its first; selector 0x0c gives a zero byte.
struct U24 { uint32_t w0, w1, w2; };
__device__ __forceinline__ U24 pack_u24(f32x4 x) {
    uint32_t r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t u = __float_as_uint(x[e]);
        r[e] = u + 0x7fu + ((u >> 8) & 1u);
    }
    return U24{__builtin_amdgcn_perm(r[1], r[0], 0x05030201u), __builtin_amdgcn_perm(r[2], r[1], 0x06050302u),
               __builtin_amdgcn_perm(r[3], r[2], 0x07060503u)};
}
__device__ __forceinline__ f32x4 unpack_u24(const U24 &w) {
    return f32x4{__uint_as_float(__builtin_amdgcn_perm(w.w0, w.w0, 0x0201000cu)),
                 __uint_as_float(__builtin_amdgcn_perm(w.w1, w.w0, 0x0504030cu)),
                 __uint_as_float(__builtin_amdgcn_perm(w.w2, w.w1, 0x0403020cu)), __uint_as_float(w.w2 & 0xffffff00u)};
}

// lower Aqk fragment index of (token tile tt, token k-block kb2), kb2 <= tt / 2
__device__ __forceinline__ int aidx(int tt, int kb2) { return tt < 2 ? tt : 2 + 2 * (tt - 2) + kb2; }

__device__ __forceinline__ int mid_row(int I) { return 16 * I + 8; }

// pair p -> (I, J), I >= J, in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
__device__ __forceinline__ void pair_ij(int p, int &I, int &J) {
    I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
    J = p - I * (I + 1) / 2;
}
// off-diagonal pair (I > J) -> bridge index in (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ __forceinline__ int bridge_idx(int I, int J) { return (I - 1) * I / 2 + J; }

// ------------------------------------------------------------------ chunk addressing
// The prefill runs its chunks in windows (one window when the workspace holds every chunk's
// record).  Dense batch: window w holds the chunks c in [w Wc, (w + 1) Wc) of every sequence,
// sequence n's chunk c at record n Wc + (c - w Wc).  Packed batch: window w holds the chunks whose
// first token t0 has floor(t0 / 64) in [w Wc, (w + 1) Wc); the chunk's slot
// n + floor(cu[n] / 64) + c = n + floor(t0 / 64) lies in [w Wc, (w + 1) Wc + N), and its record is
// slot - w Wc.  Slots are injective, so every chunk has one record and no prefix pass is needed.
struct Window {
    int w;      // window index
    long Wc;    // chunk indices per window
    long nrec;  // records of this window (chunk-local grid = nrec * H workgroups)
};

struct ChunkPos {
    bool valid;
    int n, c, Cc;
    long tok0;
};
// Largest n in [0, N) with n + cu[n] / 64 <= slot (strictly increasing in n).
__device__ __forceinline__ ChunkPos locate_packed(long slot, const int32_t *cu, int N) {
    ChunkPos p;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long)mid + cu[mid] / kChunk <= slot) lo = mid; else hi = mid - 1;
    }
    p.n = lo;
    const long s = cu[lo], L = (long)cu[lo + 1] - s;
    p.c = (int)(slot - (lo + s / kChunk));
    p.valid = p.c >= 0 && (long)p.c * kChunk < L;
    p.tok0 = s + (long)p.c * kChunk;
    p.Cc = p.valid ? (int)min((long)kChunk, L - (long)p.c * kChunk) : 0;
    return p;
}

// (record, head, chunk) of chunk-local workgroup `id` in window `win`.  The grid runs in reverse
// consumption order: the chunks the state scan reads first are written last, so they are the
// most likely to still be in the memory-side cache.
__device__ __forceinline__ ChunkPos local_chunk(long id, const int32_t *cu, int N, int T, int H, const Window &win,
                                                long &rec, int &h) {
    if (cu) {
        rec = win.nrec - 1 - id / H;
        h = (int)(id % H);
        ChunkPos p = locate_packed((long)win.w * win.Wc + rec, cu, N);
        const long f = p.tok0 / kChunk;  // window of the chunk
        p.valid = p.valid && f >= (long)win.w * win.Wc && f < (long)(win.w + 1) * win.Wc;
        return p;
    }
    const long ncs = ((long)T + kChunk - 1) / kChunk;
    const long c0 = (long)win.w * win.Wc, ncw = min(win.Wc, ncs - c0);  // chunks of this window
    const long per_c = (long)N * H;
    const long cl = ncw - 1 - id / per_c, rem = id % per_c;
    h = (int)(rem % H);
    ChunkPos p;
    p.n = (int)(rem / H);
    p.c = (int)(c0 + cl);
    rec = (long)p.n * win.Wc + cl;
    p.tok0 = (long)p.n * T + (long)p.c * kChunk;
    p.Cc = (int)min((long)kChunk, (long)T - (long)p.c * kChunk);
    p.valid = true;
    return p;
}

// ------------------------------------------------------------------ kernel 1: chunk-local
// The 8 k-slot values of one LDS row for lane group grp: elements 32 kb + kslot(grp, s), read
// as two runs of 4 consecutive elements (rows and runs are 16-byte aligned for fp32, 8-byte for
// bf16).
__device__ __forceinline__ void ld_kslots(const float *row, int kb, int grp, float *out) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(row + 32 * kb + 4 * grp);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(row + 32 * kb + 16 + 4 * grp);
#pragma unroll
    for (int u = 0; u < 4; ++u) { out[u] = a[u]; out[4 + u] = b[u]; }
}
__device__ __forceinline__ void ld_kslots(const uint16_t *row, int kb, int grp, float *out) {
    const f32x4 a = load4(row + 32 * kb + 4 * grp);
    const f32x4 b = load4(row + 32 * kb + 16 + 4 * grp);
#pragma unroll
    for (int u = 0; u < 4; ++u) { out[u] = a[u]; out[4 + u] = b[u]; }
}

template <bool BF16, int D> struct alignas(16) ChunkSmem {
    using TIO = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int GS = D + 4, KS = D + 8, VS = kChunk + 8, AS = kChunk + 4;
    static constexpr int CQ = D / 4;          // channel quads
    static constexpr int RG = 256 / CQ;       // row groups in the load / cumulative-sum layout
    static constexpr int RPG = kChunk / RG;   // rows per group
    union {
        float G[kChunk][GS];  // cumulative log2-decay, then
        float T[kChunk][AS];  // the UT transform Tm
    } g;
    union {
        struct { TIO K[kChunk][KS]; TIO Q[kChunk][KS]; } in;
        struct { float Akk[kChunk][AS]; float Aqk[kChunk][AS]; } a;
        TIO VT[D][VS];        // V transposed (VT[j][t]), written once Akk and Aqk are dead
    } kq;
    float tot[RG][D];         // per row-group sums of the log-decay (cumulative-sum carries)
    float bridge[6][D];
    float beta[kChunk];
    int flag;
};

// Four consecutive io elements kept in their storage form (bf16 bits or fp32).
template <typename TIO> struct Raw4;
template <> struct Raw4<uint16_t> {
    uint2 w;
    static __device__ __forceinline__ Raw4 load(const uint16_t *p) { return Raw4{*reinterpret_cast<const uint2 *>(p)}; }
    static __device__ __forceinline__ Raw4 zero() { return Raw4{make_uint2(0u, 0u)}; }
    __device__ __forceinline__ void store(uint16_t *p) const { *reinterpret_cast<uint2 *>(p) = w; }
    __device__ __forceinline__ uint16_t elem(int u) const {
        const uint32_t x = (u < 2) ? w.x : w.y;
        return (uint16_t)((u & 1) ? (x >> 16) : (x & 0xffffu));
    }
};
template <> struct Raw4<float> {
    f32x4 w;
    static __device__ __forceinline__ Raw4 load(const float *p) { return Raw4{*reinterpret_cast<const f32x4 *>(p)}; }
    static __device__ __forceinline__ Raw4 zero() { return Raw4{zero4()}; }
    __device__ __forceinline__ void store(float *p) const { *reinterpret_cast<f32x4 *>(p) = w; }
    __device__ __forceinline__ float elem(int u) const { return w[u]; }
};

// Phases shared by the chunk-local kernels once Akk (beta applied, strictly lower) and Aqk
// (lower, incl. the diagonal) are in LDS: the UT transform Tm = (I + Akk)^-1, the Aqk
// fragments, V^T, and W = T' X, U = T' V.  `vv` holds this thread's V rows (layout of the load
// phase: rows rg*RPG.., channels c4..c4+3); `Xf` the X^T = (K e^G)^T fragments of k-block `wave`.
template <bool BF16, int D, int RPG, typename SM>
__device__ __forceinline__ void ut_and_outputs(SM &sm, const Raw4<typename SM::TIO> (&vv)[RPG],
                                               const typename Prec<BF16>::Plain (&Xf)[2][2], char *wsb, int rg,
                                               int c4) {
    using TIO = typename SM::TIO;
    using P = Prec<BF16>;
    using L = WsLayout<BF16, D>;
    using Plain = typename P::Plain;
    using Split = typename P::Split;
    constexpr int NKB = L::NKB, NRT = L::NRT;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    char *wsW = wsb + L::offW, *wsA = wsb + L::offA;
    float *wsU = reinterpret_cast<float *>(wsb + L::offU);
    // ---------------- phase 4: Tm = (I + Akk)^-1 (unit lower triangular), fp32
    if (wave == 0) {  // 16x16 diagonal blocks: lane owns column j of block b
        const int b = lane >> 4, j = lane & 15;
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc += sm.kq.a.Akk[16 * b + i][16 * b + m] * tc[m];
            tc[i] = i == j ? 1.f : (i < j ? 0.f : -acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.g.T[16 * b + i][16 * b + j] = tc[i];
    }
    __syncthreads();
    for (int I = 1; I < 4; ++I) {  // block rows: T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ
        const int J = wave;
        if (J < I) {
            f32x4 x = zero4();
            for (int M = J; M < I; ++M) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    x = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.kq.a.Akk[16 * I + r16][16 * M + 4 * grp + s],
                                                             sm.g.T[16 * M + 4 * grp + s][16 * J + r16], x, 0, 0, 0);
            }
            f32x4 y = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.g.T[16 * I + r16][16 * I + 4 * grp + s], x[s], y, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.g.T[16 * I + 4 * grp + e][16 * J + r16] = -y[e];
        }
        __syncthreads();
    }

    // ---------------- phase 5: Aqk fragments; then V^T into the dead Akk/Aqk region;
    // W = T' X and U = T' V.
    if constexpr (BF16) {  // Aqk fragments of token tile `wave` (token k-blocks 0 .. wave / 2)
        const int tt = wave, t = 16 * tt + r16;
        float vals[2][8];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            if (kb2 <= tt / 2) {
                ld_kslots(&sm.kq.a.Aqk[t][0], kb2, grp, vals[kb2]);
#pragma unroll
                for (int s = 0; s < 8; ++s)  // causal mask, incl. the diagonal (entries above were never written)
                    if (32 * kb2 + kslot(grp, s) > t) vals[kb2][s] = 0.f;
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) vals[kb2][s] = 0.f;
            }
        }
        uint4 hi[2];
        uint2 lo8[2];
        const float down = split_bf16_fp8<2>(vals, hi, lo8);  // one scale per token row
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
            if (kb2 <= tt / 2) {
                reinterpret_cast<uint4 *>(wsA)[aidx(tt, kb2) * 64 + lane] = hi[kb2];
                reinterpret_cast<uint2 *>(wsb + L::offAl)[aidx(tt, kb2) * 64 + lane] = lo8[kb2];
            }
        if (lane < 16) reinterpret_cast<uint16_t *>(wsb + L::offEa)[t] = bf16_exact(down);
    } else {
        for (int f = wave; f < 6; f += 4) {  // Aqk fragments
            const int tt = f < 2 ? f : 2 + (f - 2) / 2, kb2 = f < 2 ? 0 : (f - 2) % 2;
            const int t = 16 * tt + r16;
            float vals[8];
            ld_kslots(&sm.kq.a.Aqk[t][0], kb2, grp, vals);
#pragma unroll
            for (int s = 0; s < 8; ++s)  // causal mask, incl. the diagonal (entries above were never written)
                if (32 * kb2 + kslot(grp, s) > t) vals[s] = 0.f;
            P::st_split(wsA, L::nA, f, lane, P::split(vals));
        }
    }
    __syncthreads();  // Akk, Aqk are dead from here on
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // channel c4 + u: RPG consecutive tokens, one vector store
        union { TIO e[RPG]; uint4 q[(RPG * sizeof(TIO) + 15) / 16]; uint2 d; } col;
#pragma unroll
        for (int r = 0; r < RPG; ++r) col.e[r] = vv[r].elem(u);
        TIO *dst = &sm.kq.VT[c4 + u][rg * RPG];
        if constexpr (RPG * sizeof(TIO) == 8) {
            *reinterpret_cast<uint2 *>(dst) = col.d;
        } else {
#pragma unroll
            for (int w = 0; w < (int)(RPG * sizeof(TIO) / 16); ++w) reinterpret_cast<uint4 *>(dst)[w] = col.q[w];
        }
    }
    __syncthreads();
    // T' = Tm Diag(beta) fragments; the same values serve as the A operand (row t, k = t')
    // of U and as the B operand (k = t', column t) of W^T.
    Split Tf[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int tt = f < 2 ? f : 2 + (f - 2) / 2, kb2 = f < 2 ? 0 : (f - 2) % 2;
        float vals[8], bv[8];
        ld_kslots(&sm.g.T[16 * tt + r16][0], kb2, grp, vals);
        ld_kslots(&sm.beta[0], kb2, grp, bv);
#pragma unroll
        for (int s = 0; s < 8; ++s)  // Tm is zero above its 16x16 diagonal blocks (never written)
            vals[s] = ((32 * kb2 + kslot(grp, s)) >> 4) <= tt ? vals[s] * bv[s] : 0.f;
        Tf[f] = P::split(vals);
    }
    for (int kb = wave; kb < NKB; kb += 4) {  // W fragments (tt, kb)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int kb2 = 0; kb2 <= tt / 2; ++kb2) acc[r2] = mfma(Xf[r2][kb2], Tf[aidx(tt, kb2)], acc[r2]);
            float vals[8] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3], acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
            P::st_plain(wsW, L::nW, tt * NKB + kb, lane, P::plain(vals));
        }
    }
    // bf16: for each value column, the exponent s that brings the chunk's largest |U| in the column
    // into [1, 2).  The state scan forms Ud in bf8 (for the fp8 low planes of Kh^T and Aqk) as
    // bf8(Ud 2^s) and scales the products back by 2^-s, so that Ud's bf8 form stays inside bf8's
    // normal range whatever the magnitude of v (Ud = U - W S is of U's order).
    for (int jt = wave; jt < NRT; jt += 4) {  // U tiles (jt, tt)
        Plain Vf[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            float vals[8];
            ld_kslots(&sm.kq.VT[16 * jt + r16][0], kb2, grp, vals);
            Vf[kb2] = P::plain(vals);
        }
        float um = 0.f;  // largest |U| of this lane's column (r16) over its rows
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb2 = 0; kb2 <= tt / 2; ++kb2) acc = mfma(Tf[aidx(tt, kb2)], Vf[kb2], acc);
            if constexpr (BF16) {
                reinterpret_cast<U24 *>(wsb + L::offU)[(jt * 4 + tt) * 64 + lane] = pack_u24(acc);
                um = fmaxf(um, fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])), fmaxf(fabsf(acc[2]), fabsf(acc[3]))));
            } else {
                reinterpret_cast<f32x4 *>(wsU)[(jt * 4 + tt) * 64 + lane] = acc;
            }
        }
        if constexpr (BF16) {
            um = fmaxf(um, __shfl_xor(um, 16));
            um = fmaxf(um, __shfl_xor(um, 32));
            const int eu = (int)((__float_as_uint(um) >> 23) & 0xffu) - 127;  // floor(log2 um), normal um
            const int su = um > 0.f ? min(126, max(-126, -eu)) : 0;
            if (lane < 16) reinterpret_cast<int8_t *>(wsb + L::offEs)[16 * jt + lane] = (int8_t)su;
        }
    }
}

// The low-rank gate as the chunk-local kernel receives it (see LR below).
struct LowRankGate {
    const uint16_t *z;     // [tokens, r] bf16 bits
    const uint16_t *w_up;  // [H * d, r] bf16 bits
    const float *b;        // [H * d]
    int r;                 // multiple of 32, at most 128
};

// LR: the log-decay is not read from memory but formed here from the low-rank gate,
// g = -softplus(z W_up^T + b) (one bf16 MFMA per 16x16 tile and 32 rank indices), so the fp32
// g never travels through HBM.  The values are bitwise those the gate prologue writes out.
template <bool BF16, int D, bool LR = false>
__global__ void __launch_bounds__(256, 2)
chunk_local_kernel(const typename ChunkSmem<BF16, D>::TIO *__restrict__ q,
                   const typename ChunkSmem<BF16, D>::TIO *__restrict__ k,
                   const typename ChunkSmem<BF16, D>::TIO *__restrict__ v,
                   const float *__restrict__ g, const float *__restrict__ beta,
                   const int32_t *__restrict__ cu, int N, int T, int H, Window win, char *__restrict__ ws,
                   LowRankGate lr) {
    using TIO = typename ChunkSmem<BF16, D>::TIO;
    using P = Prec<BF16>;
    using L = WsLayout<BF16, D>;
    using Plain = typename P::Plain;
    using Split = typename P::Split;
    constexpr int NKB = L::NKB;
    __shared__ ChunkSmem<BF16, D> sm;

    long rec;
    int h;
    const ChunkPos pos = local_chunk(blockIdx.x, cu, N, T, H, win, rec, h);
    if (!pos.valid) return;  // uniform over the block
    const int Cc = pos.Cc;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    char *wsb = ws + ((size_t)rec * H + h) * L::bytes;
    const long rowstride = (long)H * D;  // elements between consecutive tokens
    const long base_in = (pos.tok0 * H + h) * (long)D;

    // ---------------- phase 1: loads (rows >= Cc are zero), cumulative log2-decay
    // Thread (rg, cq) owns rows rg*RPG .. rg*RPG+RPG-1 and channels 4cq .. 4cq+3.  All global
    // loads are issued before any of them is used.
    using SM = ChunkSmem<BF16, D>;
    constexpr int RPG = SM::RPG;
    const int rg = tid / SM::CQ, c4 = (tid % SM::CQ) * 4;
    f32x4 gv[RPG];
    Raw4<TIO> kv[RPG], qv[RPG], vv[RPG];
    // Low-rank gate: wave w forms the 16x16 tiles (tt, ct) of g for ct = w, w + 4, ... with
    // A = z rows (tokens), B = W_up rows h*D + channel, k = rank index.  The operands of the
    // first 32 rank indices are loaded before q, k, v, so the MFMAs and the nonlinearity below
    // wait only for them and run while the q, k, v loads are still in flight.
    constexpr int NCTW = (D / 16 + 3) / 4;  // column tiles per wave (low-rank gate)
    FragB za[4], wb[NCTW];  // (unused, and removed by the compiler, when !LR)
    auto load_gate_ops = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + r16;
            const uint16_t *zr = lr.z + (pos.tok0 + (t < Cc ? t : 0)) * (long)lr.r + 32 * kb + 4 * grp;
            za[tt] = frag_bits(*reinterpret_cast<const uint2 *>(zr), *reinterpret_cast<const uint2 *>(zr + 16));
        }
#pragma unroll
        for (int u = 0; u < NCTW; ++u) {
            const int c = 16 * (wave + 4 * u) + r16;
            const uint16_t *wr = lr.w_up + ((long)h * D + c) * lr.r + 32 * kb + 4 * grp;
            wb[u] = frag_bits(*reinterpret_cast<const uint2 *>(wr), *reinterpret_cast<const uint2 *>(wr + 16));
        }
    };
    if constexpr (LR) load_gate_ops(0);
    // Rows past the end of a partial chunk read row 0 instead (always valid) and are zeroed
    // afterwards, so every load is unconditional and all of them are in flight together.
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int t = rg * RPG + r;
        const long off = base_in + (t < Cc ? t : 0) * rowstride + c4;
        if constexpr (!LR) gv[r] = *reinterpret_cast<const f32x4 *>(g + off);
        kv[r] = Raw4<TIO>::load(k + off);
        qv[r] = Raw4<TIO>::load(q + off);
        vv[r] = Raw4<TIO>::load(v + off);
    }
    if constexpr (LR) {
        // g of this chunk and head; rows past a partial chunk's end are zero.  The tiles go to the
        // G array of LDS, which the cumulative sum below then reads in its own layout.
        static_assert(BF16, "the low-rank gate takes bf16 operands");
        f32x4 acc[4][NCTW];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int u = 0; u < NCTW; ++u) acc[tt][u] = zero4();
        for (int kb = 0; kb < lr.r / 32; ++kb) {
            if (kb > 0) load_gate_ops(kb);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int u = 0; u < NCTW; ++u) acc[tt][u] = mfma(za[tt], wb[u], acc[tt][u]);
        }
#pragma unroll
        for (int u = 0; u < NCTW; ++u) {
            const int c = 16 * (wave + 4 * u) + r16;
            const float bc = lr.b[(long)h * D + c];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tt + 4 * grp + e;
                    sm.g.G[t][c] = t < Cc ? gate_log_alpha(acc[tt][u][e] + bc) : 0.f;
                }
        }
    }
    if constexpr (LR) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RPG; ++r) gv[r] = *reinterpret_cast<const f32x4 *>(&sm.g.G[rg * RPG + r][c4]);
    }
    const float bt_raw = beta[(pos.tok0 + (tid < Cc ? tid : 0)) * H + h];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        if (rg * RPG + r >= Cc) {
            gv[r] = zero4();
            kv[r] = Raw4<TIO>::zero();
            qv[r] = Raw4<TIO>::zero();
            vv[r] = Raw4<TIO>::zero();
        }
    }
    const float bt = tid < Cc ? bt_raw : 0.f;
    if (tid == 0) sm.flag = 0;
    if (tid < kChunk) sm.beta[tid] = bt;
    f32x4 run = zero4();
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int t = rg * RPG + r;
        run += gv[r] * kLog2e;
        gv[r] = run;
        kv[r].store(&sm.kq.in.K[t][c4]);
        qv[r].store(&sm.kq.in.Q[t][c4]);
    }
    *reinterpret_cast<f32x4 *>(&sm.tot[rg][c4]) = run;
    __syncthreads();
    f32x4 carry = zero4();
    for (int r2 = 0; r2 < rg; ++r2) carry += *reinterpret_cast<const f32x4 *>(&sm.tot[r2][c4]);
#pragma unroll
    for (int r = 0; r < RPG; ++r) *reinterpret_cast<f32x4 *>(&sm.g.G[rg * RPG + r][c4]) = gv[r] + carry;
    __syncthreads();

    // ---------------- phase 2: element-wise products, written as operand fragments
    char *wsQ = wsb + L::offQ;
    float *wsE = reinterpret_cast<float *>(wsb + L::offE);
    if (tid < D) wsE[tid] = fast_exp2(sm.g.G[kChunk - 1][tid]);
    for (int e = tid; e < 6 * D; e += 256) {
        const int p = e / D, c = e % D;
        const int I = p < 1 ? 1 : p < 3 ? 2 : 3, J = p - (I - 1) * I / 2;
        sm.bridge[p][c] = fast_exp2(sm.g.G[mid_row(I)][c] - sm.g.G[mid_row(J)][c]);
    }
    bool span_bad = false;
    Plain Xf[2][2];  // X^T fragments (rows: channel tiles 2kb, 2kb+1; k: token blocks) kept for W
    for (int kb = wave; kb < NKB; kb += 4) {
        // Qh = Q e^G, as A fragments (row t, k = channel)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + r16, m = mid_row(tt);
            float gt[8], gm[8], vals[8];
            ld_kslots(&sm.g.G[t][0], kb, grp, gt);
            ld_kslots(&sm.g.G[m][0], kb, grp, gm);
            ld_kslots(&sm.kq.in.Q[t][0], kb, grp, vals);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                span_bad |= fabsf(gt[s] - gm[s]) > 115.f;
                vals[s] *= fast_exp2(gt[s]);
            }
            P::st_plain(wsQ, L::nQ, tt * NKB + kb, lane, P::plain(vals));
        }
        // Kh^T = (K e^{gamma - G})^T and X^T = (K e^G)^T, as A fragments (row channel, k = token)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const int rt = 2 * kb + r2, i = 16 * rt + r16;
            const float gam = sm.g.G[kChunk - 1][i];
            float kh[2][8];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                float xv[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int t = 32 * kb2 + kslot(grp, s);
                    const float gt = sm.g.G[t][i];
                    const float kv = IO<TIO>::load(&sm.kq.in.K[t][0], i);
                    kh[kb2][s] = kv * fast_exp2(gam - gt);
                    xv[s] = kv * fast_exp2(gt);
                }
                Xf[r2][kb2] = P::plain(xv);
            }
            st_kh<BF16, D>(wsb, rt, lane, kh);
        }
    }
    if (span_bad) atomicOr(&sm.flag, 1);
    __syncthreads();

    // ---------------- phase 3: decayed Gram matrices Akk (times beta, strictly lower), Aqk
    // Waves form two pair groups x two channel halves: wave (pg, ch) sums channels of half ch
    // for the five sub-block pairs of group pg; one reduction round adds the two halves.
    const bool fallback = sm.flag != 0;
    if (!fallback) {
        constexpr int KBW = NKB / 2;  // channel k-blocks per half
        const int pg = wave >> 1, ch = wave & 1;
        f32x4 accK[5], accQ[5];
#pragma unroll
        for (int u = 0; u < 5; ++u) { accK[u] = zero4(); accQ[u] = zero4(); }
        // the pair group is a compile-time constant inside, so every array index is static
        auto gram_group = [&](auto pg_c) {
            constexpr int PG = decltype(pg_c)::value;
#pragma unroll
            for (int kk = 0; kk < KBW; ++kk) {
                const int kb = ch * KBW + kk;
                // row factors of the blocks this group uses: pairs (0,0) (1,0) (1,1) (2,0) (2,1) for
                // group 0, (2,2) (3,0) (3,1) (3,2) (3,3) for group 1.  The A side (k_i, q_i times
                // e^{G_i - G_mI}) is split once per block row and shared by the block's pairs; the
                // bridge e^{G_mI - G_mJ} of an off-diagonal pair scales the B side
                // (k_j e^{G_mJ - G_j}), which is split per pair.
                Split sK[4], sQ[4];
                float kB[4][8];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const bool needA = PG == 0 ? I <= 2 : I >= 2;
                    const bool needB = PG == 0 ? I <= 1 : true;
                    if (!needA && !needB) continue;
                    const int i = 16 * I + r16, m = mid_row(I);
                    float gi[8], gm[8], kv[8];
                    ld_kslots(&sm.g.G[i][0], kb, grp, gi);
                    ld_kslots(&sm.g.G[m][0], kb, grp, gm);
                    ld_kslots(&sm.kq.in.K[i][0], kb, grp, kv);
                    if (needA) {
                        float qv[8], ka[8], qa[8];
                        ld_kslots(&sm.kq.in.Q[i][0], kb, grp, qv);
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            const float fa = fast_exp2(gi[s] - gm[s]);
                            ka[s] = kv[s] * fa;
                            qa[s] = qv[s] * fa;
                        }
                        sK[I] = P::split(ka);
                        sQ[I] = P::split(qa);
                    }
                    if (needB) {
#pragma unroll
                        for (int s = 0; s < 8; ++s) kB[I][s] = kv[s] * fast_exp2(gm[s] - gi[s]);
                    }
                }
#pragma unroll
                for (int u = 0; u < 5; ++u) {
                    int I, J;
                    pair_ij(PG * 5 + u, I, J);
                    float bv[8];
                    if (I > J) {
                        float br[8];
                        ld_kslots(&sm.bridge[bridge_idx(I, J)][0], kb, grp, br);
#pragma unroll
                        for (int s = 0; s < 8; ++s) bv[s] = kB[J][s] * br[s];
                    } else {
#pragma unroll
                        for (int s = 0; s < 8; ++s) bv[s] = kB[J][s];
                    }
                    const Split bop = P::split(bv);
                    accK[u] = mfma(sK[I], bop, accK[u]);
                    accQ[u] = mfma(sQ[I], bop, accQ[u]);
                }
            }
        };
        if (pg == 0) gram_group(std::integral_constant<int, 0>{});
        else gram_group(std::integral_constant<int, 1>{});
        __syncthreads();  // every wave is done reading K, Q (aliased by Akk, Aqk below)
        if (ch == 1) {
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                int I, J;
                pair_ij(pg * 5 + u, I, J);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * I + 4 * grp + e, col = 16 * J + r16;
                    sm.kq.a.Akk[row][col] = accK[u][e];
                    sm.kq.a.Aqk[row][col] = accQ[u][e];
                }
            }
        }
        __syncthreads();
        if (ch == 0) {
#pragma unroll
            for (int u = 0; u < 5; ++u) {
                int I, J;
                pair_ij(pg * 5 + u, I, J);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * I + 4 * grp + e, col = 16 * J + r16;
                    // only the entries below the diagonal are ever read; beta scales Akk rows
                    sm.kq.a.Akk[row][col] = (accK[u][e] + sm.kq.a.Akk[row][col]) * sm.beta[row];
                    sm.kq.a.Aqk[row][col] = accQ[u][e] + sm.kq.a.Aqk[row][col];
                }
            }
        }
        __syncthreads();
    } else {
        // exact element-wise fallback for extreme decay inside a 16-token sub-block
        float rk[16], rq[16];
        const int i = tid >> 2, j0 = (tid & 3) * 16;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int j = j0 + jj;
            float ak = 0.f, aq = 0.f;
            if (j <= i) {
                for (int c = 0; c < D; ++c) {
                    const float e = fast_exp2(sm.g.G[i][c] - sm.g.G[j][c]);
                    const float kj = IO<TIO>::load(&sm.kq.in.K[j][0], c);
                    ak += IO<TIO>::load(&sm.kq.in.K[i][0], c) * kj * e;
                    aq += IO<TIO>::load(&sm.kq.in.Q[i][0], c) * kj * e;
                }
            }
            rk[jj] = ak * sm.beta[i];
            rq[jj] = aq;
        }
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            sm.kq.a.Akk[i][j0 + jj] = rk[jj];
            sm.kq.a.Aqk[i][j0 + jj] = rq[jj];
        }
        __syncthreads();
    }

    ut_and_outputs<BF16, D, RPG>(sm, vv, Xf, wsb, rg, c4);
}

// ------------------------------------------------------------------ kernel 1s: chunk-local, one decay per token
// Chunk-local kernel for a decay shared by all channels of a head: one log-decay per token and
// head (the Gated DeltaNet special case of the operator), or none (alpha = 1: DeltaNet).  The
// factor e^{G_i - G_j} of the decayed Gram matrices then leaves the channel sum, so Akk and Aqk
// are the plain products K K^T and Q K^T (bf16 inputs: exact products, fp32 sums) scaled
// element-wise, with no per-channel exponentials.  The record it writes is the one of the
// per-channel kernel (e^gamma repeated over the channels), read by the same state scan.
template <bool BF16, int D> struct alignas(16) ChunkSmemS {
    using TIO = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int KS = D + 8, VS = kChunk + 8, AS = kChunk + 4;
    static constexpr int CQ = D / 4;          // channel quads
    static constexpr int RG = 256 / CQ;       // row groups in the load layout
    static constexpr int RPG = kChunk / RG;   // rows per group
    union {
        float T[kChunk][AS];  // the UT transform Tm
    } g;
    union {
        struct { TIO K[kChunk][KS]; TIO Q[kChunk][KS]; } in;
        struct { float Akk[kChunk][AS]; float Aqk[kChunk][AS]; } a;
        TIO VT[D][VS];
    } kq;
    float G[kChunk];    // cumulative log2-decay of each token
    float eG[kChunk];   // 2^G
    float eGm[kChunk];  // 2^(gamma - G)
    float beta[kChunk];
};

template <bool BF16, int D>
__global__ void __launch_bounds__(256, (BF16 ? 3 : 1))  // bf16: 53 KB LDS, three workgroups per CU
chunk_local_scalar_kernel(const typename ChunkSmemS<BF16, D>::TIO *__restrict__ q,
                          const typename ChunkSmemS<BF16, D>::TIO *__restrict__ k,
                          const typename ChunkSmemS<BF16, D>::TIO *__restrict__ v,
                          const float *__restrict__ g, const float *__restrict__ beta,
                          const int32_t *__restrict__ cu, int N, int T, int H, Window win, char *__restrict__ ws) {
    using SM = ChunkSmemS<BF16, D>;
    using TIO = typename SM::TIO;
    using P = Prec<BF16>;
    using L = WsLayout<BF16, D>;
    using Plain = typename P::Plain;
    constexpr int NKB = L::NKB;
    constexpr int RPG = SM::RPG;
    __shared__ SM sm;

    long rec;
    int h;
    const ChunkPos pos = local_chunk(blockIdx.x, cu, N, T, H, win, rec, h);
    if (!pos.valid) return;  // uniform over the block
    const int Cc = pos.Cc;
    const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
    char *wsb = ws + ((size_t)rec * H + h) * L::bytes;
    const long rowstride = (long)H * D;
    const long base_in = (pos.tok0 * H + h) * (long)D;

    // ---------------- phase 1: loads (rows >= Cc are zero); per-token cumulative log2-decay
    const int rg = tid / SM::CQ, c4 = (tid % SM::CQ) * 4;
    Raw4<TIO> kv[RPG], qv[RPG], vv[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int t = rg * RPG + r;
        const long off = base_in + (t < Cc ? t : 0) * rowstride + c4;
        kv[r] = Raw4<TIO>::load(k + off);
        qv[r] = Raw4<TIO>::load(q + off);
        vv[r] = Raw4<TIO>::load(v + off);
    }
    if (wave == 0) {  // lane t: token t of the chunk
        const long tp = (pos.tok0 + (lane < Cc ? lane : 0)) * H + h;
        const float braw = beta[tp];
        float gl = g ? g[tp] * kLog2e : 0.f;
        if (lane >= Cc) gl = 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum over the 64 lanes
            const float y = __shfl_up(gl, off);
            if (lane >= off) gl += y;
        }
        const float gam = __shfl(gl, 63);
        sm.G[lane] = gl;
        sm.eG[lane] = fast_exp2(gl);
        sm.eGm[lane] = fast_exp2(gam - gl);
        sm.beta[lane] = lane < Cc ? braw : 0.f;
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int t = rg * RPG + r;
        if (t >= Cc) {
            kv[r] = Raw4<TIO>::zero();
            qv[r] = Raw4<TIO>::zero();
            vv[r] = Raw4<TIO>::zero();
        }
        kv[r].store(&sm.kq.in.K[t][c4]);
        qv[r].store(&sm.kq.in.Q[t][c4]);
    }
    __syncthreads();

    // ---------------- phase 2: Qh = Q e^G, Kh^T = (K e^{gamma - G})^T, X^T = (K e^G)^T
    char *wsQ = wsb + L::offQ;
    float *wsE = reinterpret_cast<float *>(wsb + L::offE);
    if (tid < D) wsE[tid] = sm.eG[kChunk - 1];  // e^gamma, the same for every channel
    Plain Xf[2][2];
    for (int kb = wave; kb < NKB; kb += 4) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + r16;
            float vals[8];
            ld_kslots(&sm.kq.in.Q[t][0], kb, grp, vals);
            const float f = sm.eG[t];
#pragma unroll
            for (int s = 0; s < 8; ++s) vals[s] *= f;
            P::st_plain(wsQ, L::nQ, tt * NKB + kb, lane, P::plain(vals));
        }
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const int rt = 2 * kb + r2, i = 16 * rt + r16;
            float kh[2][8];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                float eg[8], egm[8], xv[8];
                ld_kslots(&sm.eG[0], kb2, grp, eg);
                ld_kslots(&sm.eGm[0], kb2, grp, egm);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float kvv = IO<TIO>::load(&sm.kq.in.K[32 * kb2 + kslot(grp, s)][0], i);
                    kh[kb2][s] = kvv * egm[s];
                    xv[s] = kvv * eg[s];
                }
                Xf[r2][kb2] = P::plain(xv);
            }
            st_kh<BF16, D>(wsb, rt, lane, kh);
        }
    }

    // ---------------- phase 3: Akk = beta_i e^{G_i - G_j} k_i.k_j (j < i), Aqk = e^{G_i - G_j} q_i.k_j (j <= i)
    // The ten lower 16x16 tile pairs are dealt to the waves (pairs w, w + 4, w + 8); each wave sums
    // all channels of its pairs, so no reduction between waves is needed.
    f32x4 accK[3], accQ[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        accK[u] = zero4();
        accQ[u] = zero4();
        const int p = wave + 4 * u;
        if (p < 10) {
            int I, J;
            pair_ij(p, I, J);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float ka[8], qa[8], kbv[8];
                ld_kslots(&sm.kq.in.K[16 * I + r16][0], kb, grp, ka);
                ld_kslots(&sm.kq.in.Q[16 * I + r16][0], kb, grp, qa);
                ld_kslots(&sm.kq.in.K[16 * J + r16][0], kb, grp, kbv);
                const Plain bop = P::plain(kbv);
                accK[u] = mfma(P::plain(ka), bop, accK[u]);
                accQ[u] = mfma(P::plain(qa), bop, accQ[u]);
            }
        }
    }
    __syncthreads();  // every wave is done reading K, Q (aliased by Akk, Aqk below)
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int p = wave + 4 * u;
        if (p < 10) {
            int I, J;
            pair_ij(p, I, J);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * I + 4 * grp + e, col = 16 * J + r16;
                const float dec = col <= row ? fast_exp2(sm.G[row] - sm.G[col]) : 0.f;  // <= 1
                sm.kq.a.Akk[row][col] = col < row ? accK[u][e] * dec * sm.beta[row] : 0.f;
                sm.kq.a.Aqk[row][col] = accQ[u][e] * dec;
            }
        }
    }
    __syncthreads();

    ut_and_outputs<BF16, D, RPG>(sm, vv, Xf, wsb, rg, c4);
}

// ------------------------------------------------------------------ kernel 2: state scan
// A workgroup serves NCT tiles of 16 value columns of one (sequence, head) chain with NS waves
// per tile (NS = 2 or 4): wave `part` keeps rows part*D/NS .. of the tile's fp32 state in
// accumulator registers and owns 4 / NS of the chunk's four 16-token tiles.  After every state
// update each wave splits its rows into hi + lo bf16 operand fragments and publishes them in LDS
// (sx), so at the next chunk every wave holds the whole state as the B operand: it forms W S and
// Qh S of its own token tiles over all of d_k, then Ud = U - W S of those tiles, which it splits
// and publishes (ux).  After the exchange barrier every wave reads all of Ud, updates its own
// state rows with Kh^T Ud and finishes its output tiles with Aqk Ud.  Four parts shorten the
// serial chain per chunk; they are used when the problem has too few tiles to fill the GPU with
// two-part workgroups.
// The operands shared by all tiles (W, Qh, Kh^T, Aqk, e^gamma: one contiguous block at the start
// of the chunk's workspace record) are copied into LDS by direct global->LDS loads.  Every read
// of a chunk's block is complete at that chunk's exchange barrier, so with two buffers the copy
// of chunk c+2 can start right after the exchange barrier of chunk c.  Two extra waves per
// workgroup (producers: one for the even chunks, one for the odd ones, so each has at most one
// chunk in flight and waits for it with vmcnt(0)) issue these copies: a wave stalls while the
// memory pipeline accepts its loads, and this keeps those stalls off the waves that issue the
// MFMAs.  Issuing a whole block takes a wave longer than the stretch from an exchange barrier to
// the next top barrier, so each block is issued in two halves, the second after the next top
// barrier.  When two buffers do not fit, the compute waves copy the next chunk themselves after
// the current one.  U goes to registers one chunk ahead.  Output rows are
// left in LDS and written after the next barrier with 16-byte stores.
template <bool BF16, int D> struct ScanStage {
    using L = WsLayout<BF16, D>;
    static constexpr size_t bytes = L::offU;                     // W, Qh, Kh^T, Aqk, e^gamma
    static constexpr int kLoads = (int)(bytes / 1024);           // one 1 KB wave-load each
    static constexpr bool kProducer = 2 * bytes <= 128 * 1024;   // double buffer + producer waves
    static constexpr int kNP = kProducer ? 2 : 0;                // producer waves per workgroup
    static_assert(bytes % 1024 == 0, "staged block is a whole number of wave-loads");
};

template <bool BF16, int D, int NCT, int NS>
constexpr int scan_threads() { return 64 * (NS * NCT + ScanStage<BF16, D>::kNP); }

// Wave-loads of the staged block that the segment map reads: W, Kh^T and e^gamma (Qh and Aqk
// only serve the read-out).
template <bool BF16, int D> constexpr bool map_needs_load(int i) {
    using L = WsLayout<BF16, D>;
    return i < (int)(L::offQ / 1024) || (i >= (int)(L::offK / 1024) && i < (int)(L::offA / 1024)) ||
           i >= (int)(L::offE / 1024);
}

// MAP = true: the segment map instead of the read-out.  Every chain gets twice the workgroups:
// the first GPC run the chunks from S = 0 with the chunks' U (the offset B, into sN), the other
// GPC from S = I with U taken as zero (the linear part A, into sA); no output rows, no Qh S.
template <bool BF16, int D, int NCT, int NS, bool MAP = false>
__global__ void __launch_bounds__((scan_threads<BF16, D, NCT, NS>()))
chunk_scan_kernel(const int32_t *__restrict__ cu, int T, int H, int nchains, float scale,
                  const float *s0, float *sN,  // may alias: each element is read before it is written
                  typename ChunkSmem<BF16, D>::TIO *__restrict__ o, const char *__restrict__ ws,
                  float *__restrict__ sA, Window win) {
    using TIO = typename ChunkSmem<BF16, D>::TIO;
    using P = Prec<BF16>;
    using L = WsLayout<BF16, D>;
    using St = ScanStage<BF16, D>;
    using Plain = typename P::Plain;
    using Split = typename P::Split;
    constexpr bool kProd = St::kProducer;
    constexpr int NKB = L::NKB, NRT = L::NRT, NJT = D / 16, GPC = NJT / NCT;
    constexpr int KBH = NKB / NS, RTH = NRT / NS;  // k-blocks and row tiles per part
    constexpr int NW = NS * NCT;                   // compute waves
    constexpr int NOT = 4 / NS;                    // output token tiles per wave
    constexpr int LPW = (St::kLoads + NW - 1) / NW;  // copies per compute wave (no producer)
    constexpr int OC = NCT * 16;                     // output columns of the workgroup
    static_assert(GPC * NCT == NJT && KBH >= 1 && KBH * NS == NKB && (NS == 2 || NS == 4), "tiling");
    // two separate arrays (not one [2][bytes] array) so that alias analysis can tell a read of
    // one buffer from an in-flight copy into the other
    __shared__ __attribute__((aligned(16))) char stage0[St::bytes];
    __shared__ __attribute__((aligned(16))) char stage1[kProd ? St::bytes : 16];
    // the state of each column tile as the B operand of W S and Qh S (hi and lo planes of its
    // split, k-block fragments), written by the wave that holds the rows after every update
    __shared__ __attribute__((aligned(16))) char sx[NCT][2 * NKB * 1024];
    // Ud of each column tile as the B operand of the state update and Aqk Ud (hi and lo planes,
    // token k-block fragments), each 16-token tile written by the wave that owns it
    // (bf16: then Ud in bf8 for the Kh^T low plane, 8 bytes per lane and token k-block)
    __shared__ __attribute__((aligned(16))) char ux[NCT][2 * 2 * 1024 + (BF16 ? 1024 : 0)];
    // the Kh^T low plane of the current chunk (bf16 with producer waves): loaded into registers by
    // the chunk's producer with its stage copies, written here after the chunk's top barrier, read
    // after its exchange barrier
    constexpr bool kKlx = BF16 && kProd;
    constexpr int kKlFrags = L::nK;  // fragments of 512 bytes
    __shared__ __attribute__((aligned(16))) long klx[kKlx ? kKlFrags * 64 : 1];
    __shared__ __attribute__((aligned(16))) TIO obuf[kProd && !MAP ? kChunk : 1][kProd && !MAP ? OC : 1];  // output rows

    // the GPC workgroups of one chain go to the same XCD (blocks are dealt round-robin to 8 XCDs)
    constexpr int NG = MAP ? 2 * GPC : GPC;  // workgroups per chain
    const int b = blockIdx.x, xcd = b & 7, sl = b >> 3;
    const int jgm = sl % NG, chain = (sl / NG) * 8 + xcd;
    if (chain >= nchains) return;  // uniform over the workgroup
    const bool amap = MAP && jgm >= GPC;  // this workgroup forms columns of A
    const int jg = amap ? jgm - GPC : jgm;
    const int n = chain / H, h = chain % H;
    const int wave = wave_id(), lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
    const bool producer = kProd && wave >= NW;
    const int ct = producer ? 0 : wave / NS, part = wave % NS;
    const int jt = jg * NCT + ct;
    const int col = 16 * jt + r16;
    // output token tiles of this wave: with two parts {0, 3} and {1, 2} (equal MFMA work), with
    // four parts tile `part`
    auto own_tile = [&](int i) __attribute__((always_inline)) {
        return NS == 4 ? part : (part ? (i ? 2 : 1) : (i ? 3 : 0));
    };

    // this chain's chunks in window `win` (see Window): [c_lo, c_hi); the state enters from s0 in
    // the window that holds the sequence's first chunk and from sN (the state the previous window
    // left) otherwise.  From here on s_tok, L_n and chunk indices count from chunk c_lo.
    long s_tok, L_n, rec0;
    if (cu) {
        s_tok = cu[n];
        L_n = (long)cu[n + 1] - s_tok;
        rec0 = n + s_tok / kChunk - (long)win.w * win.Wc;
    } else {
        s_tok = (long)n * T;
        L_n = T;
        rec0 = (long)n * win.Wc - (long)win.w * win.Wc;
    }
    const long nck_seq = (L_n + kChunk - 1) / kChunk;
    const long first = cu ? s_tok / kChunk : 0;  // window coordinate of chunk 0
    const long c_lo = max(0L, (long)win.w * win.Wc - first);
    const long c_hi = min(nck_seq, (long)(win.w + 1) * win.Wc - first);
    // an empty sequence hands its initial state on in window 0 only
    const bool active = c_lo < c_hi || (nck_seq == 0 && win.w == 0);
    if (!active) return;  // uniform over the workgroup
    const long nck = max(0L, c_hi - c_lo);
    s_tok += c_lo * kChunk;
    L_n -= c_lo * kChunk;
    const long slot0 = rec0 + c_lo;
    const float *sin = c_lo == 0 ? s0 : sN;
    const int HD = H * D;
    auto record = [&](long c) __attribute__((always_inline)) { return ws + ((size_t)(slot0 + c) * H + h) * L::bytes; };
    auto copy_one = [&](const char *src, char *dst, int i) __attribute__((always_inline)) {
        __builtin_amdgcn_global_load_lds(src + (size_t)i * 1024 + lane * 16,
                                         (__attribute__((address_space(3))) void *)(dst + i * 1024), 16, 0, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // ================================================================ producer wave
    if (producer) {
        // wave-loads [i0, i1) of chunk c into buffer BUF
        auto copy_range = [&](long c, auto bufc, int i0, int i1) __attribute__((always_inline)) {
            char *dst = decltype(bufc)::value ? stage1 : stage0;
            const char *src = record(c);
#pragma unroll
            for (int i = 0; i < St::kLoads; ++i)
                if (i >= i0 && i < i1 && (!MAP || map_needs_load<BF16, D>(i))) copy_one(src, dst, i);
        };
        constexpr int kHalf = St::kLoads / 2;
        const int pw = wave - NW;  // this producer copies the chunks c with c % 2 == pw
        long klr[kKlx ? kKlFrags : 1];  // the low plane of this producer's next chunk
        auto load_kl = [&](long c) __attribute__((always_inline)) {
            if constexpr (kKlx) {
                const long *pk = reinterpret_cast<const long *>(record(c) + L::offKl) + lane;
#pragma unroll
                for (int f = 0; f < kKlFrags; ++f) klr[f] = pk[f * 64];
            }
        };
        if (pw < nck) {
            if (pw == 0) copy_range(0, I0{}, 0, St::kLoads);
            else copy_range(1, I1{}, 0, St::kLoads);
            load_kl(pw);
        }
        // Chunk c + 2 goes into chunk c's buffer in two halves, so that neither takes longer to
        // issue than the stretch it has (a wave issues about one 1 KB wave-load per 30-40
        // clocks): the first after the exchange barrier of chunk c (no wave reads that buffer any
        // more), the second after the top barrier of chunk c + 1.  The producer waits for both
        // before the top barrier of chunk c + 2.
        auto pstep = [&](long c, auto bufc) __attribute__((always_inline)) {
            constexpr int buf = decltype(bufc)::value;
            const bool mine = buf == pw;  // chunk c's parity is buf
            if (mine) __builtin_amdgcn_s_waitcnt(0);  // this producer's copies of chunk c landed
            // top barrier without a fence (a fence would make the other producer wait for its
            // copies of the next chunk too)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            // chunk c's low plane into LDS (every read of chunk c - 1's was done before this barrier;
            // the exchange barrier below publishes it)
            if constexpr (kKlx)
                if (mine) {
#pragma unroll
                    for (int f = 0; f < kKlFrags; ++f) klx[f * 64 + lane] = klr[f];
                }
            // second half of chunk c + 1 (chunks 0 and 1 were copied whole), into the other buffer
            if (!mine && c >= 1 && c + 1 < nck) copy_range(c + 1, std::integral_constant<int, 1 - buf>{}, kHalf, St::kLoads);
            // exchange barrier: past it, no wave reads this chunk's buffer any more
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (mine && c + 2 < nck) {
                copy_range(c + 2, bufc, 0, kHalf);
                load_kl(c + 2);
            }
        };
        for (long c = 0; c < nck; c += 2) {
            pstep(c, I0{});
            if (c + 1 < nck) pstep(c + 1, I1{});
        }
        __syncthreads();  // pairs with the compute waves' last barrier
        return;
    }

    // ================================================================ compute waves
    // output rows of chunk c from obuf, 16 bytes per lane; compute wave w takes row blocks
    // w, w + NW, ... of RPI rows each
    auto store_rows = [&](long c) __attribute__((always_inline)) {
        constexpr int LPR = OC * (int)sizeof(TIO) / 16, RPI = 64 / LPR, EPL = 16 / (int)sizeof(TIO);
        constexpr int NBLK = kChunk / RPI;
        static_assert(LPR * RPI == 64, "row split");
        const long tok0 = s_tok + c * kChunk;
        const int Cc = (int)min((long)kChunk, L_n - c * kChunk);
        const int r0 = lane / LPR, seg = lane % LPR;
        TIO *dst = o + (tok0 * H + h) * (long)D + jg * OC + seg * EPL;
#pragma unroll
        for (int kk = 0; kk < (NBLK + NW - 1) / NW; ++kk) {
            const int blk = kk * NW + wave;
            if (blk < NBLK) {
                const int t = blk * RPI + r0;
                const uint4 val = *reinterpret_cast<const uint4 *>(&obuf[t][seg * EPL]);
                if (t < Cc) *reinterpret_cast<uint4 *>(dst + (long)t * HD) = val;
            }
        }
    };
    // this wave's share of the copies of chunk c (no producer wave): wave-load j * NW + wave
    auto stage_all = [&](long c) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int i = j * NW + wave;
            if (i < St::kLoads && (!MAP || map_needs_load<BF16, D>(i))) copy_one(record(c), stage0, i);
        }
    };
    // U of the own token tiles; the tiles alternate between two register sets (even chunks in
    // uA, odd in uB), so a prefetched tile is never copied between registers before it has arrived
    using UT = typename std::conditional<BF16, U24, f32x4>::type;  // a U tile as stored
    UT uA[NOT], uB[NOT];
    auto prefetch_u = [&](long c, UT (&u)[NOT]) __attribute__((always_inline)) {
        if (amap) {  // the linear part: U is zero
#pragma unroll
            for (int i = 0; i < NOT; ++i) u[i] = UT{};
            return;
        }
        const UT *pu = reinterpret_cast<const UT *>(record(c) + L::offU) + jt * 4 * 64 + lane;
#pragma unroll
        for (int i = 0; i < NOT; ++i) u[i] = pu[own_tile(i) * 64];
    };
    auto u_value = [&](const UT &u) __attribute__((always_inline)) {
        if constexpr (BF16) return unpack_u24(u);
        else return u;
    };

    f32x4 S[RTH];
    const long sbase = (long)chain * D * D;
#pragma unroll
    for (int r = 0; r < RTH; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[r][e] = MAP ? (amap && 16 * (part * RTH + r) + 4 * grp + e == col ? 1.f : 0.f)
                          : sin ? sin[sbase + (long)(16 * (part * RTH + r) + 4 * grp + e) * D + col] : 0.f;

    // this wave's rows of the state, split, into sx (k-blocks part * KBH ..); the next top barrier
    // publishes them
    auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KBH; ++kk) {
            float vals[8] = {S[2 * kk][0], S[2 * kk][1], S[2 * kk][2], S[2 * kk][3],
                             S[2 * kk + 1][0], S[2 * kk + 1][1], S[2 * kk + 1][2], S[2 * kk + 1][3]};
            P::st_split(&sx[ct][0], NKB, part * KBH + kk, lane, P::split(vals));
        }
    };
    publish_state();
    if (nck > 0) {
        if (!kProd) stage_all(0);
        prefetch_u(0, uA);
    }
    // One chunk.  The buffer index is a compile-time constant (the loop below is unrolled by
    // two), so the compiler can tell the LDS reads of this chunk from the copies into the
    // other buffer and does not make the reads wait for those copies.
    auto chunk_step = [&](long c, auto bufc, UT (&u_cur)[NOT], UT (&u_nx)[NOT]) __attribute__((always_inline)) {
        constexpr int buf = decltype(bufc)::value;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
        __syncthreads();                // ... and every copy: chunk c is in LDS, and so is the state
        const bool more = c + 1 < nck;
        const char *sb = buf ? stage1 : stage0;
        // bf16: 2^s for this lane's value column, under which Ud takes its bf8 form (see
        // ut_and_outputs), and 2^-s; the linear part of a segment map (U taken as zero, from S = I)
        // keeps s = 0
        float usc = 1.f, uinv = 1.f;
        if constexpr (BF16) {
            const int su = amap ? 0 : (int)reinterpret_cast<const int8_t *>(sb + L::offEs)[col];
            usc = __uint_as_float((uint32_t)(127 + su) << 23);
            uinv = __uint_as_float((uint32_t)(127 - su) << 23);
        }
        // the state (every k-block) and the W and Qh fragments of the own token tiles; bf16 ones are
        // all requested before the first product (fp32 ones take twice the registers and are read
        // next to their use)
        const char *sxb = &sx[ct][0];
        auto ldS = [&](int kb) __attribute__((always_inline)) { return P::ld_split(sxb, NKB, kb, lane); };
        auto ldW = [&](int i, int kb) __attribute__((always_inline)) { return P::ld_plain(sb + L::offW, L::nW, own_tile(i) * NKB + kb, lane); };
        auto ldQ = [&](int i, int kb) __attribute__((always_inline)) { return P::ld_plain(sb + L::offQ, L::nQ, own_tile(i) * NKB + kb, lane); };
        Split sop[BF16 ? NKB : 1];
        Plain wf[NOT][BF16 ? NKB : 1], qf[NOT][BF16 ? NKB : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sop[kb] = ldS(kb);
#pragma unroll
                for (int i = 0; i < NOT; ++i) {
                    wf[i][kb] = ldW(i, kb);
                    if constexpr (!MAP) qf[i][kb] = ldQ(i, kb);
                }
            }
        }
        if (more) prefetch_u(c + 1, u_nx);
        // low plane of this part's Kh^T rows (bf16, fp8 e4m3), used after the exchange barrier:
        // from LDS where the producer put it, else straight from the record
        long kl[BF16 ? RTH : 1][2];
        if constexpr (BF16 && !kKlx) {
            const long *pk = reinterpret_cast<const long *>(record(c) + L::offKl) + lane;
#pragma unroll
            for (int r = 0; r < RTH; ++r)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) kl[r][kb2] = pk[((part * RTH + r) * 2 + kb2) * 64];
        }
        // W S and Qh S of the own token tiles over all of d_k, k-blocks in order
        f32x4 wsa[NOT], qsa[NOT];
#pragma unroll
        for (int i = 0; i < NOT; ++i) { wsa[i] = zero4(); qsa[i] = zero4(); }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const Split so = BF16 ? sop[BF16 ? kb : 0] : ldS(kb);
#pragma unroll
            for (int i = 0; i < NOT; ++i) {
                wsa[i] = mfma(BF16 ? wf[i][BF16 ? kb : 0] : ldW(i, kb), so, wsa[i]);
                if constexpr (!MAP) qsa[i] = mfma(BF16 ? qf[i][BF16 ? kb : 0] : ldQ(i, kb), so, qsa[i]);
            }
        }
        // Ud = U - W S of the own tiles, split, into ux (tile tt fills half tt & 1 of token
        // k-block tt >> 1 in both planes)
#pragma unroll
        for (int i = 0; i < NOT; ++i) {
            const int ot = own_tile(i);
            const f32x4 ud = u_value(u_cur[i]) - wsa[i];
            char *dst = &ux[ct][0] + ((ot >> 1) * 64 + lane) * 16;
            if constexpr (BF16) {
                const uint32_t h01 = pk_bf16(ud[0], ud[1]), h23 = pk_bf16(ud[2], ud[3]);
                const uint32_t l01 = pk_bf16(ud[0] - __uint_as_float(h01 << 16), ud[1] - __uint_as_float(h01 & 0xffff0000u));
                const uint32_t l23 = pk_bf16(ud[2] - __uint_as_float(h23 << 16), ud[3] - __uint_as_float(h23 & 0xffff0000u));
                *reinterpret_cast<uint2 *>(dst + (ot & 1) * 8) = make_uint2(h01, h23);
                *reinterpret_cast<uint2 *>(dst + 2048 + (ot & 1) * 8) = make_uint2(l01, l23);
                // bf8 of Ud 2^s (clamped to its largest finite value) for the low planes of Kh^T and Aqk
                float c8[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) c8[e] = fminf(fmaxf(ud[e] * usc, -57344.f), 57344.f);
                int w8 = __builtin_amdgcn_cvt_pk_bf8_f32(c8[0], c8[1], 0, false);
                w8 = __builtin_amdgcn_cvt_pk_bf8_f32(c8[2], c8[3], w8, true);
                *reinterpret_cast<int *>(&ux[ct][0] + 4096 + ((ot >> 1) * 64 + lane) * 8 + (ot & 1) * 4) = w8;
            } else {
                *reinterpret_cast<f32x4 *>(dst + (ot & 1) * 2048) = ud;
            }
        }
        // operands of the second part of the chunk, requested before the barrier
        // (with a producer the buffer is refilled right after the exchange barrier, so every
        // read of it must be issued before; without one, fp32 fragments are read next to use)
        constexpr bool kEarlyK = BF16 || kProd;
        auto ldK = [&](int r, int kb2) __attribute__((always_inline)) { return P::ld_plain(sb + L::offK, L::nK, (part * RTH + r) * 2 + kb2, lane); };
        Plain kf[RTH][2];
        if (kEarlyK) {
#pragma unroll
            for (int r = 0; r < RTH; ++r)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) kf[r][kb2] = ldK(r, kb2);
        }
        // Aqk fragments of the own output tiles: one k-block for tiles 0 and 1, two for 2 and 3
        // (fp32: both planes; bf16: the bf16 plane, the fp8 low plane and the low plane's scales
        // for the tile's output rows 4 grp .. 4 grp + 3)
        Split af[BF16 ? 1 : NOT][2];
        Plain ah[BF16 ? NOT : 1][2];
        long al[BF16 ? NOT : 1][2];
        f32x4 asc[BF16 ? NOT : 1];
        if constexpr (!MAP) {
#pragma unroll
            for (int i = 0; i < NOT; ++i) {
                const int ot = own_tile(i);
                const int f0 = aidx(ot, 0), f1 = aidx(ot, ot >= 2 ? 1 : 0);
                if constexpr (BF16) {
                    ah[i][0] = P::ld_plain(sb + L::offA, L::nA, f0, lane);
                    ah[i][1] = P::ld_plain(sb + L::offA, L::nA, f1, lane);
                    al[i][0] = reinterpret_cast<const long *>(sb + L::offAl)[f0 * 64 + lane];
                    al[i][1] = reinterpret_cast<const long *>(sb + L::offAl)[f1 * 64 + lane];
                    asc[i] = load4(reinterpret_cast<const uint16_t *>(sb + L::offEa) + 16 * ot + 4 * grp);
                } else {
                    af[i][0] = P::ld_split(sb + L::offA, L::nA, f0, lane);
                    af[i][1] = P::ld_split(sb + L::offA, L::nA, f1, lane);
                }
            }
        }
        f32x4 e_cur[RTH], e_lo[BF16 ? RTH : 1];
#pragma unroll
        for (int r = 0; r < RTH; ++r) {
            e_cur[r] = *reinterpret_cast<const f32x4 *>(sb + L::offE + 4 * (16 * (part * RTH + r) + 4 * grp));
            if constexpr (BF16) e_lo[r] = load4(reinterpret_cast<const uint16_t *>(sb + L::offEl) + 16 * (part * RTH + r) + 4 * grp);
        }
        if constexpr (BF16) {  // the products with Ud's bf8 form are scaled back by 2^-s
#pragma unroll
            for (int r = 0; r < RTH; ++r) e_lo[r] *= uinv;
#pragma unroll
            for (int i = 0; i < (MAP ? 0 : NOT); ++i) asc[i] *= uinv;
        }
        // rows of the previous chunk (left in obuf before the top barrier; refilled after the
        // exchange barrier)
        if constexpr (!MAP)
            if (kProd && c > 0) store_rows(c - 1);
        // exchange barrier: only LDS traffic must be complete (lgkmcnt); copies into the other
        // stage buffer stay in flight (a fence here would wait for them too)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // Ud of all four token tiles (every wave reads the same split values)
        Split Uop[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) Uop[kb2] = P::ld_split(&ux[ct][0], 2, kb2, lane);
        // O rows of the own tiles (Qh S, then Aqk Ud) and the state update; the products that
        // need only the first token k-block of Ud come first
        f32x4 oo[NOT], Sn[RTH];
#pragma unroll
        for (int i = 0; i < NOT; ++i) oo[i] = qsa[i];
#pragma unroll
        for (int r = 0; r < RTH; ++r) Sn[r] = S[r] * e_cur[r];
        if constexpr (kKlx) {
#pragma unroll
            for (int r = 0; r < RTH; ++r)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) kl[r][kb2] = klx[((part * RTH + r) * 2 + kb2) * 64 + lane];
        }
        if constexpr (BF16) {
            // the Kh^T and Aqk low planes times Ud in bf8, scaled back per state row / output row
            long u8[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) u8[kb2] = *reinterpret_cast<const long *>(&ux[ct][0] + 4096 + (kb2 * 64 + lane) * 8);
#pragma unroll
            for (int r = 0; r < RTH; ++r) {
                f32x4 a8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(kl[r][0], u8[0], zero4(), 0, 0, 0);
                a8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(kl[r][1], u8[1], a8, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) Sn[r][e] = fmaf(a8[e], e_lo[r][e], Sn[r][e]);
            }
#pragma unroll
            for (int i = 0; i < (MAP ? 0 : NOT); ++i) {
                f32x4 a8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(al[i][0], u8[0], zero4(), 0, 0, 0);
                if (own_tile(i) >= 2) a8 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_bf8(al[i][1], u8[1], a8, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) oo[i][e] = fmaf(a8[e], asc[i][e], oo[i][e]);
            }
        }
        // Aqk as the read-out takes it: its bf16 plane (the low plane was added above), both fp32
        // planes otherwise
        auto aop = [&](int i, int kb2) __attribute__((always_inline)) {
            if constexpr (BF16) return ah[i][kb2];
            else return af[i][kb2];
        };
#pragma unroll
        for (int i = 0; i < (MAP ? 0 : NOT); ++i) oo[i] = mfma(aop(i, 0), Uop[0], oo[i]);
        // Kh^T as the state update takes it: its bf16 plane (the low plane was added above), fp32
        // as stored otherwise
        auto khop = [&](int r, int kb2) __attribute__((always_inline)) {
            return kEarlyK ? kf[r][kb2] : ldK(r, kb2);
        };
#pragma unroll
        for (int r = 0; r < RTH; ++r) Sn[r] = mfma(khop(r, 0), Uop[0], Sn[r]);
#pragma unroll
        for (int i = 0; i < (MAP ? 0 : NOT); ++i)
            if (own_tile(i) >= 2) oo[i] = mfma(aop(i, 1), Uop[1], oo[i]);
#pragma unroll
        for (int r = 0; r < RTH; ++r) S[r] = mfma(khop(r, 1), Uop[1], Sn[r]);
        // every read of sx for this chunk was complete at the exchange barrier
        publish_state();
        if (kProd) {
            // rows of this chunk (the previous ones were read before the exchange barrier)
#pragma unroll
            for (int i = 0; i < (MAP ? 0 : NOT); ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    IO<TIO>::store(&obuf[16 * own_tile(i) + 4 * grp + e][0], ct * 16 + r16, scale * oo[i][e]);
        } else {
            if constexpr (!MAP) {
                const int Cc = (int)min((long)kChunk, L_n - c * kChunk);
                TIO *ob = o + ((s_tok + c * kChunk) * H + h) * (long)D + col;
#pragma unroll
                for (int i = 0; i < NOT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * own_tile(i) + 4 * grp + e;
                        if (t < Cc) IO<TIO>::store(ob, (long)t * HD, scale * oo[i][e]);
                    }
            }
            if (more) {
                __syncthreads();  // every wave is done with the single buffer
                stage_all(c + 1);
            }
        }
    };
    for (long c = 0; c < nck; c += 2) {
        chunk_step(c, I0{}, uA, uB);
        if (c + 1 < nck) chunk_step(c + 1, std::integral_constant<int, kProd ? 1 : 0>{}, uB, uA);
    }
    if (kProd) {
        __syncthreads();  // the last chunk's rows are in obuf (and pairs with the producers' last barrier)
        if constexpr (!MAP)
            if (nck > 0) store_rows(nck - 1);
    }
    float *const sout = amap ? sA : sN;
    if (sout) {
#pragma unroll
        for (int r = 0; r < RTH; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sout[sbase + (long)(16 * (part * RTH + r) + 4 * grp + e) * D + col] = S[r][e];
    }
}

// ------------------------------------------------------------------ host side
size_t fwd_bytes_per_chunk_head(bool bf16, int d) {
    if (bf16) return d == 128 ? WsLayout<true, 128>::bytes : WsLayout<true, 64>::bytes;
    return d == 128 ? WsLayout<false, 128>::bytes : WsLayout<false, 64>::bytes;
}

long fwd_chunk_slots(int B, int T, int N, bool varlen) {
    const long ncs = ((long)T + kChunk - 1) / kChunk;
    return varlen ? (long)N + ncs : (long)B * ncs;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Records of a window of Wc chunk indices (see Window): dense N Wc, packed Wc + N.
static long window_records(long Wc, int N, bool varlen) { return varlen ? Wc + N : (long)N * Wc; }

bool plan_fwd_windows(bool bf16, int d, int B, int T, int H, int N, bool varlen, bool have_final_state,
                      size_t ws_bytes, WindowPlan &p) {
    const size_t rec = fwd_bytes_per_chunk_head(bf16, d);
    const long ncs = ((long)T + kChunk - 1) / kChunk;
    const size_t full = (size_t)fwd_chunk_slots(B, T, N, varlen) * (size_t)H * rec;
    p = WindowPlan{ncs, 1, 0, false};
    // one pass whenever the workspace holds every record (measured: windows are not faster on
    // the 4 x 4096-token batch nor on the 131072-token sequence)
    if (ws_bytes >= full || ncs <= 1 || H == 0) return ws_bytes >= full;
    // the state travels between windows in final_state, else in the workspace after the records
    const size_t carry = have_final_state ? 0 : align256((size_t)N * H * d * d * sizeof(float));
    if (ws_bytes <= carry) return false;
    const size_t per_chunk = (varlen ? 1 : (size_t)N) * (size_t)H * rec;  // bytes per chunk index
    const size_t fixed = varlen ? (size_t)N * H * rec : 0;
    if (ws_bytes - carry < fixed + per_chunk) return false;
    const long Wc = std::min<long>(ncs, (long)((ws_bytes - carry - fixed) / per_chunk));
    p.Wc = Wc;
    p.nwin = (ncs + Wc - 1) / Wc;
    p.carry = !have_final_state;
    p.carry_off = align256((size_t)window_records(Wc, N, varlen) * H * rec);
    return true;
}

size_t fwd_min_workspace(bool bf16, int d, int B, int T, int H, int N, bool varlen, bool have_final_state) {
    const size_t rec = fwd_bytes_per_chunk_head(bf16, d);
    const long ncs = ((long)T + kChunk - 1) / kChunk;
    const size_t full = (size_t)fwd_chunk_slots(B, T, N, varlen) * (size_t)H * rec;
    if (ncs <= 1 || H == 0) return full;
    const size_t carry = have_final_state ? 0 : align256((size_t)N * H * d * d * sizeof(float));
    return std::min<size_t>(full, align256((size_t)window_records(1, N, varlen) * H * rec) + carry);
}

// Window w of a plan with Wc chunk indices per window (the whole batch when Wc covers every chunk).
static Window make_window(const FwdArgs &a, long Wc, int w) {
    const bool varlen = a.cu_seqlens != nullptr;
    const long ncs = ((long)a.T + kChunk - 1) / kChunk;
    Window win;
    win.w = w;
    win.Wc = Wc;
    if (varlen) win.nrec = std::min<long>(Wc + a.N, (long)a.N + ncs - (long)w * Wc);
    else win.nrec = (long)a.N * std::min<long>(Wc, ncs - (long)w * Wc);
    return win;
}
static Window full_window(const FwdArgs &a) { return make_window(a, ((long)a.T + kChunk - 1) / kChunk, 0); }

template <bool BF16, int D, bool LR = false>
static hipError_t launch_local_t(const FwdArgs &a, const Window &win, hipStream_t st) {
    if (win.nrec <= 0 || a.H <= 0) return hipSuccess;
    const LowRankGate lr{a.gate_z, a.gate_w_up, a.gate_b, a.gate_r};
    return launch_kernel(chunk_local_kernel<BF16, D, LR>, dim3((unsigned)(win.nrec * a.H)), dim3(256), st, a.q,
                         a.k, a.v, a.g, a.beta, a.cu_seqlens, a.N, a.T, a.H, win, a.ws, lr);
}

template <bool BF16, int D, int NCT, int NS, bool MAP>
static hipError_t launch_scan_nct(const FwdArgs &a, const Window &win, hipStream_t st, int nchains) {
    const long blocks = (long)((nchains + 7) / 8) * 8 * (D / 16 / NCT) * (MAP ? 2 : 1);
    return launch_kernel(chunk_scan_kernel<BF16, D, NCT, NS, MAP>, dim3((unsigned)blocks),
                         dim3(scan_threads<BF16, D, NCT, NS>()), st, a.cu_seqlens, a.T, a.H, nchains, a.scale,
                         MAP ? nullptr : a.s0, a.sN, a.o, a.ws, MAP ? a.map_A : nullptr, win);
}

// Compute units of the current device, queried once per device (the value never changes).
static int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Column tiles per workgroup: two when that still gives every CU a workgroup (the tiles then
// share one LDS copy of the chunk's operands), else one.  At d = 128 four waves per tile (a
// shorter serial chain per chunk than two; the results are bitwise the same, since every wave
// forms its products over all of d_k in the same order), at d = 64 two.  The segment map (MAP)
// has twice the column tiles: those of B and those of A.
template <bool BF16, int D, bool MAP = false>
static hipError_t launch_scan_t(const FwdArgs &a, const Window &win, hipStream_t st) {
    const int nchains = a.N * a.H;
    if (nchains <= 0) return hipSuccess;
    const int cus = device_cu_count();
    const long tiles = (long)nchains * (D / 16) * (MAP ? 2 : 1);
    constexpr int NS = D == 128 ? 4 : 2;
    if (tiles / 2 >= cus) return launch_scan_nct<BF16, D, 2, NS, MAP>(a, win, st, nchains);
    return launch_scan_nct<BF16, D, 1, NS, MAP>(a, win, st, nchains);
}

template <bool BF16, int D>
static hipError_t launch_local_scalar_t(const FwdArgs &a, const Window &win, hipStream_t st) {
    if (win.nrec <= 0 || a.H <= 0) return hipSuccess;
    return launch_kernel(chunk_local_scalar_kernel<BF16, D>, dim3((unsigned)(win.nrec * a.H)), dim3(256), st, a.q,
                         a.k, a.v, a.g, a.beta, a.cu_seqlens, a.N, a.T, a.H, win, a.ws);
}

static hipError_t launch_local_win(const FwdArgs &a, const Window &win, hipStream_t st) {
    if (a.scalar_gate) {
        if (a.bf16) return a.dk == 128 ? launch_local_scalar_t<true, 128>(a, win, st) : launch_local_scalar_t<true, 64>(a, win, st);
        return a.dk == 128 ? launch_local_scalar_t<false, 128>(a, win, st) : launch_local_scalar_t<false, 64>(a, win, st);
    }
    if (a.gate_z) {  // low-rank gate: bf16 only (checked by the caller)
        return a.dk == 128 ? launch_local_t<true, 128, true>(a, win, st) : launch_local_t<true, 64, true>(a, win, st);
    }
    if (a.bf16) return a.dk == 128 ? launch_local_t<true, 128>(a, win, st) : launch_local_t<true, 64>(a, win, st);
    return a.dk == 128 ? launch_local_t<false, 128>(a, win, st) : launch_local_t<false, 64>(a, win, st);
}

static hipError_t launch_scan_win(const FwdArgs &a, const Window &win, hipStream_t st) {
    if (a.bf16) return a.dk == 128 ? launch_scan_t<true, 128>(a, win, st) : launch_scan_t<true, 64>(a, win, st);
    return a.dk == 128 ? launch_scan_t<false, 128>(a, win, st) : launch_scan_t<false, 64>(a, win, st);
}

hipError_t launch_fwd_local(const FwdArgs &a, hipStream_t st) { return launch_local_win(a, full_window(a), st); }

hipError_t launch_fwd_scan(const FwdArgs &a, hipStream_t st) { return launch_scan_win(a, full_window(a), st); }

hipError_t launch_fwd_segment_map(const FwdArgs &a, hipStream_t st) {
    const Window win = full_window(a);
    if (a.bf16) return a.dk == 128 ? launch_scan_t<true, 128, true>(a, win, st) : launch_scan_t<true, 64, true>(a, win, st);
    return a.dk == 128 ? launch_scan_t<false, 128, true>(a, win, st) : launch_scan_t<false, 64, true>(a, win, st);
}

hipError_t launch_fwd(const FwdArgs &a, size_t ws_bytes, hipStream_t st) {
    WindowPlan p;
    if (!plan_fwd_windows(a.bf16, a.dk, a.B, a.T, a.H, a.N, a.cu_seqlens != nullptr, a.sN != nullptr, ws_bytes, p))
        return hipErrorInvalidValue;  // the caller checks the workspace first
    FwdArgs b = a;
    if (p.nwin > 1 && p.carry) b.sN = reinterpret_cast<float *>(static_cast<char *>(a.ws) + p.carry_off);
    for (int w = 0; w < (int)p.nwin; ++w) {
        const Window win = make_window(b, p.Wc, w);
        hipError_t e = launch_local_win(b, win, st);
        if (e == hipSuccess) e = launch_scan_win(b, win, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
