// kda_common.h -- device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kWave = 64;
constexpr int kChunk = 64;         // tokens per chunk
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite values; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float round_bf16(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// Element loads/stores for the io dtype (float or bf16 stored as uint16_t).
template <typename T> struct IO;
template <> struct IO<float> {
    static __device__ __forceinline__ float load(const float *p, long i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, long i, float x) { p[i] = x; }
};
template <> struct IO<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p, long i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t *p, long i, float x) {
        p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);  // v_cvt_pk_bf16_f32: round to nearest even
    }
};

// 4 consecutive elements as fp32 (p 8-byte aligned for bf16, 16-byte for fp32)
__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const uint16_t *p) {
    uint2 w = *reinterpret_cast<const uint2 *>(p);
    f32x4 r;
    r.x = __uint_as_float(w.x << 16);
    r.y = __uint_as_float(w.x & 0xffff0000u);
    r.z = __uint_as_float(w.y << 16);
    r.w = __uint_as_float(w.y & 0xffff0000u);
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLn2 = 0.6931471805599453f;

// log(alpha) of the low-rank gate from its pre-activation x: -softplus(x) = -log(1 + e^x),
// evaluated as -(max(x, 0) + log(1 + e^{-|x|})) with the hardware base-2 exp and log, so no
// intermediate overflows.  The gate prologue and the fused chunk-local kernel both call this
// one function, so the log-decay they produce is bitwise the same.
__device__ __forceinline__ float gate_log_alpha(float x) {
    const float e = fast_exp2(-fabsf(x) * kLog2e);  // in (0, 1]
    return -(fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2);
}

// ---------------------------------------------------------------- MFMA operand fragments
//
// One fragment holds, for one lane, the 8 "k-slot" values of a 16 x 32 (rows x k) operand
// block.  Lane l = 16 * grp + r16 supplies row (or column, for the B operand) r16 and
// k-slots s = 0..7 which stand for the k-index
//        k = 16 * (s >> 2) + 4 * grp + (s & 3)        (within the 32-wide k block).
// The A and B operands of one product always use this same map, so the MFMA sums over
// all 32 k indices whatever the hardware's own k order is.  The map is chosen so that an
// accumulator (lane l holds rows 4 * grp + i, column r16 of a 16 x 16 tile) of two
// vertically adjacent tiles is, without any data movement, the B operand of the next
// product whose k dimension is those 32 rows.
//
// Precision modes:
//   Frag<float>:  fp32 values; one product is 8 v_mfma_f32_16x16x4_f32.
//   FragB:        one bf16x8; one product is one v_mfma_f32_16x16x32_bf16.
//   Frag2:        bf16 hi + lo split of fp32 values (hi = bf16(x), lo = bf16(x - hi)),
//                 giving ~16 significant bits; products use hi*hi + hi*lo + lo*hi.

struct FragF { float v[8]; };
struct FragB { bf16x8 h; };
struct Frag2 { bf16x8 h, l; };

__device__ __forceinline__ bf16x8 to_bf16x8(const float *x) {
    bf16x8 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = (__bf16)x[s];
    return r;
}

__device__ __forceinline__ FragB make_fragB(const float *x) { return FragB{to_bf16x8(x)}; }

// Two fp32 values rounded to nearest-even bf16, packed (a in the low half): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// hi = bf16(x), lo = bf16(x - hi), element by element.  Written per pair so that the rounded pair
// is converted once and its two values are read back from the packed word (a shift and a mask).
__device__ __forceinline__ Frag2 make_frag2(const float *x) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t h = pk_bf16(x[2 * p], x[2 * p + 1]);
        const float f0 = __uint_as_float(h << 16), f1 = __uint_as_float(h & 0xffff0000u);
        hw[p] = h;
        lw[p] = pk_bf16(x[2 * p] - f0, x[2 * p + 1] - f1);
    }
    Frag2 f;
    f.h = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    f.l = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    return f;
}
__device__ __forceinline__ FragF make_fragF(const float *x) {
    FragF f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f.v[s] = x[s];
    return f;
}

// Fragment from stored bf16 bits: slots 0..3 from `lo` (4 consecutive elements of the k block,
// starting at 4 grp), slots 4..7 from `hi` (starting at 16 + 4 grp), as the k-slot map requires.
__device__ __forceinline__ FragB frag_bits(uint2 lo, uint2 hi) {
    return FragB{__builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y))};
}

__device__ __forceinline__ f32x4 mfma(const FragB &a, const FragB &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const Frag2 &a, const Frag2 &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.l, b.h, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const Frag2 &a, const FragB &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.l, b.h, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const FragB &a, const Frag2 &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.h, b.h, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const FragF &a, const FragF &b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
    return c;
}

// k index (0..31) of slot s for lane group grp
__device__ __forceinline__ int kslot(int grp, int s) { return 16 * (s >> 2) + 4 * grp + (s & 3); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Index of the calling wave in its one-dimensional workgroup, as a scalar (wave-uniform) value, so
// that branches on it compile to scalar branches, not to EXEC-masked regions.  An MFMA under an
// EXEC-masked branch whose result is used after the branch was observed to give wrong results;
// with a scalar condition no such region is formed.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

}  // namespace kda
