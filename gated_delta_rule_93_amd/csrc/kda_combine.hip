// kda_combine.hip -- one hop of the prefix over the segments of a chain: the state that leaves a
// segment whose affine map is (A, B) when S enters it, out = A S + B, in fp32.
//
// Blog post-114, chapter 3: the chunked form computes the blocks' contributions in parallel and
// merges them into the state one block after the other, and K3's KCP carries that idea across
// devices.  With a device's segment taken as one block, its contribution is the affine map
// S_out = A S_in + B (A = d_k x d_k, B = d_k x d_v), formed by the state scan's segment-map mode;
// what stays serial across the segments is this product, one per segment boundary.
//
// One 256-thread workgroup per 32 x 32 tile of one map's output.  Row block i0.. of A and column
// block j0.. of S are staged in LDS; each thread forms 4 adjacent outputs with fused multiply-adds
// over k in ascending order, then adds B (a fixed order: the result is reproducible).  With B
// absent the same kernel composes two maps' linear parts (A2 A1), the step of a tree-shaped prefix.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {
constexpr int kTile = 32;
}

template <int D>
__global__ void __launch_bounds__(256) state_combine_kernel(const float *__restrict__ A, const float *__restrict__ S,
                                                            const float *B, float *out) {
    constexpr int NT = D / kTile;
    __shared__ __attribute__((aligned(16))) float As[kTile][D + 4];  // rows i0 .. i0 + 31 of A
    __shared__ __attribute__((aligned(16))) float Ss[D][kTile + 4];  // columns j0 .. j0 + 31 of S
    const long c = blockIdx.x / (NT * NT);
    const int tile = blockIdx.x % (NT * NT), i0 = (tile / NT) * kTile, j0 = (tile % NT) * kTile;
    const float *Ac = A + c * D * D, *Sc = S + c * D * D;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < kTile * D / 4; idx += 256) {
        const int r = idx / (D / 4), c4 = idx % (D / 4);
        *reinterpret_cast<float4 *>(&As[r][4 * c4]) = *reinterpret_cast<const float4 *>(Ac + (long)(i0 + r) * D + 4 * c4);
    }
    for (int idx = tid; idx < D * kTile / 4; idx += 256) {
        const int r = idx / (kTile / 4), c4 = idx % (kTile / 4);
        *reinterpret_cast<float4 *>(&Ss[r][4 * c4]) = *reinterpret_cast<const float4 *>(Sc + (long)r * D + j0 + 4 * c4);
    }
    __syncthreads();
    const int ty = tid >> 3, tx = tid & 7;  // output row i0 + ty, columns j0 + 4 tx .. + 3
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int k = 0; k < D; ++k) {
        const float a = As[ty][k];
        const float4 s = *reinterpret_cast<const float4 *>(&Ss[k][4 * tx]);
        acc.x = fmaf(a, s.x, acc.x);
        acc.y = fmaf(a, s.y, acc.y);
        acc.z = fmaf(a, s.z, acc.z);
        acc.w = fmaf(a, s.w, acc.w);
    }
    const long off = c * D * D + (long)(i0 + ty) * D + j0 + 4 * tx;
    const float4 b = B ? *reinterpret_cast<const float4 *>(B + off)  // read before the write: out may be B
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4 *>(out + off) = make_float4(acc.x + b.x, acc.y + b.y, acc.z + b.z, acc.w + b.w);
}

hipError_t launch_state_combine(int count, int d, const float *A, const float *S, const float *B, float *out,
                                hipStream_t st) {
    if (count <= 0) return hipSuccess;
    const unsigned tiles = (unsigned)((d / kTile) * (d / kTile));
    const dim3 grid((unsigned)count * tiles);
    if (d == 128) return launch_kernel(state_combine_kernel<128>, grid, dim3(256), st, A, S, B, out);
    return launch_kernel(state_combine_kernel<64>, grid, dim3(256), st, A, S, B, out);
}

}  // namespace kda
