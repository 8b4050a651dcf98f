// Per-block int8 quantization of activations (tract PR #2432, pipeline
// figure: "activation -> int8, per-block"; MLX PR #4802: x quantized to int8).
//
// Each thread owns 8 consecutive elements of the flattened [M][K] array; the
// bs/8 threads of one block are consecutive lanes of a wavefront and combine
// their maxima and code sums with lane exchanges. Loads are 16 bytes per
// thread (bf16) or 2 x 16 bytes (f32); the 8 codes are written with one
// 8-byte store. The block scale is amax / 127 in correctly rounded float32 and
// every code is round-half-even of a correctly rounded float32 quotient
// (act_code: a reciprocal multiply, with the exact quotient near ties).
// GM: the scales and code sums are written group-major, [K/bs][M], which is
// the layout the packed-weight GEMM stages with contiguous loads.
#include "common.h"
#include "kernels.h"

namespace q4 {

template <int BS, bool BF16, bool GM>
__global__ __launch_bounds__(256) void quantize_act_kernel(long long nthreads, const void* __restrict__ x,
                                                           int8_t* __restrict__ xq, float* __restrict__ xs,
                                                           int32_t* __restrict__ xsum, int M, int ngroups) {
    constexpr int L = BS / 8;  // lanes per block
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nthreads) return;  // the element count is a multiple of BS: whole blocks exit together

    float v[8];
    if (BF16) {
        uint4 p = reinterpret_cast<const uint4*>(x)[t];
        uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_float(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_float(w[i] >> 16);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(x) + 2 * t;
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int off = 1; off < L; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));

    const float s = amax / 127.0f;  // correctly rounded float32 division
    const float inv = act_inverse(s);
    int q[8];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // round half to even of the correctly rounded float32 quotient v / s
        const int c = (amax != 0.0f) ? act_code(v[i], s, inv) : 0;
        q[i] = c;
        sum += c;
    }
#pragma unroll
    for (int off = 1; off < L; off <<= 1) sum += __shfl_xor(sum, off, 64);

    uint32_t lo = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
                  ((uint32_t)(q[3] & 0xFF) << 24);
    uint32_t hi = (uint32_t)(q[4] & 0xFF) | ((uint32_t)(q[5] & 0xFF) << 8) | ((uint32_t)(q[6] & 0xFF) << 16) |
                  ((uint32_t)(q[7] & 0xFF) << 24);
    reinterpret_cast<uint2*>(xq)[t] = make_uint2(lo, hi);
    if ((threadIdx.x & (L - 1)) == 0) {
        long long blk = t / L;
        if (GM) {
            const long long m = blk / ngroups;
            blk = (blk - m * ngroups) * M + m;
        }
        xs[blk] = (amax != 0.0f) ? s : 0.0f;
        xsum[blk] = sum;
    }
}

template <int BS, bool GM>
static hipError_t launch_bs(int M, int K, bool bf16, const void* x, int8_t* xq, float* xs, int32_t* xsum,
                            hipStream_t stream) {
    const long long nthreads = (long long)M * K / 8;
    const unsigned grid = (unsigned)((nthreads + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL((quantize_act_kernel<BS, true, GM>), dim3(grid), dim3(256), 0, stream, nthreads, x, xq, xs,
                           xsum, M, K / BS);
    else
        hipLaunchKernelGGL((quantize_act_kernel<BS, false, GM>), dim3(grid), dim3(256), 0, stream, nthreads, x, xq, xs,
                           xsum, M, K / BS);
    return hipGetLastError();
}

template <bool GM>
static hipError_t launch_layout(int M, int K, int bs, bool bf16, const void* x, int8_t* xq, float* xs, int32_t* xsum,
                                hipStream_t stream) {
    switch (bs) {
        case 32: return launch_bs<32, GM>(M, K, bf16, x, xq, xs, xsum, stream);
        case 64: return launch_bs<64, GM>(M, K, bf16, x, xq, xs, xsum, stream);
        case 128: return launch_bs<128, GM>(M, K, bf16, x, xq, xs, xsum, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantize_act(int M, int K, int bs, bool bf16, const void* x, int8_t* xq, float* xs, int32_t* xsum,
                               hipStream_t stream) {
    return launch_layout<false>(M, K, bs, bf16, x, xq, xs, xsum, stream);
}

hipError_t launch_quantize_act_gm(int M, int K, int bs, bool bf16, const void* x, int8_t* xq, float* xs,
                                  int32_t* xsum, hipStream_t stream) {
    return launch_layout<true>(M, K, bs, bf16, x, xq, xs, xsum, stream);
}

}  // namespace q4
