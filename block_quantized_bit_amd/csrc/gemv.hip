// W4A8 decode GEMV (M = 1) for Q4_0 and affine 4-bit weights.
//
// tract PR #2432 ("The kernel"; follow-up decode measurements): the decode
// product streams the 4-bit weights once, takes an exact int8 dot per
// 32-weight block and rescales each block's integer in float. MLX PR #4802:
// affine groups add bias * sum(x), applied in the kernel.
//
// Mapping: one wavefront per weight row. A row is K/32 chunks of 16 bytes
// (32 codes each); lane l takes chunks l, l + 64, ... so every load
// instruction of a wavefront reads 1 KiB of contiguous codes with 128-bit
// loads. The two nibble planes of a chunk pair with the two 16-byte halves of
// the activation block, so the unpack is one AND (low) and one shift + AND
// (high) per dword and no byte shuffles; eight v_dot4_i32_i8 give the block's
// integer dot. The float partial sums are reduced across the wavefront with
// DPP row operations and lane reads.
#include "common.h"
#include "kernels.h"

namespace q4 {

__device__ __forceinline__ int dot_chunk(const uint4& w, const uint4& xa, const uint4& xb) {
    int d = 0;
    d = __builtin_amdgcn_sdot4((int)lo_nibbles(w.x), (int)xa.x, d, false);
    d = __builtin_amdgcn_sdot4((int)lo_nibbles(w.y), (int)xa.y, d, false);
    d = __builtin_amdgcn_sdot4((int)lo_nibbles(w.z), (int)xa.z, d, false);
    d = __builtin_amdgcn_sdot4((int)lo_nibbles(w.w), (int)xa.w, d, false);
    d = __builtin_amdgcn_sdot4((int)hi_nibbles(w.x), (int)xb.x, d, false);
    d = __builtin_amdgcn_sdot4((int)hi_nibbles(w.y), (int)xb.y, d, false);
    d = __builtin_amdgcn_sdot4((int)hi_nibbles(w.z), (int)xb.z, d, false);
    d = __builtin_amdgcn_sdot4((int)hi_nibbles(w.w), (int)xb.w, d, false);
    return d;
}

// FMT 0: Q4_0 (G = 32, fp16 scale, value d * (q - 8)); FMT 1: affine (G = 64
// or 128, bf16 scale s and bias b, value s * q + b).
template <int FMT, int G, bool PARTIALS>
__global__ __launch_bounds__(256) void gemv_kernel(int K, int N, const uint8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ wscale,
                                                   const uint16_t* __restrict__ wbias, const int8_t* __restrict__ xq,
                                                   const float* __restrict__ xs, const int32_t* __restrict__ xsum,
                                                   float* __restrict__ y, int32_t* __restrict__ partials) {
    constexpr int CPG = G / 32;  // chunks per block / group
    constexpr int U = 2;         // chunks per lane per iteration, loads issued together
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;  // whole wavefront
    const int nchunks = K >> 5;
    const int ngroups = K / G;
    const uint4* row = reinterpret_cast<const uint4*>(wq + (size_t)n * (size_t)(K >> 1));
    const uint4* xv = reinterpret_cast<const uint4*>(xq);
    const size_t sbase = (size_t)n * (size_t)ngroups;

    float acc = 0.0f;
    for (int c0 = 0; c0 < nchunks; c0 += 64 * U) {
        uint4 w[U], xa[U], xb[U];
        float sc[U], sb[U], a[U];
        int s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            if (c < nchunks) {
                const int gi = c / CPG;
                w[u] = row[c];
                xa[u] = xv[2 * c];
                xb[u] = xv[2 * c + 1];
                if (!PARTIALS) {
                    if (FMT == 0) {
                        sc[u] = half_to_float(wscale[sbase + gi]);
                    } else {
                        sc[u] = bf16_to_float(wscale[sbase + gi]);
                        sb[u] = bf16_to_float(wbias[sbase + gi]);
                    }
                    a[u] = xs[gi];
                }
                s[u] = xsum[gi];
            } else {
                w[u] = make_uint4(0, 0, 0, 0);
                xa[u] = w[u];
                xb[u] = w[u];
                sc[u] = sb[u] = a[u] = 0.0f;
                s[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const int dot = dot_chunk(w[u], xa[u], xb[u]);
            if (PARTIALS) {
                int p = dot;
                if (FMT == 0) {
                    p = dot - 8 * s[u];
                } else {
                    // chunks of one group sit in CPG consecutive lanes
#pragma unroll
                    for (int off = 1; off < CPG; off <<= 1) p += __shfl_xor(p, off, 64);
                }
                if (c < nchunks && (c % CPG) == 0) partials[sbase + c / CPG] = p;
            } else if (c < nchunks) {
                if (FMT == 0) {
                    const int p = dot - 8 * s[u];            // sum (q - 8) * xq over the block
                    acc += (sc[u] * a[u]) * (float)p;
                } else {
                    acc += a[u] * (sc[u] * (float)dot);
                    if ((c % CPG) == 0) acc += a[u] * (sb[u] * (float)s[u]);  // bias * dequantized sum x
                }
            }
        }
    }
    if (!PARTIALS) {
        acc = wave_sum(acc);
        if (lane == 0) y[n] = acc;
    }
}

template <int FMT, int G>
static hipError_t launch_fmt(int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                             const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                             hipStream_t stream) {
    const dim3 grid((unsigned)((N + 3) / 4)), block(256);
    const uint16_t* ws = static_cast<const uint16_t*>(wscale);
    const uint16_t* wb = static_cast<const uint16_t*>(wbias);
    if (partials)
        hipLaunchKernelGGL((gemv_kernel<FMT, G, true>), grid, block, 0, stream, K, N, wq, ws, wb, xq, xs, xsum, y,
                           partials);
    else
        hipLaunchKernelGGL((gemv_kernel<FMT, G, false>), grid, block, 0, stream, K, N, wq, ws, wb, xq, xs, xsum, y,
                           partials);
    return hipGetLastError();
}

hipError_t launch_gemv(int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale, const void* wbias,
                       const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                       hipStream_t stream) {
    if (fmt == 0) return launch_fmt<0, 32>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_fmt<1, 64>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_fmt<1, 128>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
