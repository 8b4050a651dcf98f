// W4A8 decode GEMV (M = 1) for Q4_0 and affine 4-bit weights.
//
// tract PR #2432 ("The kernel"; follow-up decode measurements): the decode
// product streams the 4-bit weights once, takes an exact int8 dot per
// 32-weight block and rescales each block's integer in float; the per-call
// activation re-quantization is part of the overhead the page measures, so
// the fused variant here quantizes the activations inside the same launch.
// MLX PR #4802: affine groups add bias * sum(x), applied in the kernel.
//
// Mapping: a workgroup of W wavefronts owns W*R consecutive weight rows; each
// wavefront owns R rows. A row is K/32 chunks of 16 bytes (32 codes); lane l
// takes chunks l, l + 64, ... of each of its rows, so every load instruction
// of a wavefront reads 1 KiB of contiguous codes with 128-bit loads. All code
// and scale loads of a pass are issued before any arithmetic.
// While they are in flight the fused variant quantizes x into LDS (4 elements
// per thread, the lanes of one block combine maxima and sums by lane
// exchange); a large workgroup (16 wavefronts by default) shares that work.
// The plain variant reads each chunk's codes straight from global memory (or,
// as a tuning option, copies them to LDS first). Each lane reads its chunk's
// 32 codes once and reuses them for all R rows.
// The two nibble planes of a chunk pair with the two 16-byte halves of the
// activation block, so the unpack is one AND (low) and one shift + AND (high)
// per dword with no byte shuffles; eight v_dot4_i32_i8 give the block's
// integer dot. Float partial sums are reduced across the wavefront with DPP
// row operations and lane reads.
#include <stdio.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

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

constexpr int U = 2;  // chunks per lane per pass (a pass covers 64*U chunks = 4096 weights)
constexpr int EPT = 4;  // activations per thread while staging

// Stage the activation codes of the whole row in LDS.
// FUSED: quantize x (float32 or bfloat16) per block of G, EPT elements per
// thread, the G/EPT lanes of a block combining maxima and sums by lane
// exchange; else copy xq / xs / xsum.
template <int G, int NT, bool FUSED, bool XBF16>
__device__ __forceinline__ void stage_activations(int K, const void* __restrict__ x, const int8_t* __restrict__ xq,
                                                  const float* __restrict__ xs, const int32_t* __restrict__ xsum,
                                                  int8_t* xq_l, float* xs_l, int32_t* xsum_l, int8_t* xq_out,
                                                  float* xs_out, int32_t* xsum_out) {
    const int tid = threadIdx.x;
    const int ngroups = K / G;
    if (FUSED) {
        constexpr int L = G / EPT;  // lanes per block
        const bool out = xq_out != nullptr && blockIdx.x == 0;
        for (int u = tid; u < K / EPT; u += NT) {
            float v[EPT];
            if (XBF16) {
                const uint2 p = reinterpret_cast<const uint2*>(x)[u];
                v[0] = bf16_to_float(p.x & 0xFFFFu);
                v[1] = bf16_to_float(p.x >> 16);
                v[2] = bf16_to_float(p.y & 0xFFFFu);
                v[3] = bf16_to_float(p.y >> 16);
            } else {
                const float4 a = reinterpret_cast<const float4*>(x)[u];
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            }
            float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
            for (int off = 1; off < L; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
            const float s = amax / 127.0f;
            const float inv = act_inverse(s);
            uint32_t pk = 0;
            int sum = 0;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int c = (amax != 0.0f) ? act_code(v[i], s, inv) : 0;
                sum += c;
                pk |= (uint32_t)(c & 0xFF) << (8 * i);
            }
#pragma unroll
            for (int off = 1; off < L; off <<= 1) sum += __shfl_xor(sum, off, 64);
            reinterpret_cast<uint32_t*>(xq_l)[u] = pk;
            if (out) reinterpret_cast<uint32_t*>(xq_out)[u] = pk;
            if ((u & (L - 1)) == 0) {
                const int g = u / L;
                const float sv = (amax != 0.0f) ? s : 0.0f;
                xs_l[g] = sv;
                xsum_l[g] = sum;
                if (out) {
                    xs_out[g] = sv;
                    xsum_out[g] = sum;
                }
            }
        }
    } else {
        for (int u = tid; u < (K >> 4); u += NT)
            reinterpret_cast<uint4*>(xq_l)[u] = reinterpret_cast<const uint4*>(xq)[u];
        for (int g = tid; g < ngroups; g += NT) {
            if (xs) xs_l[g] = xs[g];
            xsum_l[g] = xsum[g];
        }
    }
}

// FMT 0: Q4_0 (G = 32, fp16 scale, value d * (q - 8)); FMT 1: affine (G = 64
// or 128, bf16 scale s and bias b, value s * q + b). WAVES wavefronts per
// workgroup, R rows per wavefront. LDS_ACT: activations staged in LDS (always
// for FUSED); otherwise each lane reads its chunk's codes from global memory.
template <int FMT, int G, int R, int WAVES, bool FUSED, bool LDS_ACT, bool XBF16, bool PARTIALS>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(
    int K, int N, const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wscale,
    const uint16_t* __restrict__ wbias, const void* __restrict__ x, const int8_t* __restrict__ xq,
    const float* __restrict__ xs, const int32_t* __restrict__ xsum, float* __restrict__ y,
    int32_t* __restrict__ partials, int8_t* __restrict__ xq_out, float* __restrict__ xs_out,
    int32_t* __restrict__ xsum_out) {
    constexpr int CPG = G / 32;  // chunks per block / group
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    int8_t* xq_l = lds;                                           // K bytes
    float* xs_l = reinterpret_cast<float*>(lds + K);             // K/G floats
    int32_t* xsum_l = reinterpret_cast<int32_t*>(xs_l + K / G);  // K/G ints

    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * WAVES + (threadIdx.x >> 6)) * R;
    const int nchunks = K >> 5;
    const int ngroups = K / G;
    const size_t rowbytes = (size_t)(K >> 1);

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    for (int c0 = 0; c0 < nchunks; c0 += 64 * U) {
        uint4 w[R][U];
        float sc[R][U], sb[R][U];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int n = row0 + r, c = c0 + lane + 64 * u;
                sc[r][u] = sb[r][u] = 0.0f;
                if (n < N && c < nchunks) {
                    w[r][u] = *reinterpret_cast<const uint4*>(wq + (size_t)n * rowbytes + 16 * (size_t)c);
                    if (!PARTIALS) {
                        const size_t si = (size_t)n * ngroups + c / CPG;
                        if (FMT == 0) {
                            sc[r][u] = half_to_float(wscale[si]);
                        } else {
                            sc[r][u] = bf16_to_float(wscale[si]);
                            sb[r][u] = bf16_to_float(wbias[si]);
                        }
                    }
                } else {
                    w[r][u] = make_uint4(0, 0, 0, 0);
                }
            }
        if (LDS_ACT && c0 == 0) {
            stage_activations<G, 64 * WAVES, FUSED, XBF16>(K, x, xq, xs, xsum, xq_l, xs_l, xsum_l, xq_out, xs_out,
                                                           xsum_out);
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const bool valid = c < nchunks;
            uint4 xa = make_uint4(0, 0, 0, 0), xb = xa;
            float a = 0.0f;
            int s = 0;
            if (valid) {
                if (LDS_ACT) {
                    xa = *reinterpret_cast<const uint4*>(xq_l + 32 * c);
                    xb = *reinterpret_cast<const uint4*>(xq_l + 32 * c + 16);
                    if (!PARTIALS) a = xs_l[c / CPG];
                    s = xsum_l[c / CPG];
                } else {
                    xa = *reinterpret_cast<const uint4*>(xq + 32 * c);
                    xb = *reinterpret_cast<const uint4*>(xq + 32 * c + 16);
                    if (!PARTIALS) a = xs[c / CPG];
                    s = xsum[c / CPG];
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int dot = dot_chunk(w[r][u], xa, xb);
                if (PARTIALS) {
                    int p = dot;
                    if (FMT == 0) {
                        p = dot - 8 * s;
                    } else {
#pragma unroll
                        for (int off = 1; off < CPG; off <<= 1) p += __shfl_xor(p, off, 64);
                    }
                    const int n = row0 + r;
                    if (valid && n < N && (c % CPG) == 0) partials[(size_t)n * ngroups + c / CPG] = p;
                } else if (FMT == 0) {
                    const int p = dot - 8 * s;  // sum (q - 8) * xq over the block
                    acc[r] += (sc[r][u] * a) * (float)p;
                } else {
                    acc[r] += a * (sc[r][u] * (float)dot);
                    if ((c % CPG) == 0) acc[r] += a * (sb[r][u] * (float)s);  // bias * dequantized sum x
                }
            }
        }
    }
    if (!PARTIALS) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float t = wave_sum(acc[r]);
            if (lane == 0 && row0 + r < N) y[row0 + r] = t;
        }
    }
}

// Launch shape: (rows per wave, waves per workgroup, activations in LDS).
struct GemvShape {
    int r, waves, lds;
};

GemvShape gemv_shape(bool fused) {
    static int cfg[2][3] = {{-1, -1, -1}, {-1, -1, -1}};
    int* c = cfg[fused ? 1 : 0];
    if (c[0] < 0) {
        // defaults; the environment variables are tuning knobs only
        c[0] = 1;
        c[1] = fused ? 16 : 8;
        c[2] = fused ? 1 : 0;
        const char* e = getenv(fused ? "Q4_GEMV_FUSED_SHAPE" : "Q4_GEMV_SHAPE");  // "R,WAVES,LDS"
        int r, w, l;
        if (e && sscanf(e, "%d,%d,%d", &r, &w, &l) == 3 && (r == 1 || r == 2 || r == 4) &&
            (w == 4 || w == 8 || w == 16)) {
            c[0] = r;
            c[1] = w;
            c[2] = fused ? 1 : (l != 0);
        }
    }
    return GemvShape{c[0], c[1], c[2]};
}

template <int FMT, int G, int R, int WAVES, bool FUSED, bool LDS_ACT, bool XBF16, bool PARTIALS>
hipError_t launch_one(int K, int N, const uint8_t* wq, const void* wscale, const void* wbias, const void* x,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      int8_t* xq_out, float* xs_out, int32_t* xsum_out, hipStream_t stream) {
    const dim3 grid((unsigned)((N + WAVES * R - 1) / (WAVES * R))), block(64 * WAVES);
    const size_t lds = LDS_ACT ? (size_t)K + 8 * (size_t)(K / G) : 0;
    hipLaunchKernelGGL((gemv_kernel<FMT, G, R, WAVES, FUSED, LDS_ACT, XBF16, PARTIALS>), grid, block, lds, stream, K,
                       N, wq, static_cast<const uint16_t*>(wscale), static_cast<const uint16_t*>(wbias), x, xq, xs,
                       xsum, y, partials, xq_out, xs_out, xsum_out);
    return hipGetLastError();
}

template <int FMT, int G, int WAVES, bool FUSED, bool LDS_ACT, bool XBF16, bool PARTIALS>
hipError_t launch_r(int r, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias, const void* x,
                    const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                    int8_t* xq_out, float* xs_out, int32_t* xsum_out, hipStream_t stream) {
    if (r == 2)
        return launch_one<FMT, G, 2, WAVES, FUSED, LDS_ACT, XBF16, PARTIALS>(K, N, wq, wscale, wbias, x, xq, xs, xsum,
                                                                            y, partials, xq_out, xs_out, xsum_out,
                                                                            stream);
    if (r == 4)
        return launch_one<FMT, G, 4, WAVES, FUSED, LDS_ACT, XBF16, PARTIALS>(K, N, wq, wscale, wbias, x, xq, xs, xsum,
                                                                            y, partials, xq_out, xs_out, xsum_out,
                                                                            stream);
    return launch_one<FMT, G, 1, WAVES, FUSED, LDS_ACT, XBF16, PARTIALS>(K, N, wq, wscale, wbias, x, xq, xs, xsum, y,
                                                                        partials, xq_out, xs_out, xsum_out, stream);
}

template <int FMT, int G, bool FUSED, bool LDS_ACT, bool XBF16, bool PARTIALS>
hipError_t launch_w(GemvShape sh, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                    const void* x, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                    int32_t* partials, int8_t* xq_out, float* xs_out, int32_t* xsum_out, hipStream_t stream) {
    if (sh.waves == 8)
        return launch_r<FMT, G, 8, FUSED, LDS_ACT, XBF16, PARTIALS>(sh.r, K, N, wq, wscale, wbias, x, xq, xs, xsum, y,
                                                                   partials, xq_out, xs_out, xsum_out, stream);
    if (sh.waves == 16)
        return launch_r<FMT, G, 16, FUSED, LDS_ACT, XBF16, PARTIALS>(sh.r, K, N, wq, wscale, wbias, x, xq, xs, xsum,
                                                                    y, partials, xq_out, xs_out, xsum_out, stream);
    return launch_r<FMT, G, 4, FUSED, LDS_ACT, XBF16, PARTIALS>(sh.r, K, N, wq, wscale, wbias, x, xq, xs, xsum, y,
                                                               partials, xq_out, xs_out, xsum_out, stream);
}

template <int FMT, int G>
hipError_t launch_fmt(int K, int N, const uint8_t* wq, const void* wscale, const void* wbias, const int8_t* xq,
                      const float* xs, const int32_t* xsum, float* y, int32_t* partials, hipStream_t stream) {
    const GemvShape sh = gemv_shape(false);
    if (partials)  // the partials view reads the codes straight from global memory
        return launch_r<FMT, G, 4, false, false, false, true>(1, K, N, wq, wscale, wbias, nullptr, xq, xs, xsum, y,
                                                             partials, nullptr, nullptr, nullptr, stream);
    if (sh.lds)
        return launch_w<FMT, G, false, true, false, false>(sh, K, N, wq, wscale, wbias, nullptr, xq, xs, xsum, y,
                                                          nullptr, nullptr, nullptr, nullptr, stream);
    return launch_w<FMT, G, false, false, false, false>(sh, K, N, wq, wscale, wbias, nullptr, xq, xs, xsum, y,
                                                       nullptr, nullptr, nullptr, nullptr, stream);
}

template <int FMT, int G>
hipError_t launch_fused_fmt(int K, int N, bool xbf16, const void* x, const uint8_t* wq, const void* wscale,
                            const void* wbias, float* y, int8_t* xq_out, float* xs_out, int32_t* xsum_out,
                            hipStream_t stream) {
    const GemvShape sh = gemv_shape(true);
    if (xbf16)
        return launch_w<FMT, G, true, true, true, false>(sh, K, N, wq, wscale, wbias, x, nullptr, nullptr, nullptr, y,
                                                        nullptr, xq_out, xs_out, xsum_out, stream);
    return launch_w<FMT, G, true, true, false, false>(sh, K, N, wq, wscale, wbias, x, nullptr, nullptr, nullptr, y,
                                                     nullptr, xq_out, xs_out, xsum_out, stream);
}

}  // namespace

hipError_t launch_gemv(int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale, const void* wbias,
                       const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                       hipStream_t stream) {
    if (fmt == 0) return launch_fmt<0, 32>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_fmt<1, 64>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_fmt<1, 128>(K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_fused(int K, int N, int bs, int fmt, bool xbf16, const void* x, const uint8_t* wq,
                             const void* wscale, const void* wbias, float* y, int8_t* xq_out, float* xs_out,
                             int32_t* xsum_out, hipStream_t stream) {
    if (fmt == 0)
        return launch_fused_fmt<0, 32>(K, N, xbf16, x, wq, wscale, wbias, y, xq_out, xs_out, xsum_out, stream);
    if (bs == 64)
        return launch_fused_fmt<1, 64>(K, N, xbf16, x, wq, wscale, wbias, y, xq_out, xs_out, xsum_out, stream);
    if (bs == 128)
        return launch_fused_fmt<1, 128>(K, N, xbf16, x, wq, wscale, wbias, y, xq_out, xs_out, xsum_out, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
