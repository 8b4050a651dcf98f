// W4A8 GEMM for a few activation rows (M <= 32): the regime between the
// decode GEMV (M = 1) and the tiled prefill GEMM.
//
// tract PR #2432 (follow-up decode measurements): the weights dominate the
// traffic of a decode-sized product, so they must be streamed once.
// MLX PR #4802: below M = 32 its int8 path is not taken and x is dequantized
// instead; here the int8 path covers every M.
//
// A workgroup owns 16 output columns and all M rows, so every weight block is
// read once for all rows. Its 8 wavefronts split K into contiguous ranges of
// whole blocks or groups; each runs v_mfma_i32_16x16x32_i8 (16 rows x 16
// columns x one 32-weight block) per K step, with one or two 16-row tiles.
// The wavefronts' float partial sums are added in LDS in a fixed order (no
// atomics, so results do not depend on scheduling).
//
// Operands of the 16x16x32 int8 MFMA (lane l, q = l / 16): A holds row l % 16
// and k = 8q .. 8q+7 of the step; B holds column l % 16 and the same k; D
// holds column l % 16, rows 4q .. 4q+3. In the 16-byte code chunk of a 32-weight
// block, weight k < 16 is the low nibble of byte k and weight k >= 16 the high
// nibble of byte k - 16, so lane q loads the 8 bytes at 8 * (q & 1) and keeps
// nibble plane q >> 1: one shift and one AND per dword, no byte shuffles.
//
// Rescale after each block (Q4_0) or group (affine, 2 or 4 MFMA steps):
//   acc += xs[m] * (d[n] * P)          Q4_0 (P from codes q - 8)
//   acc += xs[m] * (s[n] * A) + (xs * xsum)[m] * b[n]   affine
// The activation scales (and xs * xsum) of all rows are staged in LDS once.
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int SW = 8;          // wavefronts per workgroup, each with a contiguous K range
constexpr int SNT = 64 * SW;   // threads per workgroup
constexpr int SN = 16;         // output columns per workgroup
constexpr int PS = 16;         // K steps whose loads are issued together
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data format
constexpr uint32_t OUT = 0x80000000u;   // beyond every buffer range: reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

template <int FMT, int G, int MT, bool PARTIALS>
__global__ __launch_bounds__(SNT, 1) void gemm_small_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                            const uint16_t* __restrict__ wscale,
                                                            const uint16_t* __restrict__ wbias,
                                                            const int8_t* __restrict__ xq,
                                                            const float* __restrict__ xs,
                                                            const int32_t* __restrict__ xsum, float* __restrict__ y,
                                                            int32_t* __restrict__ partials) {
    constexpr int SPG = G / 32;     // MFMA steps per block or group
    constexpr bool AFF = FMT == 1;
    constexpr int MR = 16 * MT;     // rows covered by the MFMA tiles
    static_assert(PS % SPG == 0, "a load pass holds whole groups");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ngroups = K / G;
    float* sxs = reinterpret_cast<float*>(smem);                  // [ngroups][MR]
    float* sxb = sxs + (size_t)ngroups * MR;                      // [ngroups][MR], affine
    float* red = sxs + (size_t)ngroups * MR * (AFF ? 2 : 1);      // [SW][MT][16 x 16]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int n = blockIdx.x * SN + c;

    // this wavefront's groups [gb, ge) and K steps [sb, se)
    const int gpw = (ngroups + SW - 1) / SW;
    const int gb = min(ngroups, wave * gpw), ge = min(ngroups, gb + gpw);
    const int sb = gb * SPG, se = ge * SPG;

    const __amdgpu_buffer_rsrc_t r_b = rsrc(wq, (uint32_t)((size_t)N * (K / 2)));
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)((size_t)M * K));
    const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, PARTIALS ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    const __amdgpu_buffer_rsrc_t r_wb =
        rsrc(wbias, (PARTIALS || !AFF) ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    const uint32_t ob = (n < N) ? (uint32_t)(n * (K / 2) + 8 * (q & 1)) : OUT;  // + 16 per step
    const uint32_t os = (n < N) ? (uint32_t)(n * ngroups * 2) : OUT;            // + 2 per group
    uint32_t oa[MT];                                                              // + 32 per step
#pragma unroll
    for (int t = 0; t < MT; ++t) oa[t] = (16 * t + c < M) ? (uint32_t)((16 * t + c) * K + 8 * q) : OUT;
    const int shift = 4 * (q >> 1);

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    constexpr int GPP = PS / SPG;  // groups per pass
    uint2 wv[PS], av[PS][MT];
    uint32_t wsb[GPP], wbb[GPP];
    // issue one pass's loads; steps and groups past the range read zero
    auto load_pass = [&](int s0) {
#pragma unroll
        for (int p = 0; p < PS; ++p) {
            const bool in = s0 + p < se;
            wv[p] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r_b, in ? ob : OUT, (s0 + p) * 16, 0));
#pragma unroll
            for (int t = 0; t < MT; ++t)
                av[p][t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r_a, in ? oa[t] : OUT, (s0 + p) * 32, 0));
        }
#pragma unroll
        for (int u = 0; u < GPP; ++u) {
            const int g = s0 / SPG + u;
            const uint32_t o = (g < ge) ? os : OUT;
            if (!PARTIALS) {
                wsb[u] = __builtin_amdgcn_raw_buffer_load_b16(r_ws, o, g * 2, 0);
                wbb[u] = AFF ? __builtin_amdgcn_raw_buffer_load_b16(r_wb, o, g * 2, 0) : 0u;
            }
        }
    };

    // The first pass's weight loads go out before the activation scales are
    // staged, so the staging hides behind them.
    load_pass(sb);
    if (!PARTIALS) {
        // rows of xs (and xsum) are read along the groups, written transposed
        for (int i = tid; i < MR * ngroups; i += SNT) {
            const int m = i / ngroups, g = i - m * ngroups;
            float v = 0.0f, b = 0.0f;
            if (m < M) {
                v = xs[(size_t)m * ngroups + g];
                if (AFF) b = v * (float)xsum[(size_t)m * ngroups + g];
            }
            sxs[g * MR + m] = v;
            if (AFF) sxb[g * MR + m] = b;
        }
        __syncthreads();
    }

    for (int s0 = sb; s0 < se; s0 += PS) {
        if (s0 != sb) load_pass(s0);
#pragma unroll
        for (int u = 0; u < GPP; ++u) {
            const int g = s0 / SPG + u;
            v4i P[MT];
#pragma unroll
            for (int e = 0; e < SPG; ++e) {
                const int p = u * SPG + e;
                uint32_t lo = (wv[p].x >> shift) & 0x0F0F0F0Fu, hi = (wv[p].y >> shift) & 0x0F0F0F0Fu;
                if (FMT == 0) {
                    lo = minus8_bytes(lo);
                    hi = minus8_bytes(hi);
                }
                const long bop = (long)(((uint64_t)hi << 32) | lo);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const long aop = (long)(((uint64_t)av[p][t].y << 32) | av[p][t].x);
                    const v4i z = {0, 0, 0, 0};
                    P[t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, e == 0 ? z : P[t], 0, 0, 0);
                }
            }
            if (PARTIALS) {
                if (g < ge && n < N) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = 16 * t + 4 * q + r;
                            if (m < M) partials[((size_t)m * N + n) * ngroups + g] = P[t][r];
                        }
                }
                continue;
            }
            // groups past the range have zero codes and zero weight scale and bias
            const int gs = min(g, ngroups - 1);
            const float w = AFF ? bf16_to_float(wsb[u]) : half_to_float(wsb[u]);
            const float b = AFF ? bf16_to_float(wbb[u]) : 0.0f;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float4 xv = *reinterpret_cast<const float4*>(&sxs[gs * MR + 16 * t + 4 * q]);
                acc[t][0] += xv.x * (w * (float)P[t][0]);
                acc[t][1] += xv.y * (w * (float)P[t][1]);
                acc[t][2] += xv.z * (w * (float)P[t][2]);
                acc[t][3] += xv.w * (w * (float)P[t][3]);
                if (AFF) {
                    const float4 bv = *reinterpret_cast<const float4*>(&sxb[gs * MR + 16 * t + 4 * q]);
                    acc[t][0] += bv.x * b;
                    acc[t][1] += bv.y * b;
                    acc[t][2] += bv.z * b;
                    acc[t][3] += bv.w * b;
                }
            }
        }
    }
    if (PARTIALS) return;

    // combine the wavefronts' partial sums in wavefront order
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wave * MT + t) * 256 + (4 * q + r) * 16 + c] = acc[t][r];
    __syncthreads();
    for (int o = tid; o < MT * 256; o += SNT) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < SW; ++w) s += red[w * MT * 256 + o];
        const int m = 16 * (o >> 8) + ((o >> 4) & 15), nn = blockIdx.x * SN + (o & 15);
        if (m < M && nn < N) y[(size_t)m * N + nn] = s;
    }
}

template <int FMT, int G, int MT>
hipError_t launch_mt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                     const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                     hipStream_t stream) {
    const size_t ngroups = (size_t)(K / G);
    const size_t lds = partials ? 0 : (ngroups * 16 * MT * 4 * (FMT == 1 ? 2 : 1) + (size_t)SW * MT * 256 * 4);
    auto k = partials ? gemm_small_kernel<FMT, G, MT, true> : gemm_small_kernel<FMT, G, MT, false>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((N + SN - 1) / SN), dim3(SNT), lds, stream, M, K, N, wq,
                       static_cast<const uint16_t*>(wscale), static_cast<const uint16_t*>(wbias), xq, xs, xsum, y,
                       partials);
    return hipGetLastError();
}

template <int FMT, int G>
hipError_t launch_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    if (M <= 16) return launch_mt<FMT, G, 1>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return launch_mt<FMT, G, 2>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
}

}  // namespace

hipError_t launch_gemm_small(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                             const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                             int32_t* partials, hipStream_t stream) {
    if (M < 1 || M > GEMM_SMALL_MAX_M) return hipErrorInvalidValue;
    if (fmt == 0) return launch_fmt<0, 32>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_fmt<1, 64>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_fmt<1, 128>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
