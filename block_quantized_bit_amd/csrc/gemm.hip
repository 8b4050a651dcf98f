// W4A8 prefill GEMM on the gfx950 int8 matrix cores.
//
// tract PR #2432 ("The kernel"): the integer dot of every 32-weight block is
// exact and each block's integer is rescaled in float before accumulation.
// MLX PR #4802: with affine weights the int8 x int8 MMA runs on the original
// codes and the per-group scale and bias are applied inside the kernel.
//
// Tiling: a workgroup of 4 wavefronts computes a 128 x 128 tile of Y; each
// wavefront owns 64 x 64 (2 x 2 tiles of v_mfma_i32_32x32x32_i8). The K loop
// walks 128-wide stages. Per stage the int8 activation tile and the weight
// tile are staged through LDS; the weight nibbles are unpacked once, on the
// way into LDS (to q - 8 as signed bytes for Q4_0, to q for affine), so every
// MFMA reads ready int8 operands. One 32-wide K step is one Q4_0 block; an
// affine group of 64 / 128 accumulates 2 / 4 steps in int32. After each block
// or group the int32 tile is rescaled into float accumulators:
//   Q4_0:   acc += xs[m] * d[n] * P
//   affine: acc += xs[m] * (s[n] * A) + (xs * xsum)[m] * b[n]
// The next stage's global loads are issued into registers before the current
// stage is computed, so their latency overlaps the matrix work.
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int BM = 128, BN = 128, KS = 128;
constexpr int LDS_STRIDE = KS + 16;  // bytes per LDS row; the pad spreads rows over the banks

template <int FMT, int G, bool PARTIALS>
__global__ __launch_bounds__(256) void gemm_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ wscale,
                                                   const uint16_t* __restrict__ wbias, const int8_t* __restrict__ xq,
                                                   const float* __restrict__ xs, const int32_t* __restrict__ xsum,
                                                   float* __restrict__ y, int32_t* __restrict__ partials) {
    constexpr int GPS = KS / G;  // blocks or groups per stage
    constexpr int SPG = G / 32;  // 32-wide MFMA steps per block or group

    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float xs_s[GPS][BM];
    __shared__ __attribute__((aligned(16))) float xb_s[GPS][BM];
    __shared__ float ws_s[GPS][BN];
    __shared__ float wb_s[GPS][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int ngroups = K / G;
    const int nstages = (K + KS - 1) / KS;
    const size_t wrow = (size_t)(K >> 1);

    uint4 ra[4], rb[2];
    float rxs[2], rxb[2], rws[2], rwb[2];

    auto load_stage = [&](int st) {
        const int k0 = st * KS;
        const int ks = min(KS, K - k0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, r = idx >> 3, c16 = idx & 7;
            const int m = m0 + r;
            ra[i] = (m < M && c16 * 16 < ks) ? *reinterpret_cast<const uint4*>(xq + (size_t)m * K + k0 + c16 * 16)
                                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, c = idx >> 2, b = idx & 3;
            const int n = n0 + c;
            const uint32_t pad = (FMT == 0) ? 0x88888888u : 0u;  // codes of a zero weight
            rb[i] = (n < N && b * 32 < ks)
                        ? *reinterpret_cast<const uint4*>(wq + (size_t)n * wrow + (size_t)((k0 >> 5) + b) * 16)
                        : make_uint4(pad, pad, pad, pad);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            rxs[i] = rxb[i] = rws[i] = rwb[i] = 0.0f;
            if (idx < GPS * 128) {
                const int gi = idx >> 7, r = idx & 127;
                const int g = k0 / G + gi;
                if (gi * G < ks) {
                    const int m = m0 + r, n = n0 + r;
                    if (!PARTIALS && m < M) {
                        rxs[i] = xs[(size_t)m * ngroups + g];
                        if (FMT == 1) rxb[i] = rxs[i] * (float)xsum[(size_t)m * ngroups + g];
                    }
                    if (!PARTIALS && n < N) {
                        if (FMT == 0) {
                            rws[i] = half_to_float(wscale[(size_t)n * ngroups + g]);
                        } else {
                            rws[i] = bf16_to_float(wscale[(size_t)n * ngroups + g]);
                            rwb[i] = bf16_to_float(wbias[(size_t)n * ngroups + g]);
                        }
                    }
                }
            }
        }
    };

    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, r = idx >> 3, c16 = idx & 7;
            *reinterpret_cast<uint4*>(&As[r * LDS_STRIDE + c16 * 16]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, c = idx >> 2, b = idx & 3;
            uint4 lo = make_uint4(lo_nibbles(rb[i].x), lo_nibbles(rb[i].y), lo_nibbles(rb[i].z), lo_nibbles(rb[i].w));
            uint4 hi = make_uint4(hi_nibbles(rb[i].x), hi_nibbles(rb[i].y), hi_nibbles(rb[i].z), hi_nibbles(rb[i].w));
            if (FMT == 0) {
                lo = make_uint4(minus8_bytes(lo.x), minus8_bytes(lo.y), minus8_bytes(lo.z), minus8_bytes(lo.w));
                hi = make_uint4(minus8_bytes(hi.x), minus8_bytes(hi.y), minus8_bytes(hi.z), minus8_bytes(hi.w));
            }
            *reinterpret_cast<uint4*>(&Bs[c * LDS_STRIDE + b * 32]) = lo;
            *reinterpret_cast<uint4*>(&Bs[c * LDS_STRIDE + b * 32 + 16]) = hi;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i;
            if (idx < GPS * 128) {
                const int gi = idx >> 7, r = idx & 127;
                xs_s[gi][r] = rxs[i];
                xb_s[gi][r] = rxb[i];
                ws_s[gi][r] = rws[i];
                wb_s[gi][r] = rwb[i];
            }
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int half = lane >> 5, l32 = lane & 31;
    const int arow0 = wm * 64 + l32, brow0 = wn * 64 + l32;

    load_stage(0);
    for (int st = 0; st < nstages; ++st) {
        __syncthreads();
        store_stage();
        __syncthreads();
        if (st + 1 < nstages) load_stage(st + 1);

        const int k0 = st * KS;
        const int ks = min(KS, K - k0);
#pragma unroll
        for (int gi = 0; gi < GPS; ++gi) {
            if (gi * G >= ks) break;
            v16i pi[2][2];
#pragma unroll
            for (int s = 0; s < SPG; ++s) {
                const int kk = gi * G + s * 32 + 16 * half;
                v4i a0 = *reinterpret_cast<const v4i*>(&As[arow0 * LDS_STRIDE + kk]);
                v4i a1 = *reinterpret_cast<const v4i*>(&As[(arow0 + 32) * LDS_STRIDE + kk]);
                v4i b0 = *reinterpret_cast<const v4i*>(&Bs[brow0 * LDS_STRIDE + kk]);
                v4i b1 = *reinterpret_cast<const v4i*>(&Bs[(brow0 + 32) * LDS_STRIDE + kk]);
                if (s == 0) {
                    const v16i z = {};
                    pi[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, z, 0, 0, 0);
                    pi[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b1, z, 0, 0, 0);
                    pi[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, z, 0, 0, 0);
                    pi[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, z, 0, 0, 0);
                } else {
                    pi[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, pi[0][0], 0, 0, 0);
                    pi[0][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b1, pi[0][1], 0, 0, 0);
                    pi[1][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, pi[1][0], 0, 0, 0);
                    pi[1][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, pi[1][1], 0, 0, 0);
                }
            }
            // D layout of the 32x32 MFMA: lane holds column l32, rows
            // 8*(r/4) + 4*half + r%4 for r = 0..15.
            if (PARTIALS) {
                const int g = k0 / G + gi;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int n = n0 + wn * 64 + nt * 32 + l32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                            if (m < M && n < N) partials[((size_t)m * N + n) * ngroups + g] = pi[mt][nt][r];
                        }
                    }
            } else {
                float wsv[2], wbv[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    wsv[nt] = ws_s[gi][wn * 64 + nt * 32 + l32];
                    wbv[nt] = wb_s[gi][wn * 64 + nt * 32 + l32];
                }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    float xsv[16], xbv[16];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r0 = wm * 64 + mt * 32 + 8 * j + 4 * half;
                        const float4 v = *reinterpret_cast<const float4*>(&xs_s[gi][r0]);
                        xsv[4 * j] = v.x; xsv[4 * j + 1] = v.y; xsv[4 * j + 2] = v.z; xsv[4 * j + 3] = v.w;
                        if (FMT == 1) {
                            const float4 u = *reinterpret_cast<const float4*>(&xb_s[gi][r0]);
                            xbv[4 * j] = u.x; xbv[4 * j + 1] = u.y; xbv[4 * j + 2] = u.z; xbv[4 * j + 3] = u.w;
                        }
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float p = (float)pi[mt][nt][r];
                            if (FMT == 0)
                                acc[mt][nt][r] += (xsv[r] * wsv[nt]) * p;
                            else
                                acc[mt][nt][r] += xsv[r] * (wsv[nt] * p) + xbv[r] * wbv[nt];
                        }
                }
            }
        }
    }

    if (!PARTIALS) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int n = n0 + wn * 64 + nt * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (m < M && n < N) y[(size_t)m * N + n] = acc[mt][nt][r];
                }
            }
    }
}

template <int FMT, int G>
hipError_t launch_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(256);
    const uint16_t* ws = static_cast<const uint16_t*>(wscale);
    const uint16_t* wb = static_cast<const uint16_t*>(wbias);
    if (partials)
        hipLaunchKernelGGL((gemm_kernel<FMT, G, true>), grid, block, 0, stream, M, K, N, wq, ws, wb, xq, xs, xsum,
                           y, partials);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, G, false>), grid, block, 0, stream, M, K, N, wq, ws, wb, xq, xs, xsum,
                           y, partials);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                       const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                       int32_t* partials, hipStream_t stream) {
    if (fmt == 0) return launch_fmt<0, 32>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_fmt<1, 64>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_fmt<1, 128>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
