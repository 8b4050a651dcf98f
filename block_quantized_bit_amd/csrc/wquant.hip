// Weight quantization on the GPU (model preparation): Q4_0, affine 4-bit and
// Q4_K. One thread per block, group or super-block; every rounding decision
// is taken in float32 with correctly rounded division and round-half-even.
//
// tract PR #2432: Q4_0 codes with one scale per 32-weight block, value
// d * (q - 8), d from the block's signed extreme. MLX PR #4802: affine groups
// with a scale and bias per group. C-Kernel-Engine gemm_kernels_q4k.c: Q4_K
// super-blocks of 256 weights, 6-bit sub-block scales and mins, value
// d * sc * q - dmin * m.
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

template <bool BF16>
__device__ __forceinline__ float load_w(const void* w, size_t i) {
    if (BF16) return bf16_to_float(static_cast<const uint16_t*>(w)[i]);
    return static_cast<const float*>(w)[i];
}

// Code k of a row goes to byte 16*(k/32) + (k%32)%16, low nibble if k%32 < 16.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_q4_0_kernel(long long nblocks, int K, const void* __restrict__ w,
                                                            uint8_t* __restrict__ wq, uint16_t* __restrict__ wd) {
    const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const size_t base = (size_t)b * 32;  // blocks are contiguous in [N][K] since K % 32 == 0
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = load_w<BF16>(w, base + j);
    int imax = 0;
    float amax = fabsf(v[0]);
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        const float a = fabsf(v[j]);
        if (a > amax) { amax = a; imax = j; }
    }
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) mx = (j == imax) ? v[j] : mx;
    const uint16_t d16 = float_to_half_bits(mx / -8.0f);
    const float d = half_to_float(d16);
    uint32_t out[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int jl = 4 * t + bb;
            int ql = 8, qh = 8;
            if (d != 0.0f) {
                ql = min(15, max(0, (int)rintf(v[jl] / d) + 8));
                qh = min(15, max(0, (int)rintf(v[jl + 16] / d) + 8));
            }
            word |= (uint32_t)(ql | (qh << 4)) << (8 * bb);
        }
        out[t] = word;
    }
    *reinterpret_cast<uint4*>(wq + (size_t)b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    wd[b] = d16;
}

// Affine codes 0 .. 2^BITS - 1 (MLX PR #4802 serves 4, 6 and 8 bits). Layouts:
// BITS 4: the nibble planes above; BITS 8: one byte per code; BITS 6: the low
// 4 bits in the 4-bit layout, then at plane_off the high 2 bits, 8 bytes per
// 32-code block: word h holds code 16h + c of the block in byte c % 4, bits
// 2 * (c / 4) and 2 * (c / 4) + 1.
template <int G, bool BF16, int BITS>
__global__ __launch_bounds__(256) void quantize_affine_kernel(long long ngroups_total, int K,
                                                              const void* __restrict__ w, uint8_t* __restrict__ wq,
                                                              uint16_t* __restrict__ ws, uint16_t* __restrict__ wb,
                                                              size_t plane_off) {
    constexpr int QMAX = (1 << BITS) - 1;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= ngroups_total) return;
    const size_t base = (size_t)g * G;
    float mn = load_w<BF16>(w, base), mx = mn;
    for (int j = 1; j < G; ++j) {
        const float v = load_w<BF16>(w, base + j);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
    const float range = mx - mn;
    const uint16_t s16 = float_to_bf16_bits(range / (float)QMAX);
    const uint16_t b16 = float_to_bf16_bits(mn);
    const float s = bf16_to_float(s16), bias = bf16_to_float(b16);
    auto code = [&](int j) {
        if (s == 0.0f) return 0;
        const float t = load_w<BF16>(w, base + j) - bias;
        return min(QMAX, max(0, (int)rintf(t / s)));
    };
    for (int blk = 0; blk < G / 32; ++blk) {
        if (BITS == 8) {
            uint32_t out[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                uint32_t word = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) word |= (uint32_t)code(32 * blk + 4 * t + bb) << (8 * bb);
                out[t] = word;
            }
            uint4* dst = reinterpret_cast<uint4*>(wq + base + 32 * blk);
            dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
            dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
            continue;
        }
        uint32_t out[4], hp[2] = {0u, 0u};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t word = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int ql = code(32 * blk + 4 * t + bb), qh = code(32 * blk + 16 + 4 * t + bb);
                word |= (uint32_t)((ql & 15) | ((qh & 15) << 4)) << (8 * bb);
                if (BITS == 6) {  // codes 4t + bb and 16 + 4t + bb: byte bb, bits 2t of words 0 and 1
                    hp[0] |= (uint32_t)(ql >> 4) << (8 * bb + 2 * t);
                    hp[1] |= (uint32_t)(qh >> 4) << (8 * bb + 2 * t);
                }
            }
            out[t] = word;
        }
        *reinterpret_cast<uint4*>(wq + base / 2 + 16 * blk) = make_uint4(out[0], out[1], out[2], out[3]);
        if (BITS == 6) *reinterpret_cast<uint2*>(wq + plane_off + base / 4 + 8 * blk) = make_uint2(hp[0], hp[1]);
    }
    ws[g] = s16;
    wb[g] = b16;
}

__global__ __launch_bounds__(256) void quantize_q4k_kernel(long long nsb_total, const float* __restrict__ w,
                                                           uint8_t* __restrict__ blocks) {
    const long long sbi = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (sbi >= nsb_total) return;
    const float* x = w + (size_t)sbi * 256;
    float a[8], c[8], amax = 0.0f, cmax = 0.0f;
    for (int s = 0; s < 8; ++s) {
        float lo = 0.0f, hi = x[32 * s];
        for (int j = 0; j < 32; ++j) {
            const float v = x[32 * s + j];
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
        a[s] = (hi - lo) / 15.0f;
        c[s] = -lo;
        amax = fmaxf(amax, a[s]);
        cmax = fmaxf(cmax, c[s]);
    }
    const uint16_t d16 = float_to_half_bits(amax / 63.0f);
    const uint16_t dm16 = float_to_half_bits(cmax / 63.0f);
    const float d = half_to_float(d16), dmin = half_to_float(dm16);
    uint32_t sc[8], mn[8];
    for (int s = 0; s < 8; ++s) {
        sc[s] = (d != 0.0f) ? (uint32_t)min(63, max(0, (int)rintf(a[s] / d))) : 0u;
        mn[s] = (dmin != 0.0f) ? (uint32_t)min(63, max(0, (int)rintf(c[s] / dmin))) : 0u;
    }
    // sixteen 6-bit fields, little-endian: sc[0..7] at bits 0..47, m[0..7] at 48..95
    uint64_t f_lo = 0, f_hi = 0;  // bits 0..47 and 48..95
    for (int s = 0; s < 8; ++s) {
        f_lo |= (uint64_t)sc[s] << (6 * s);
        f_hi |= (uint64_t)mn[s] << (6 * s);
    }
    const uint32_t w0 = (uint32_t)d16 | ((uint32_t)dm16 << 16);
    const uint32_t w1 = (uint32_t)f_lo;
    const uint32_t w2 = (uint32_t)(f_lo >> 32) | (uint32_t)(f_hi << 16);
    const uint32_t w3 = (uint32_t)(f_hi >> 16);
    uint8_t* blk = blocks + (size_t)sbi * 144;
    *reinterpret_cast<uint4*>(blk) = make_uint4(w0, w1, w2, w3);
    for (int cc = 0; cc < 4; ++cc) {  // qs[32cc + l]: low nibble weight 64cc + l, high nibble 64cc + 32 + l
        const float ds_lo = d * (float)sc[2 * cc], dm_lo = dmin * (float)mn[2 * cc];
        const float ds_hi = d * (float)sc[2 * cc + 1], dm_hi = dmin * (float)mn[2 * cc + 1];
        for (int t = 0; t < 8; ++t) {
            uint32_t word = 0;
            for (int bb = 0; bb < 4; ++bb) {
                const int l = 4 * t + bb;
                int ql = 0, qh = 0;
                if (ds_lo != 0.0f) ql = min(15, max(0, (int)rintf((x[64 * cc + l] + dm_lo) / ds_lo)));
                if (ds_hi != 0.0f) qh = min(15, max(0, (int)rintf((x[64 * cc + 32 + l] + dm_hi) / ds_hi)));
                word |= (uint32_t)(ql | (qh << 4)) << (8 * bb);
            }
            *reinterpret_cast<uint32_t*>(blk + 16 + 32 * cc + 4 * t) = word;
        }
    }
}

template <int G, int BITS>
hipError_t launch_affine(long long nb, int K, bool bf16, const void* w, uint8_t* wq, uint16_t* ws, uint16_t* wb,
                         size_t plane_off, hipStream_t stream) {
    const unsigned grid = (unsigned)((nb + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL((quantize_affine_kernel<G, true, BITS>), dim3(grid), dim3(256), 0, stream, nb, K, w, wq, ws,
                           wb, plane_off);
    else
        hipLaunchKernelGGL((quantize_affine_kernel<G, false, BITS>), dim3(grid), dim3(256), 0, stream, nb, K, w, wq,
                           ws, wb, plane_off);
    return hipGetLastError();
}

template <int G>
hipError_t launch_affine_bits(int bits, long long nb, int K, bool bf16, const void* w, uint8_t* wq, uint16_t* ws,
                              uint16_t* wb, size_t plane_off, hipStream_t stream) {
    if (bits == 4) return launch_affine<G, 4>(nb, K, bf16, w, wq, ws, wb, plane_off, stream);
    if (bits == 6) return launch_affine<G, 6>(nb, K, bf16, w, wq, ws, wb, plane_off, stream);
    if (bits == 8) return launch_affine<G, 8>(nb, K, bf16, w, wq, ws, wb, plane_off, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize_weights(int N, int K, int bs, int fmt, int bits, bool bf16, const void* w, uint8_t* wq,
                                   void* wscale, void* wbias, hipStream_t stream) {
    const long long nb = (long long)N * (K / bs);
    const unsigned grid = (unsigned)((nb + 255) / 256);
    uint16_t* ws = static_cast<uint16_t*>(wscale);
    uint16_t* wb = static_cast<uint16_t*>(wbias);
    const size_t plane_off = (size_t)N * (K / 2);  // 6-bit: the high 2-bit plane follows the nibble planes
    if (fmt == 0) {
        if (bits != 4) return hipErrorInvalidValue;
        if (bf16) hipLaunchKernelGGL((quantize_q4_0_kernel<true>), dim3(grid), dim3(256), 0, stream, nb, K, w, wq, ws);
        else hipLaunchKernelGGL((quantize_q4_0_kernel<false>), dim3(grid), dim3(256), 0, stream, nb, K, w, wq, ws);
        return hipGetLastError();
    }
    if (bs == 64) return launch_affine_bits<64>(bits, nb, K, bf16, w, wq, ws, wb, plane_off, stream);
    if (bs == 128) return launch_affine_bits<128>(bits, nb, K, bf16, w, wq, ws, wb, plane_off, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_q4k_quantize_weights(int N, int K, const float* w, void* blocks, hipStream_t stream) {
    const long long nsb = (long long)N * (K / 256);
    hipLaunchKernelGGL(quantize_q4k_kernel, dim3((unsigned)((nsb + 255) / 256)), dim3(256), 0, stream, nsb, w,
                       static_cast<uint8_t*>(blocks));
    return hipGetLastError();
}

}  // namespace q4
