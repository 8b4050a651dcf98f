// Q4_K fused-dequant GEMV and GEMM with float32 activations.
//
// C-Kernel-Engine gemm_kernels_q4k.c: weights are dequantized in registers
// and used at once by the multiply-add, never written to memory; the GEMV
// (one token) is memory-bound, the GEMM reuses each dequantized weight for
// every activation row. Weight value: d * sc[s] * q - dmin * m[s].
//
// Block: 144 bytes = 16-byte header {fp16 d, fp16 dmin, 12 bytes of 6-bit
// scales and mins} + qs[128]. A 16-byte qs chunk j (0..7) of a block holds,
// for chunk c = j / 2 of 64 weights and l0 = 16 * (j % 2), the 16 weights
// 64c + l0 + t in its low nibbles (sub-block 2c) and 64c + 32 + l0 + t in its
// high nibbles (sub-block 2c + 1).
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int QK = 256;
constexpr int BLOCK_BYTES = 144;

// 6-bit fields of the header: sc[s] at bit 6s and m[s] at bit 48 + 6s of the
// 96-bit little-endian string (hdr.y, hdr.z, hdr.w). Returns sc[2c], sc[2c+1],
// m[2c], m[2c+1] as floats.
__device__ __forceinline__ void q4k_pair_scales(const uint4& hdr, int c, float& sc0, float& sc1, float& m0,
                                                float& m1) {
    const uint64_t lo = (uint64_t)hdr.y | ((uint64_t)hdr.z << 32);   // bits 0..63
    const uint64_t hi = (uint64_t)hdr.z | ((uint64_t)hdr.w << 32);   // bits 32..95
    const uint32_t s = (uint32_t)(lo >> (12 * c)) & 0xFFFu;
    const uint32_t m = (uint32_t)(hi >> (16 + 12 * c)) & 0xFFFu;
    sc0 = (float)(s & 63u);
    sc1 = (float)(s >> 6);
    m0 = (float)(m & 63u);
    m1 = (float)(m >> 6);
}

__device__ __forceinline__ float byte_f(uint32_t v, int b) { return (float)((v >> (8 * b)) & 0xFFu); }

// Nibbles isolated into bytes, with the known-zero high bits of each byte
// hidden from the compiler: it then converts byte b with v_cvt_f32_ubyte<b>
// rather than a bit-field extract followed by a conversion.
__device__ __forceinline__ uint32_t nibbles_lo(uint32_t w) {
    uint32_t v = lo_nibbles(w);
    __asm__("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t nibbles_hi(uint32_t w) {
    uint32_t v = hi_nibbles(w);
    __asm__("" : "+v"(v));
    return v;
}

// Sum over 16 weights of code * x for the 4 dwords `q` (nibbles already
// isolated into bytes) against 16 activations.
__device__ __forceinline__ float dot16(const uint32_t q[4], const float* x) {
    float a = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) a = fmaf(byte_f(q[t], b), x[4 * t + b], a);
    return a;
}

constexpr int RSRC_WORD3 = 0x00020000;
constexpr uint32_t OUT = 0x80000000u;  // beyond every buffer range: reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

// One pass of the GEMV: header and qs chunk of each of the lane's UPL chunks,
// for R consecutive rows of the wavefront.
template <int UPL, int R>
struct Q4kPass {
    uint4 hdr[R][UPL], qs[R][UPL];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r_w, int row, int lane, int units, uint32_t rowbytes,
                                         int j) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const int u = lane + 64 * i;
                const uint32_t o = u < units ? (uint32_t)(row + r) * rowbytes + (uint32_t)(u >> 3) * BLOCK_BYTES : OUT;
                hdr[r][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o, 0, 0));
                qs[r][i] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o == OUT ? OUT : o + 16 + 16 * j, 0, 0));
            }
    }
};

// GEMV: each wavefront owns a contiguous range of rows and walks it R rows per
// pass, prefetching the next pass before the arithmetic of the current one.
// Lane l owns qs chunks u = l + 64 i of every row; the activations of its
// chunks (and their sums per half) stay in registers. The workgroup reads x
// from memory once: after the first pass of weight loads is issued, its
// threads copy x into LDS in lane order -- float4 (i, h, t) of lane l at
// ((2i + h) * 4 + t) * 64 + l, h = 0 for the low-nibble weights, 1 for the
// high -- so that each wavefront's register fill is 16-byte reads by
// consecutive lanes (no bank conflicts), and the vector memory path carries
// x once per workgroup instead of once per wavefront. The per-half sums are
// formed in the same copy: each copying thread adds its float4, and each lane
// adds the four partial sums of its half.
// Every load is a buffer load with no branch around it: the wavefront's buffer
// range covers only its own rows, and offsets past the end read zero (a zero
// header makes a row's terms zero). UPL = chunks per lane (K / 2048, rounded up).
template <int UPL, int R>
__global__ __launch_bounds__(256) void q4k_gemv_kernel(int K, int N, int rows_per_wave,
                                                       const uint8_t* __restrict__ blocks,
                                                       const float* __restrict__ x, float* __restrict__ y) {
    __shared__ float4 xlds[UPL * 8 * 64];
    __shared__ float4 slds[UPL * 2 * 64];  // (i, h, l): the sums of the half's four float4, one per t
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = gw * rows_per_wave;
    const int nrows = max(0, min(rows_per_wave, N - row0));
    const int units = K >> 5;
    const uint32_t rowbytes = (uint32_t)(K >> 8) * BLOCK_BYTES;
    const int j = lane & 7;  // qs chunk within a block (u % 8 == lane % 8)
    const int c = j >> 1, l0 = 16 * (j & 1);
    const __amdgpu_buffer_rsrc_t r_w = rsrc(blocks + (size_t)row0 * rowbytes, (uint32_t)nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t r_x = rsrc(x, (uint32_t)K * 4u);

    // x loads first (in lane order, units past K read zero), then the first
    // pass of weights; the LDS stores wait only for the x loads
    float4 xv[UPL * 2];
#pragma unroll
    for (int m = 0; m < UPL * 2; ++m) {
        const int e = (int)threadIdx.x + 256 * m;  // entry ((2i + h) * 4 + t) * 64 + l
        const int l = e & 63, t = (e >> 6) & 3, h = (e >> 8) & 1, i = e >> 9;
        const int u = l + 64 * i, jl = l & 7;
        const uint32_t k = (uint32_t)((u >> 3) * QK + 64 * (jl >> 1) + 16 * (jl & 1) + 32 * h + 4 * t);
        xv[m] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r_x, u < units ? 4 * k : OUT, 0, 0));
    }
    Q4kPass<UPL, R> cur;
    cur.load(r_w, 0, lane, units, rowbytes, j);
#pragma unroll
    for (int m = 0; m < UPL * 2; ++m) {
        const int e = (int)threadIdx.x + 256 * m;  // ((2i + h) * 4 + t) * 64 + l
        xlds[e] = xv[m];
        reinterpret_cast<float*>(slds)[((e >> 8) * 64 + (e & 63)) * 4 + ((e >> 6) & 3)] =
            (xv[m].x + xv[m].y) + (xv[m].z + xv[m].w);
    }
    __syncthreads();
    if (nrows == 0) return;

    float xl[UPL][16], xh[UPL][16], sl[UPL], sh[UPL];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 a = xlds[((2 * i) * 4 + t) * 64 + lane];
            const float4 b = xlds[((2 * i + 1) * 4 + t) * 64 + lane];
            xl[i][4 * t] = a.x; xl[i][4 * t + 1] = a.y; xl[i][4 * t + 2] = a.z; xl[i][4 * t + 3] = a.w;
            xh[i][4 * t] = b.x; xh[i][4 * t + 1] = b.y; xh[i][4 * t + 2] = b.z; xh[i][4 * t + 3] = b.w;
        }
        const float4 pl = slds[(2 * i) * 64 + lane], ph = slds[(2 * i + 1) * 64 + lane];
        sl[i] = (pl.x + pl.y) + (pl.z + pl.w);
        sh[i] = (ph.x + ph.y) + (ph.z + ph.w);
    }

    for (int p = 0; p < nrows; p += R) {
        Q4kPass<UPL, R> nxt;
        if (p + R < nrows) nxt.load(r_w, p + R, lane, units, rowbytes, j);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < UPL; ++i) {
                const uint4 h = cur.hdr[r][i], q = cur.qs[r][i];
                const float d = half_to_float(h.x & 0xFFFFu);
                const float dmin = half_to_float(h.x >> 16);
                float sc0, sc1, mm0, mm1;
                q4k_pair_scales(h, c, sc0, sc1, mm0, mm1);
                const uint32_t ql[4] = {nibbles_lo(q.x), nibbles_lo(q.y), nibbles_lo(q.z), nibbles_lo(q.w)};
                const uint32_t qh[4] = {nibbles_hi(q.x), nibbles_hi(q.y), nibbles_hi(q.z), nibbles_hi(q.w)};
                const float al = dot16(ql, xl[i]);
                const float ah = dot16(qh, xh[i]);
                acc += (d * sc0) * al - (dmin * mm0) * sl[i];
                acc += (d * sc1) * ah - (dmin * mm1) * sh[i];
            }
            acc = wave_sum(acc);
            if (lane == 0 && p + r < nrows) y[row0 + p + r] = acc;
        }
        cur = nxt;
    }
}

// GEMV for long rows: the activations are read per row instead of being held
// in registers.
__global__ __launch_bounds__(256) void q4k_gemv_long_kernel(int K, int N, const uint8_t* __restrict__ blocks,
                                                            const float* __restrict__ x, float* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const int units = K >> 5, nsb = K >> 8;
    const int j = lane & 7, c = j >> 1, l0 = 16 * (j & 1);
    float acc = 0.0f;
    for (int u = lane; u < units; u += 64) {
        const uint8_t* blk = blocks + ((size_t)n * nsb + (u >> 3)) * BLOCK_BYTES;
        const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
        const uint4 q = *reinterpret_cast<const uint4*>(blk + 16 + 16 * j);
        const int k = (u >> 3) * QK + 64 * c + l0;
        float xl[16], xh[16], sl = 0.0f, sh = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            xl[t] = x[k + t];
            xh[t] = x[k + 32 + t];
            sl += xl[t];
            sh += xh[t];
        }
        const float d = half_to_float(hdr.x & 0xFFFFu), dmin = half_to_float(hdr.x >> 16);
        float sc0, sc1, mm0, mm1;
        q4k_pair_scales(hdr, c, sc0, sc1, mm0, mm1);
        const uint32_t ql[4] = {nibbles_lo(q.x), nibbles_lo(q.y), nibbles_lo(q.z), nibbles_lo(q.w)};
        const uint32_t qh[4] = {nibbles_hi(q.x), nibbles_hi(q.y), nibbles_hi(q.z), nibbles_hi(q.w)};
        acc += (d * sc0) * dot16(ql, xl) - (dmin * mm0) * sl;
        acc += (d * sc1) * dot16(qh, xh) - (dmin * mm1) * sh;
    }
    acc = wave_sum(acc);
    if (lane == 0) y[n] = acc;
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Largest value over the 64 lanes of a wavefront; every lane receives it.
// The values are magnitudes (no sign bit), so their bit patterns order as
// unsigned integers and the maximum runs on v_max_u32 with DPP operands.
__device__ __forceinline__ float wave_max(float f) {
    uint32_t v = __builtin_bit_cast(uint32_t, f);
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return __builtin_bit_cast(float, max(max(r0, r1), max(r2, r3)));
}

// Sum over aligned groups of 8 lanes; every lane of a group receives it.
__device__ __forceinline__ float sum8(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    return v;
}

// Scale of a row's activations over a super-block, from the float4 each lane
// holds (a wavefront holds the row): the largest magnitude mx = f * 2^E,
// f in [0.5, 1) (E = -126 below the normal range), is brought into
// [2^14, 2^15) by 2^(15 - E), at most 2^126 so that the scale and its inverse
// stay normal floats. sc = 2^(15 - E), inv = 2^(E - 15).
__device__ __forceinline__ void split_scale(const float4& v, float& sc, float& inv) {
    const float mx = wave_max(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const int E = max((int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 126, -111);
    sc = __builtin_bit_cast(float, (uint32_t)(127 + 15 - E) << 23);
    inv = __builtin_bit_cast(float, (uint32_t)(127 - 15 + E) << 23);
}

// Bytes 0 and 1 (SEL01) or 2 and 3 (SEL23) of a word of isolated nibbles as
// an exact f16 pair: v_perm places each code byte under the byte 0x64, giving
// the half 0x6400 | q = 1024 + q, and subtracting 1024 leaves q.
constexpr uint32_t SEL01 = 0x04010400u, SEL23 = 0x04030402u;
__device__ __forceinline__ uint32_t code_pair_f16(uint32_t nib, uint32_t sel) {
    v2h h = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, nib, sel));
    h = h - v2h{(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, h);
}

// The 16 codes of 8 qs bytes as two f16 MFMA operands: low nibbles (byte i is
// weight k = i of the lane's 8 in one sub-block) and high nibbles (the same k
// in the next sub-block). 22 instructions for 16 codes.
__device__ __forceinline__ void codes_f16(uint2 cw, v8h& blo, v8h& bhi) {
    const uint32_t lx = cw.x & 0x0F0F0F0Fu, ly = cw.y & 0x0F0F0F0Fu;
    const uint32_t hx = (cw.x >> 4) & 0x0F0F0F0Fu, hy = (cw.y >> 4) & 0x0F0F0F0Fu;
    blo = __builtin_bit_cast(v8h, make_uint4(code_pair_f16(lx, SEL01), code_pair_f16(lx, SEL23),
                                             code_pair_f16(ly, SEL01), code_pair_f16(ly, SEL23)));
    bhi = __builtin_bit_cast(v8h, make_uint4(code_pair_f16(hx, SEL01), code_pair_f16(hx, SEL23),
                                             code_pair_f16(hy, SEL01), code_pair_f16(hy, SEL23)));
}

// GEMM on the f16 matrix cores (v_mfma_f32_16x16x32_f16), float32-accurate.
// Per sub-block the product is factored as in the GEMV,
//   sum_k (d sc q - dmin m) x = (d sc) sum_k q x - (dmin m) sum_k x,
// and sum_k q x is taken on the matrix cores: a code is an exact f16, and each
// activation enters as two f16 halves, hi = f16(x') and lo = f16(x' - hi), of
// x' = x * 2^e, the row's values over the super-block scaled by a power of two
// that puts their largest magnitude in [2^14, 2^15) (inside the f16 range, and
// lo stays a normal number for all but the row's tiny values; the scale is at
// most 2^126, so only rows whose largest magnitude in a super-block is below
// 2^-112 lose relative precision). hi + lo carries
// 22 of x's 24 significant bits, every code x half product is exact in f32, so
// the sum differs from the float32 one by rounding only; the result is scaled
// back by 2^-e (exact).
//
// A workgroup of W x KP wavefronts covers 16 activation rows x 16 W weight
// rows; wavefront (w, p) owns weight rows 16 w .. 16 w + 15 and the p-th of KP
// contiguous ranges of super-blocks, and the KP partial sums are added in LDS
// in a fixed order at the end. For every super-block the workgroup stages the
// 16 x 256 activation tile of each range in LDS as the hi and lo halves plus
// per-row sub-block sums and the row's 2^-e. Lane l of a wavefront holds
// weight row l % 16; its operands for k = 8 (l / 16) .. +7 of a sub-block are 8
// bytes of qs (low nibbles: sub-block 2c, high nibbles: 2c + 1, chunk c), so
// one sub-block is two MFMAs (hi, lo). The loads of the next D super-blocks
// are in registers while the current one is computed (each slot's registers
// are refilled in place, after their last use, so no register copy waits for
// a load in flight), and the staged tiles are double-buffered, so a
// super-block costs one barrier. All loads are buffer
// loads with no branch around them: rows past M or N and super-blocks past a
// range read zero.
constexpr int XR = QK + 16;  // halves per staged row: 544 bytes, no LDS bank conflicts on the A-operand reads (measured; 528 bytes gave 31%)

template <int W, int KP>
struct Q4kStage {
    v8h hi[2][16 * XR / 8];  // [buffer][row * XR / 8 + k / 8]
    v8h lo[2][16 * XR / 8];
    float sum[2][8][16];     // [buffer][sub-block][row]: sum of the scaled activations
    float inv[2][16];        // [buffer][row]: 2^-e
};

// The activation tile of one 16-row group and super-block, split as the
// kernel stages it, in 16-byte units: hi [16][256] f16 (units 0..511, row r
// at 32 r), lo likewise (512..1023), the per-row sub-block sums [8][16] f32
// (1024..1055) and the rows' 2^-e (1056..1059).
constexpr int TILE_UNITS = 1060;

// Splits x once per call into tiles (mt, sb) at ((mt * nsb + sb) * TILE_UNITS)
// 16-byte units of `work`, with the same arithmetic as the in-kernel staging
// of q4k_gemm_kernel. Grid (nsb, row tiles, 4): a workgroup of 4 wavefronts
// takes 4 rows of a tile's super-block, one row per wavefront and one float4
// per lane, so every row's scale is a wavefront reduction.
__global__ __launch_bounds__(256) void q4k_split_kernel(int M, int K, const float* __restrict__ x,
                                                        uint8_t* __restrict__ work) {
    const int lane = threadIdx.x & 63, c4 = lane;
    const int sb = blockIdx.x, mt = blockIdx.y, nsb = K >> 8;
    const int r = 4 * (int)blockIdx.z + (int)(threadIdx.x >> 6);
    const int m = mt * 16 + r;
    const __amdgpu_buffer_rsrc_t r_x = rsrc(x, (uint32_t)((size_t)M * K * 4));
    uint8_t* tile = work + ((size_t)mt * nsb + sb) * TILE_UNITS * 16;
    _Float16* hi = reinterpret_cast<_Float16*>(tile);
    _Float16* lo = hi + 16 * QK;
    float* sum = reinterpret_cast<float*>(tile + 1024 * 16);
    float* inv = sum + 8 * 16;
    const uint32_t o = (m < M) ? (uint32_t)(((size_t)m * K + (size_t)sb * QK + 4 * c4) * 4) : OUT;
    const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r_x, o, 0, 0));
    float sc, ivs;
    split_scale(v, sc, ivs);
    const float xs0 = v.x * sc, xs1 = v.y * sc, xs2 = v.z * sc, xs3 = v.w * sc;
    const _Float16 h0 = (_Float16)xs0, h1 = (_Float16)xs1, h2 = (_Float16)xs2, h3 = (_Float16)xs3;
    typedef _Float16 v4h __attribute__((ext_vector_type(4)));
    *reinterpret_cast<v4h*>(hi + r * QK + 4 * c4) = v4h{h0, h1, h2, h3};
    *reinterpret_cast<v4h*>(lo + r * QK + 4 * c4) =
        v4h{(_Float16)(xs0 - (float)h0), (_Float16)(xs1 - (float)h1), (_Float16)(xs2 - (float)h2),
            (_Float16)(xs3 - (float)h3)};
    const float ssum = sum8((xs0 + xs1) + (xs2 + xs3));
    if ((c4 & 7) == 0) sum[(c4 >> 3) * 16 + r] = ssum;
    if (c4 == 0) inv[r] = ivs;
}

template <int W, int KP, bool PRESPLIT, int D>
__global__ __launch_bounds__(64 * W * KP) void q4k_gemm_kernel(int M, int K, int N, const uint8_t* __restrict__ blocks,
                                                               const float* __restrict__ x, float* __restrict__ y,
                                                               const uint8_t* __restrict__ work) {
    constexpr int NTH = 64 * W;             // threads of one K range
    constexpr int XCH = 16 * QK / 4 / NTH;  // float4 of the activation tile per thread (16 / W)
    static_assert(XCH * NTH == 16 * QK / 4, "staging covers the tile");
    constexpr int UPT = 1024 / NTH;         // PRESPLIT: hi / lo units of the split tile per thread
    static_assert(UPT * NTH == 1024 && NTH >= 36, "the split tile is copied as UPT + 1 units per thread");
    static_assert(D >= 2, "the loads of the next super-block's tile are staged one iteration ahead");
    __shared__ Q4kStage<W, KP> st[KP];
    // the wavefront index is uniform: the K range, and with it every load's scalar offset, stays in SGPRs
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = wave / W, tp = tid - p * NTH;  // K range, thread within the range's group
    const int m0 = blockIdx.y * 16;
    const int n = blockIdx.x * (16 * W) + (wave % W) * 16 + (lane & 15);
    const int q = lane >> 4;
    const int nsb = K >> 8;
    const int per = (nsb + KP - 1) / KP;  // super-blocks per range
    const int sb0 = p * per, sb1 = min(nsb, sb0 + per);
    const __amdgpu_buffer_rsrc_t r_x = rsrc(x, (uint32_t)((size_t)M * K * 4));
    const __amdgpu_buffer_rsrc_t r_w = rsrc(blocks, (uint32_t)((size_t)N * nsb * BLOCK_BYTES));
    // per-lane offsets fixed for the kernel; each super-block adds a scalar offset
    uint32_t ox[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int idx = tp + NTH * i, r = idx >> 6, c4 = idx & 63;  // 1024 float4 = 16 rows x 64
        ox[i] = (m0 + r < M) ? (uint32_t)(((size_t)(m0 + r) * K + 4 * c4) * 4) : OUT;
    }
    const uint32_t ow = (n < N) ? (uint32_t)((size_t)n * nsb * BLOCK_BYTES) : OUT;
    const __amdgpu_buffer_rsrc_t r_t =
        rsrc(work, PRESPLIT ? (uint32_t)((size_t)((M + 15) / 16) * nsb * TILE_UNITS * 16) : 0u);
    const uint32_t otile = (uint32_t)((size_t)blockIdx.y * nsb * TILE_UNITS * 16);

    // The loads of one super-block: the activation tile (PRESPLIT: the split
    // tile's 16-byte units tp + NTH i, and unit 1024 + tp for tp < 36) and the
    // lane's weight header and code bytes. D of them are in flight: the
    // super-block sb's are issued D iterations before its arithmetic.
    struct Slot {
        float4 rx[PRESPLIT ? 1 : XCH];
        uint4 ru[PRESPLIT ? UPT : 1], ru5;
        uint4 rh;
        uint2 rq[4];
    };
    Slot sl[D];
    auto load_x = [&](Slot& L, int sb) {  // super-blocks past the range read zero
        const bool in = sb < sb1;
        if (PRESPLIT) {
            const uint32_t so = in ? otile + (uint32_t)sb * TILE_UNITS * 16 : 0u;
#pragma unroll
            for (int i = 0; i < UPT; ++i)
                L.ru[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        r_t, in ? (uint32_t)(tp + NTH * i) * 16 : OUT, so, 0));
            L.ru5 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  r_t, (in && tp < 36) ? (uint32_t)(1024 + tp) * 16 : OUT, so, 0));
        } else {
#pragma unroll
            for (int i = 0; i < XCH; ++i)
                L.rx[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r_x, in ? ox[i] : OUT,
                                                                                           in ? sb * QK * 4 : 0, 0));
        }
    };
    auto load_w = [&](Slot& L, int sb) {
        const bool in = sb < sb1;
        const uint32_t o = in ? ow : OUT, so = in ? (uint32_t)(sb * BLOCK_BYTES) : 0u;
        L.rh = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o, so, 0));
#pragma unroll
        for (int c = 0; c < 4; ++c)
            L.rq[c] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                    r_w, o == OUT ? OUT : o + 16 + 32 * c + 8 * q, so, 0));
    };
    // Stage the tile in buffer b: row r = wave-in-group + W i is held by the 64
    // lanes of one wavefront (lane = float4 index), so its largest magnitude
    // and its sub-block sums are wavefront and 8-lane reductions.
    auto stage = [&](int b, const Slot& L) {
        Q4kStage<W, KP>& S = st[p];
        if (PRESPLIT) {  // a copy of the split tile into the padded LDS rows
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                const int u = tp + NTH * i, half = u >> 9, r = (u >> 5) & 15, c8 = u & 31;
                v8h* dst = half ? S.lo[b] : S.hi[b];
                dst[r * (XR / 8) + c8] = __builtin_bit_cast(v8h, L.ru[i]);
            }
            if (tp < 32)
                *reinterpret_cast<uint4*>(&S.sum[b][0][0] + 4 * tp) = L.ru5;
            else if (tp < 36)
                *reinterpret_cast<uint4*>(&S.inv[b][4 * (tp - 32)]) = L.ru5;
            return;
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int idx = tp + NTH * i, r = idx >> 6, c4 = idx & 63;
            const float4 v = L.rx[i];
            float sc, ivs;
            split_scale(v, sc, ivs);
            const float xs0 = v.x * sc, xs1 = v.y * sc, xs2 = v.z * sc, xs3 = v.w * sc;
            const _Float16 h0 = (_Float16)xs0, h1 = (_Float16)xs1, h2 = (_Float16)xs2, h3 = (_Float16)xs3;
            const _Float16 l0 = (_Float16)(xs0 - (float)h0), l1 = (_Float16)(xs1 - (float)h1);
            const _Float16 l2 = (_Float16)(xs2 - (float)h2), l3 = (_Float16)(xs3 - (float)h3);
            typedef _Float16 v4h __attribute__((ext_vector_type(4)));
            *reinterpret_cast<v4h*>(reinterpret_cast<_Float16*>(S.hi[b]) + r * XR + 4 * c4) = v4h{h0, h1, h2, h3};
            *reinterpret_cast<v4h*>(reinterpret_cast<_Float16*>(S.lo[b]) + r * XR + 4 * c4) = v4h{l0, l1, l2, l3};
            const float ssum = sum8((xs0 + xs1) + (xs2 + xs3));
            if ((c4 & 7) == 0) S.sum[b][c4 >> 3][r] = ssum;
            if (c4 == 0) S.inv[b][r] = ivs;
        }
    };

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s2 = 0; s2 < D; ++s2) {
        load_x(sl[s2], sb0 + s2);
        load_w(sl[s2], sb0 + s2);
    }
    stage(0, sl[0]);
    const int row = lane & 15;  // activation row of this lane's A operands
    // The same trip count in every range (past its end: zeros). Iteration it
    // stages the tile of super-block it + 1 from its slot, refills the tile
    // part of its own slot (staged one iteration earlier) with super-block
    // it + D, computes super-block it from the weights in its slot and then
    // refills them too; the slot registers are used in place, so no register
    // copy waits for a load in flight.
    for (int it0 = 0; it0 < per; it0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int it = it0 + u;
            if (it >= per) break;
            const int sb = sb0 + it;
            __syncthreads();  // tile it is complete; every wavefront is done with the other buffer
            stage((it + 1) & 1, sl[(u + 1) % D]);
            load_x(sl[u], sb + D);
            const uint4 ch = sl[u].rh;
            const uint2* cc = sl[u].rq;
            const int b = it & 1;
            const Q4kStage<W, KP>& S = st[p];
            const float d = half_to_float(ch.x & 0xFFFFu), dmin = half_to_float(ch.x >> 16);
            v4f part = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float sc0, sc1, mm0, mm1;
                q4k_pair_scales(ch, c, sc0, sc1, mm0, mm1);
                v8h blo, bhi;
                codes_f16(cc[c], blo, bhi);
                const v8h* H = S.hi[b] + (row * XR + 64 * c + 8 * q) / 8;
                const v8h* L = S.lo[b] + (row * XR + 64 * c + 8 * q) / 8;
                const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
                v4f d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(H[0], blo, z, 0, 0, 0);
                d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(L[0], blo, d0, 0, 0, 0);
                v4f d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(H[4], bhi, z, 0, 0, 0);  // k + 32: sub-block 2c + 1
                d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(L[4], bhi, d1, 0, 0, 0);
                const v4f s0 = *reinterpret_cast<const v4f*>(&S.sum[b][2 * c][4 * q]);
                const v4f s1 = *reinterpret_cast<const v4f*>(&S.sum[b][2 * c + 1][4 * q]);
                const float a0 = d * sc0, a1 = d * sc1, e0 = dmin * mm0, e1 = dmin * mm1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    part[r] = fmaf(a0, d0[r], part[r]);
                    part[r] = fmaf(-e0, s0[r], part[r]);
                    part[r] = fmaf(a1, d1[r], part[r]);
                    part[r] = fmaf(-e1, s1[r], part[r]);
                }
            }
            const v4f iv = *reinterpret_cast<const v4f*>(&S.inv[b][4 * q]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(iv[r], part[r], acc[r]);
            load_w(sl[u], sb + D);
        }
    }
    // add the K ranges in order (p = 0, 1, ...) through LDS, reusing the staging memory
    if (KP > 1) {
        __syncthreads();
        float* pbuf = reinterpret_cast<float*>(&st[0]);  // [KP][W][64 lanes][4]
        if (p > 0) *reinterpret_cast<v4f*>(&pbuf[((p * W + wave % W) * 64 + lane) * 4]) = acc;
        __syncthreads();
        if (p == 0) {
#pragma unroll
            for (int k2 = 1; k2 < KP; ++k2)
                acc += *reinterpret_cast<const v4f*>(&pbuf[((k2 * W + wave % W) * 64 + lane) * 4]);
        }
    }
    // D layout: lane holds column lane%16, rows 4*(lane/16) + r
    if (p == 0 && n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * q + r;
            if (m < M) y[(size_t)m * N + n] = acc[r];
        }
    }
}

}  // namespace

hipError_t launch_q4k_gemv(int K, int N, const void* blocks, const float* x, float* y, hipStream_t stream) {
    const uint8_t* b = static_cast<const uint8_t*>(blocks);
    const int units = K >> 5;
    const int upl = (units + 63) / 64;
    // K <= 4096: two rows per pass, and as many workgroups as give every
    // wavefront a single pass (at 4096 x 14336: 1792 workgroups, 149
    // registers; 10.4-11.8 us against 11.4-11.9 us for one row per pass over
    // 1024 workgroups, timed side by side). Longer rows keep one row per
    // pass: two would not fit the registers beside the activations.
    if (upl <= 2) {
        constexpr int R = 2;
        const int grid = max(1, min(1792, (N + 4 * R - 1) / (4 * R)));
        const int rpw = (N + 4 * grid - 1) / (4 * grid);
        if (upl == 1)
            hipLaunchKernelGGL((q4k_gemv_kernel<1, R>), dim3(grid), dim3(256), 0, stream, K, N, rpw, b, x, y);
        else
            hipLaunchKernelGGL((q4k_gemv_kernel<2, R>), dim3(grid), dim3(256), 0, stream, K, N, rpw, b, x, y);
        return hipGetLastError();
    }
    constexpr int R = 1;
    const int want = 1024;
    const int grid = max(1, min(want, (N + 4 * R - 1) / (4 * R)));
    const int rpw = (N + 4 * grid - 1) / (4 * grid);
    switch (upl) {
        case 3: hipLaunchKernelGGL((q4k_gemv_kernel<3, R>), dim3(grid), dim3(256), 0, stream, K, N, rpw, b, x, y); break;
        case 4: hipLaunchKernelGGL((q4k_gemv_kernel<4, R>), dim3(grid), dim3(256), 0, stream, K, N, rpw, b, x, y); break;
        default:
            hipLaunchKernelGGL(q4k_gemv_long_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, K, N, b, x,
                               y);
    }
    return hipGetLastError();
}

// Super-blocks of loads in flight per wavefront. Measured at 16 x 4096 x 14336
// (cold weights): 2: 22.6 / 20.8 us (q4k_gemm / with the split), 3: 24.5 / 23.0,
// 4: 26.2 / 23.1; with the loop fully unrolled (exact load waits) 3 and 4 were
// still slower than 2.
constexpr int QD = 2;

hipError_t launch_q4k_gemm(int M, int K, int N, const void* blocks, const float* x, float* y, hipStream_t stream) {
    constexpr int W = 4;   // wavefronts (16 weight rows each) per K range
    constexpr int KP = 2;  // K ranges per workgroup (1: 34.3 us, 2: 29.5, 4: 30.0 at 16 x 4096 x 14336)
    const dim3 grid((unsigned)((N + 16 * W - 1) / (16 * W)), (unsigned)((M + 15) / 16));
    hipLaunchKernelGGL((q4k_gemm_kernel<W, KP, false, QD>), grid, dim3(64 * W * KP), 0, stream, M, K, N,
                       static_cast<const uint8_t*>(blocks), x, y, nullptr);
    return hipGetLastError();
}

size_t q4k_gemm_work_bytes(int M, int K) { return (size_t)((M + 15) / 16) * (K / QK) * TILE_UNITS * 16; }

template <int W, int KP>
hipError_t launch_presplit(int M, int K, int N, const void* blocks, const float* x, float* y, const uint8_t* wk,
                           hipStream_t stream) {
    const dim3 grid((unsigned)((N + 16 * W - 1) / (16 * W)), (unsigned)((M + 15) / 16));
    hipLaunchKernelGGL((q4k_gemm_kernel<W, KP, true, QD>), grid, dim3(64 * W * KP), 0, stream, M, K, N,
                       static_cast<const uint8_t*>(blocks), x, y, wk);
    return hipGetLastError();
}

hipError_t launch_q4k_gemm_work(int M, int K, int N, const void* blocks, const float* x, float* y, void* work,
                                hipStream_t stream) {
    uint8_t* wk = static_cast<uint8_t*>(work);
    hipLaunchKernelGGL(q4k_split_kernel, dim3((unsigned)(K / QK), (unsigned)((M + 15) / 16), 4), dim3(256), 0, stream,
                       M, K, x, wk);
    // the same launch shape as q4k_gemm (so the outputs are bit-identical); measured at 16 x 4096 x 14336:
    // 4 x 2 wavefronts 20.8 us with the split, 4 x 4 20.8, 2 x 4 26.6, 2 x 2 23.5, 1 x 4 40.5
    return launch_presplit<4, 2>(M, K, N, blocks, x, y, wk, stream);
}

}  // namespace q4
