// Few-row W4A8 product (up to 32 activation rows, 4-bit Q4_0 or affine codes)
// that streams the weights the way the decode GEMV does and takes the block
// dots on the int8 matrix cores.
//
// tract PR #2432 (follow-up decode measurements): the weights dominate the
// traffic of a decode-sized product, so they are streamed once for all rows.
// meTile PR #29 ("Why int4 wins is bandwidth, not batching"): while a product
// stays bound by its weight stream, a few more activation rows should cost
// little more time than one.
//
// Mapping. A workgroup of 16 wavefronts (8 for 17..32 rows) owns 16
// consecutive weight rows. The blocks of a row are taken four at a time (a
// "quad": 128 weights, 64 bytes of codes per row) and the wavefronts take the
// quads round-robin, so the workgroup's loads in flight cover a contiguous
// stretch of every row. In a
// wavefront, lane (q, c) = (l / 16, l % 16) loads block 4j + q of weight row c
// (one 128-bit load) and the 32 activation codes of block 4j + q of activation
// row c of each 16-row tile (two). A 4x4 transpose of dwords across the four
// 16-lane rows (two v_permlane16_swap, two v_permlane32_swap) then leaves lane
// (q, c) with dword q of each of the quad's four blocks. For block k its low
// nibbles are weights 4q .. 4q+3 and its high nibbles weights 16+4q .. 19+4q,
// which pair with activation dwords q and 4 + q of the block (transposed the
// same way): the lane's eight-code K slice of v_mfma_i32_16x16x32_i8 (A:
// activation row c, B: weight row c). The order of the 32 products of a block
// does not change its integer sum. D then holds weight row c and activation
// rows 4q .. 4q+3 of the tile.
//
// Rescale per block (Q4_0) or group (affine, 2 or 4 blocks), as in the tiled
// GEMM: each MFMA chain starts from the integer 0x4B400000 (the bits of
// C = 1.5 * 2^23), so it ends on the bits of the float C + P, and one FMA with
// the exact constant -d * C gives d * P rounded once:
//   Q4_0:   acc += xs[m] * (d[n] * P)                         P from codes q - 8
//   affine: acc += xs[m] * (s[n] * A) + (xs * xsum)[m] * b[n]
// Q4_0 codes enter the MFMA as the bytes 16 * (q - 8) (the nibble q ^ 8 in the
// high half of a byte: an XOR, a shift and ANDs per dword, no sign fix-up), so
// the chain holds 16 * P (within 2^22) and every product and sum of the
// rescale is 16 times the one above, each rounded at the same relative place;
// the final sum is scaled back by 1/16, exactly.
// The activation scales of all of K are staged in LDS once per workgroup,
// group-major, while the first quad's loads are in flight. The 16
// wavefronts' float tiles are added in LDS in a fixed order (no atomics).
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

// Wavefronts per workgroup: 16 for one 16-row activation tile, 8 for two
// (measured, Q4_0 24 and 32 rows: 4096 x 14336 24.9 -> 21.9 us and 27.9 ->
// 25.3 us, 14336 x 4096 21.6 -> 20.9 and 24.7 -> 24.2, 4096 x 4096 within
// 2%; with 3..16 rows 8 wavefronts were up to 6% slower)
constexpr int rows_waves(int mt) { return mt == 1 ? 16 : 8; }
constexpr int RN = 16;          // weight rows per workgroup
constexpr int RSRC_WORD3 = 0x00020000;
constexpr uint32_t OUT = 0x80000000u;  // beyond every buffer range: reads as zero
constexpr int W_AUX = 2;               // non-temporal weight loads: each weight byte is read once
constexpr int CHAIN_BIAS = 0x4B400000;
constexpr float CHAIN_BIAS_F = 12582912.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

// Offset o where `in`, else one past every buffer range (reads zero); a select
// rather than a branch, so no wait is forced at a join.
__device__ __forceinline__ uint32_t sel(uint32_t o, bool in) { return o | ((uint32_t)!in << 31); }

// 4x4 transpose of dwords across the four 16-lane rows of a wavefront: on
// entry the lanes of row r hold X[r][0..3] in v0..v3, on exit vk = X[k][r].
// First the 2x2 blocks' own elements: within rows (0,1) and (2,3), (even row,
// odd dword) and (odd row, even dword) swap; then the blocks: dwords 2, 3 of
// rows 0, 1 swap with dwords 0, 1 of rows 2, 3.
__device__ __forceinline__ void transpose4(uint32_t& v0, uint32_t& v1, uint32_t& v2, uint32_t& v3) {
    const auto a = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    v0 = c[0];
    v2 = c[1];
    v1 = d[0];
    v3 = d[1];
}

// One quad's loads, kept as loaded until its compute uses them, so that loads
// in flight across loop iterations are never moved between registers (a move
// would wait for the load). Besides the codes, lane l carries one activation
// scale (and code sum) of row 16u + l / 4 and one weight scale (and bias) of
// weight row l / 4, both of the quad's (l % 4)-th block or group.
template <int MT>
struct Quad {
    uint4 w;            // weight block 4j + q of row c
    uint4 a[MT][2];     // activation block 4j + q of row 16u + c (two halves)
    float xs[MT];       // activation scale
    int xsum[MT];       // activation code sum (affine)
    uint16_t ws, wb;    // weight scale and bias (bias: affine)
};

// Dynamic LDS: per wavefront, the scales of the quad being computed
// (activation scales [4][MR] floats, affine also xs * xsum [4][MR], then weight
// scales [16][4] and affine biases [16][4] as 16-bit values); after them the
// wavefronts' float tiles for the final sum.
constexpr int wave_lds_bytes(int fmt, int mt) { return (fmt == 1 ? 2 : 1) * (4 * 16 * mt * 4 + 16 * 4 * 2); }

size_t rows_mfma_lds(int fmt, int mt) {
    return (size_t)rows_waves(mt) * wave_lds_bytes(fmt, mt) + (size_t)rows_waves(mt) * mt * 256 * 4;
}

// DEPTH: quads in flight per wavefront (2, or 4 for long rows). With one
// 16-row tile and two quads in flight the kernel fits 64 registers, so two
// workgroups share a CU.
// HALF (at most 8 activation rows): one 128-bit load per quad brings rows
// 0..7 of the activation tile, lanes c < 8 taking the first and lanes c + 8
// the second half of row c's block; after the transpose a DPP row rotation by
// 8 lanes hands each lane c < 8 its second-half dwords.
template <int FMT, int G, int MT, bool PARTIALS, int DEPTH, bool HALF>
__global__ __launch_bounds__(64 * rows_waves(MT), (MT == 1 && DEPTH == 2 && !(FMT == 1 && G == 64)) ? 8 : 4) void rows_mfma_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ wscale,
                                                       const uint16_t* __restrict__ wbias,
                                                       const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                       const int32_t* __restrict__ xsum, float* __restrict__ y,
                                                       int32_t* __restrict__ partials) {
    constexpr bool AFF = FMT == 1;
    constexpr int MR = 16 * MT;
    constexpr int RW = rows_waves(MT), RNT = 64 * RW;
    static_assert(!HALF || MT == 1, "the half tile is one 16-row tile");
    using Q = Quad<MT>;
    constexpr int SPG = G / 32;   // blocks per group
    constexpr int NS = 4 / SPG;   // groups per quad
    extern __shared__ __attribute__((aligned(16))) float rows_smem[];
    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, c = lane & 15;
    const int lr = lane >> 2, ls = lane & 3;  // scale loads: row l / 4, slot l % 4
    const int n0 = blockIdx.x * RN;
    const int nrows = min(RN, N - n0);
    const int nb = K >> 5, ng = K / G, nq = (nb + 3) >> 2;
    const uint32_t rowbytes = (uint32_t)(K >> 1);
    float* xsw = rows_smem + wave * (wave_lds_bytes(FMT, MT) / 4);  // [4][MR]
    float* xbw = xsw + 4 * MR;                                       // [4][MR] (affine)
    uint16_t* wsw = reinterpret_cast<uint16_t*>(xsw + (AFF ? 8 : 4) * MR);  // [16][4]
    uint16_t* wbw = wsw + 64;                                        // [16][4] (affine)
    float* red = rows_smem + RW * (wave_lds_bytes(FMT, MT) / 4);     // [RW][MT * 256]

    const __amdgpu_buffer_rsrc_t r_w = rsrc(wq + (size_t)n0 * rowbytes, (uint32_t)nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t r_s = rsrc(wscale + (size_t)n0 * ng, PARTIALS ? 0u : (uint32_t)nrows * ng * 2u);
    const __amdgpu_buffer_rsrc_t r_b =
        rsrc(wbias + (size_t)n0 * ng, (PARTIALS || !AFF) ? 0u : (uint32_t)nrows * ng * 2u);
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)M * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t r_xs = rsrc(xs, PARTIALS ? 0u : (uint32_t)M * ng * 4u);
    const __amdgpu_buffer_rsrc_t r_sx = rsrc(xsum, (PARTIALS || !AFF) ? 0u : (uint32_t)M * ng * 4u);

    auto load = [&](Q& t, int j) {
        // the scales first: compute stores them to LDS before it needs the codes
        if (!PARTIALS) {
            const int g = (4 * j) / SPG + ls;  // groups past K and slots past NS read zero
            const bool gin = ls < NS && g < ng;
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                const int m = 16 * u + lr;
                const uint32_t o = sel(4u * (uint32_t)(m * ng + g), gin && m < M);
                t.xs[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_xs, o, 0, 0));
                t.xsum[u] = AFF ? (int)__builtin_amdgcn_raw_buffer_load_b32(r_sx, o, 0, 0) : 0;
            }
            const uint32_t os = sel(2u * (uint32_t)(lr * ng + g), gin);  // rows past N: beyond the range
            t.ws = __builtin_amdgcn_raw_buffer_load_b16(r_s, os, 0, 0);
            t.wb = AFF ? __builtin_amdgcn_raw_buffer_load_b16(r_b, os, 0, 0) : (uint16_t)0;
        }
        const int blk = 4 * j + q;
        const bool in = blk < nb;
        t.w = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, sel(c * rowbytes + 16u * blk, in), 0, W_AUX));
        if (HALF) {
            const int m = c & 7;
            const uint32_t o = sel((uint32_t)m * (uint32_t)K + 32u * blk + 16u * (c >> 3), in && m < M);
            t.a[0][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, o, 0, 0));
            return;
        }
#pragma unroll
        for (int u = 0; u < MT; ++u) {
            const int m = 16 * u + c;
            const uint32_t o = sel((uint32_t)m * (uint32_t)K + 32u * blk, in && m < M);
            t.a[u][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, o, 0, 0));
            t.a[u][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, o + 16u, 0, 0));
        }
    };

    float acc[MT][4];
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[u][i] = 0.0f;
    const v4i bias = {CHAIN_BIAS, CHAIN_BIAS, CHAIN_BIAS, CHAIN_BIAS};

    auto compute = [&](const Q& t, int j) {
        // no instruction crosses a quad's start or end: a scheduler that
        // interleaves two quads makes the first wait for the second's loads
        __builtin_amdgcn_sched_barrier(0);
        // the quad's scales through this wavefront's LDS slots (written and
        // read by this wavefront only, in program order): lane (q, c) then
        // reads the activation scales of rows 4q .. 4q+3 as one float4 per
        // group, and the weight scales of row c as one 8-byte read
        uint16_t sq[4], bq[4];
        if (!PARTIALS) {
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                xsw[ls * MR + 16 * u + lr] = t.xs[u];
                if (AFF) xbw[ls * MR + 16 * u + lr] = t.xs[u] * (float)t.xsum[u];
            }
            wsw[lr * 4 + ls] = t.ws;
            if (AFF) wbw[lr * 4 + ls] = t.wb;
            const uint2 v = *reinterpret_cast<const uint2*>(&wsw[c * 4]);
            sq[0] = (uint16_t)v.x, sq[1] = (uint16_t)(v.x >> 16), sq[2] = (uint16_t)v.y, sq[3] = (uint16_t)(v.y >> 16);
            if (AFF) {
                const uint2 b = *reinterpret_cast<const uint2*>(&wbw[c * 4]);
                bq[0] = (uint16_t)b.x, bq[1] = (uint16_t)(b.x >> 16), bq[2] = (uint16_t)b.y, bq[3] = (uint16_t)(b.y >> 16);
            }
        }
        uint32_t w[4] = {t.w.x, t.w.y, t.w.z, t.w.w};
        uint32_t a[MT][8];
        transpose4(w[0], w[1], w[2], w[3]);
        if (HALF) {
            a[0][0] = t.a[0][0].x, a[0][1] = t.a[0][0].y, a[0][2] = t.a[0][0].z, a[0][3] = t.a[0][0].w;
            transpose4(a[0][0], a[0][1], a[0][2], a[0][3]);
#pragma unroll
            for (int k = 0; k < 4; ++k)  // row_ror:8 within each 16-lane row
                a[0][4 + k] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a[0][k], 0x128, 0xF, 0xF, false);
        }
#pragma unroll
        for (int u = 0; u < MT && !HALF; ++u) {
            a[u][0] = t.a[u][0].x, a[u][1] = t.a[u][0].y, a[u][2] = t.a[u][0].z, a[u][3] = t.a[u][0].w;
            a[u][4] = t.a[u][1].x, a[u][5] = t.a[u][1].y, a[u][6] = t.a[u][1].z, a[u][7] = t.a[u][1].w;
            transpose4(a[u][0], a[u][1], a[u][2], a[u][3]);
            transpose4(a[u][4], a[u][5], a[u][6], a[u][7]);
        }
        v4i D[MT];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t lo, hi;
            if (FMT == 0) {
                // nibble q ^ 8 in the high half of a byte is the int8 16 * (q - 8)
                const uint32_t f = w[k] ^ 0x88888888u;
                lo = (f << 4) & 0xF0F0F0F0u;
                hi = f & 0xF0F0F0F0u;
            } else {
                lo = lo_nibbles(w[k]);
                hi = hi_nibbles(w[k]);
            }
            const long bop = (long)(((uint64_t)hi << 32) | lo);
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                const long aop = (long)(((uint64_t)a[u][4 + k] << 32) | a[u][k]);
                D[u] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, (k % SPG) == 0 ? bias : D[u], 0, 0, 0);
            }
            if ((k % SPG) != SPG - 1) continue;
            const int e = k / SPG;            // group slot within the quad
            const int g = (4 * j + k) / SPG;  // group (block for Q4_0) just completed
            if (PARTIALS) {
                const int n = n0 + c;
#pragma unroll
                for (int u = 0; u < MT; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 16 * u + 4 * q + i;
                        const int d = D[u][i];
                        if (g < ng && m < M && c < nrows)
                            partials[((size_t)m * N + n) * ng + g] = (d - CHAIN_BIAS) >> (FMT == 0 ? 4 : 0);
                    }
                continue;
            }
            // past K: zero codes, scales and biases, so the terms are zero
            const float sv = AFF ? bf16_to_float(sq[e]) : half_to_float(sq[e]);
            const float sc = sv * -CHAIN_BIAS_F;  // exact
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                const float4 xv = *reinterpret_cast<const float4*>(&xsw[e * MR + 16 * u + 4 * q]);
                const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int di = D[u][i];
                    acc[u][i] = fmaf(xa[i], fmaf(sv, __builtin_bit_cast(float, di), sc), acc[u][i]);
                }
                if (AFF) {
                    const float bv = bf16_to_float(bq[e]);
                    const float4 bb = *reinterpret_cast<const float4*>(&xbw[e * MR + 16 * u + 4 * q]);
                    const float xb[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(xb[i], bv, acc[u][i]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // DEPTH quads in flight per wavefront (quads past the end read zero):
    // the loop computes DEPTH quads and refills each slot as it is freed;
    // the last quads are computed after it
    Q qa, qb, qc, qd;  // qc, qd: DEPTH 4
    load(qa, wave);
    __builtin_amdgcn_sched_barrier(0);
    load(qb, wave + RW);
    if constexpr (DEPTH == 4) {
        __builtin_amdgcn_sched_barrier(0);
        load(qc, wave + 2 * RW);
        __builtin_amdgcn_sched_barrier(0);
        load(qd, wave + 3 * RW);
    }
    int j = wave;
    for (; j + DEPTH * RW < nq; j += DEPTH * RW) {
        compute(qa, j);
        load(qa, j + DEPTH * RW);
        compute(qb, j + RW);
        load(qb, j + (DEPTH + 1) * RW);
        if constexpr (DEPTH == 4) {
            compute(qc, j + 2 * RW);
            load(qc, j + 6 * RW);
            compute(qd, j + 3 * RW);
            load(qd, j + 7 * RW);
        }
    }
    if (j < nq) compute(qa, j);
    if (j + RW < nq) compute(qb, j + RW);
    if constexpr (DEPTH == 4) {
        if (j + 2 * RW < nq) compute(qc, j + 2 * RW);
        if (j + 3 * RW < nq) compute(qd, j + 3 * RW);
    }
    if (PARTIALS) return;

    // fixed-order sum of the wavefronts' tiles: red[w][16 m + n]
#pragma unroll
    for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave * (MT * 256) + 256 * u + 16 * (4 * q + i) + c] = acc[u][i];
    __syncthreads();
    for (int e = tid; e < MT * 256; e += RNT) {
        const int m = e >> 4, n = e & 15;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < RW; ++w) s += red[w * (MT * 256) + e];
        if (m < M && n < nrows) y[(size_t)m * N + n0 + n] = FMT == 0 ? s * 0.0625f : s;
    }
}

template <int FMT, int G, int MT>
hipError_t launch_mt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias, const int8_t* xq,
                     const float* xs, const int32_t* xsum, float* y, int32_t* partials, hipStream_t stream) {
    const size_t lds = rows_mfma_lds(FMT, MT);
    // one 16-row tile: four quads in flight once a wavefront has at least four
    // to do; up to 8 rows: the half tile
    constexpr int DEEP = MT == 1 ? 4 : 2;
    constexpr int RW = rows_waves(MT);
    const bool deep = (K / 128) >= 4 * RW;
    decltype(&rows_mfma_kernel<FMT, G, MT, true, 2, false>) k;
    if (MT == 1 && M <= 8)
        k = partials ? (deep ? rows_mfma_kernel<FMT, G, MT, true, DEEP, MT == 1>
                             : rows_mfma_kernel<FMT, G, MT, true, 2, MT == 1>)
                     : (deep ? rows_mfma_kernel<FMT, G, MT, false, DEEP, MT == 1>
                             : rows_mfma_kernel<FMT, G, MT, false, 2, MT == 1>);
    else
        k = partials ? (deep ? rows_mfma_kernel<FMT, G, MT, true, DEEP, false> : rows_mfma_kernel<FMT, G, MT, true, 2, false>)
                     : (deep ? rows_mfma_kernel<FMT, G, MT, false, DEEP, false> : rows_mfma_kernel<FMT, G, MT, false, 2, false>);
    if (lds > 64 * 1024) {
        const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(k), lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)((N + RN - 1) / RN)), dim3(64 * RW), lds, stream, M, K, N, wq,
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

bool rows_mfma_fits(int M, int K, int bs, int fmt, int bits) {
    (void)fmt;
    return bits == 4 && M >= 1 && M <= ROWS_MFMA_MAX_M && K >= 32 && K % bs == 0;
}

hipError_t launch_rows_mfma(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                            const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                            int32_t* partials, hipStream_t stream) {
    if (!rows_mfma_fits(M, K, fmt == 0 ? 32 : bs, fmt, 4)) return hipErrorInvalidValue;
    if (fmt == 0) return launch_fmt<0, 32>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_fmt<1, 64>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_fmt<1, 128>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
