// Input gradient with frozen 4-bit weights: dX [M][K] = dY [M][N] . dequant(W [N][K]).
//
// C-Kernel-Engine gemm_kernels_q4k.c, section "Backward Pass: Gradient w.r.t.
// Input": dL/dX = W^T . dL/dY with the weights dequantized on the fly and no
// weight gradient (the weights are frozen); the batched form is one such
// product per activation row. The same product is provided for Q4_0 and
// affine weights.
//
// The contraction runs over N, the weight rows. A workgroup owns one 256-wide
// column of K (one Q4_K super-block, or 8 Q4_0 blocks / 4 or 2 affine groups),
// one 16-row tile of dY and one range of weight rows. Every weight byte of the
// column and range is read once. Rows are staged through LDS 64 at a time
// (double-buffered; the next 64 rows' loads wait in registers meanwhile) in a
// common form: the column's 128 code bytes of the row and eight (a, b) pairs,
// one per 32-weight sub-block, with w = a*q + b:
//   Q4_K:   a = d * sc[s], b = -dmin * m[s]      (gemv_q4_k_ref: "w = d * q - m")
//   Q4_0:   a = d,         b = -8 d
//   affine: a = scale,     b = bias              of the sub-block's group
// Each of the 4 wavefronts owns 64 of the 256 k (four 16-wide tiles) and runs
// v_mfma_f32_16x16x4_f32 with dY rows as A (16 m x 4 n) and the dequantized
// weights as B (4 n x 16 k): each lane dequantizes one weight per MFMA.
// A second pass adds the per-range partial sums in a fixed order (no atomics).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int BT = 256;       // threads per workgroup (4 wavefronts)
constexpr int KCOL = 256;     // K per workgroup
constexpr int RC = 64;        // weight rows per LDS stage
constexpr int Q4K_BYTES = 144;
constexpr int RSRC_WORD3 = 0x00020000;
constexpr uint32_t OUT = 0x80000000u;
// Offset o where `in`, else o with bit 31 set (past every buffer range: reads
// zero). A bit operation rather than a select: with a condition the compiler
// can branch around the load and wait for every load in flight at the join.
__device__ __forceinline__ uint32_t sel(uint32_t o, bool in) { return o | ((uint32_t)!in << 31); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

struct BwdLds {
    uint8_t codes[RC][128 + 16];  // 16 bytes of padding per row
    float2 coef[RC][8];           // (a, b) per 32-weight sub-block
    float dy[16][RC + 4];         // dY tile, [m][n]
};

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

// Byte index and nibble shift of weight k (0..255) of a column.
template <int FMTB>
__device__ __forceinline__ void code_pos(int k, int& byte, int& shift) {
    if (FMTB == 2) {  // Q4_K: chunk c of 64 weights: low nibbles of qs[32c ..], then their high nibbles
        const int c = k >> 6, r = k & 63;
        byte = 32 * c + (r & 31);
        shift = (r >> 5) * 4;
    } else {          // Q4_0 / affine: block b of 32: low nibbles of bytes 16b .., then high nibbles
        const int b = k >> 5, j = k & 31;
        byte = 16 * b + (j & 15);
        shift = (j >> 4) * 4;
    }
}

// FMTB: 0 Q4_0 (G = 32), 1 affine (G = 64 / 128), 2 Q4_K (G = 256).
template <int FMTB, int G>
__global__ __launch_bounds__(BT, 2) void backward_partial_kernel(int M, int K, int N, int rows_per, const uint8_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ wscale,
                                                                 const uint16_t* __restrict__ wbias,
                                                                 const float* __restrict__ dy, float* __restrict__ work) {
    __shared__ BwdLds S[2];  // stage i in S[i & 1]; the next stage's loads wait in registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = blockIdx.x, nc = blockIdx.y, m0 = blockIdx.z * 16;
    const int nbeg = nc * rows_per, nend = min(N, nbeg + rows_per);
    const int nst = nend > nbeg ? (nend - nbeg + RC - 1) / RC : 0;  // 64-row stages of the range
    const int ngroups = K / G;

    const uint32_t wbytes = FMTB == 2 ? (uint32_t)((size_t)N * (K / 256) * Q4K_BYTES) : (uint32_t)((size_t)N * (K / 2));
    const __amdgpu_buffer_rsrc_t r_w = rsrc(w, wbytes);
    const __amdgpu_buffer_rsrc_t r_s = rsrc(wscale, FMTB == 2 ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    const __amdgpu_buffer_rsrc_t r_b = rsrc(wbias, FMTB == 1 ? (uint32_t)((size_t)N * ngroups * 2) : 0u);
    const __amdgpu_buffer_rsrc_t r_dy = rsrc(dy, (uint32_t)((size_t)M * N * 4));

    // this lane's four weights per MFMA step: column k = 64*wave + 16*j + lane%16
    int bidx[4], bsh[4], bsub[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = 64 * wave + 16 * j + (lane & 15);
        code_pos<FMTB>(k, bidx[j], bsh[j]);
        bsub[j] = k >> 5;
    }
    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // staging of one 64-row stage: thread (r, part) = (tid / 4, tid % 4) takes 32 code
    // bytes and two sub-blocks' (a, b) of row r; 4 dY values per thread
    const int sr = tid >> 2, part = tid & 3, s0 = 2 * part;
    uint4 rc0, rc1, rh;
    uint32_t ra0, ra1, rb0, rb1;
    float rdy[4];
    auto load = [&](int r0) {  // rows past the range read zero
        const int n = r0 + sr;
        const bool in = n < nend;
        uint32_t o = OUT;
        if (FMTB == 2) {
            o = sel((uint32_t)(((size_t)n * (K / 256) + kb) * Q4K_BYTES + 16 + 32 * part), in);
            rh = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               r_w, sel((uint32_t)(((size_t)n * (K / 256) + kb) * Q4K_BYTES), in), 0, 0));
        } else {
            o = sel((uint32_t)((size_t)n * (K / 2) + (size_t)kb * 128 + 32 * part), in);
            const int g0 = (kb * 256 + 32 * s0) / G, g1 = (kb * 256 + 32 * (s0 + 1)) / G;
            // the group offsets differ between lanes: per-lane offsets (a scalar offset
            // that varies over the wavefront makes the compiler loop over its values)
            const uint32_t ob = (uint32_t)((size_t)n * ngroups * 2);
            const uint32_t o0 = sel(ob + 2u * g0, in), o1 = sel(ob + 2u * g1, in);
            ra0 = __builtin_amdgcn_raw_buffer_load_b16(r_s, o0, 0, 0);
            ra1 = __builtin_amdgcn_raw_buffer_load_b16(r_s, o1, 0, 0);
            rb0 = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, o0, 0, 0) : 0u;
            rb1 = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, o1, 0, 0) : 0u;
        }
        // Q4_K blocks are 144 bytes: 16-byte aligned offsets (144 = 9 * 16), so 128-bit loads
        rc0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o, 0, 0));
        rc1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o + 16, 0, 0));  // bit 31 stays set
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + BT * i, m = idx >> 6, r = idx & 63, nn = r0 + r;
            const uint32_t od = sel((uint32_t)(((size_t)(m0 + m) * N + nn) * 4), m0 + m < M && nn < nend);
            rdy[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_dy, od, 0, 0));
        }
    };
    auto store = [&](BwdLds& T) {
        *reinterpret_cast<uint4*>(&T.codes[sr][32 * part]) = rc0;
        *reinterpret_cast<uint4*>(&T.codes[sr][32 * part + 16]) = rc1;
        float2 c0, c1;
        if (FMTB == 2) {
            const float d = half_to_float(rh.x & 0xFFFFu), dmin = half_to_float(rh.x >> 16);
            // the sixteen 6-bit fields of the 96-bit little-endian string in h.y, h.z, h.w
            const uint64_t lo = ((uint64_t)rh.z << 32) | rh.y;
            const uint32_t hi = rh.w;
            auto field = [&](int f) -> uint32_t {
                const int bit = 6 * f;
                if (bit + 6 <= 64) return (uint32_t)(lo >> bit) & 63u;
                if (bit >= 64) return (hi >> (bit - 64)) & 63u;
                return (uint32_t)((lo >> bit) | ((uint64_t)hi << (64 - bit))) & 63u;
            };
            c0 = make_float2(d * (float)field(s0), -dmin * (float)field(8 + s0));
            c1 = make_float2(d * (float)field(s0 + 1), -dmin * (float)field(8 + s0 + 1));
        } else if (FMTB == 0) {
            const float a0 = half_to_float(ra0), a1 = half_to_float(ra1);
            c0 = make_float2(a0, -8.0f * a0);
            c1 = make_float2(a1, -8.0f * a1);
        } else {
            c0 = make_float2(bf16_to_float(ra0), bf16_to_float(rb0));
            c1 = make_float2(bf16_to_float(ra1), bf16_to_float(rb1));
        }
        T.coef[sr][s0] = c0;
        T.coef[sr][s0 + 1] = c1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + BT * i, m = idx >> 6, r = idx & 63;
            T.dy[m][r] = rdy[i];
        }
    };

    if (nst > 0) {
        load(nbeg);
        store(S[0]);
        load(nbeg + RC);
    }
    for (int i = 0; i < nst; ++i) {
        __syncthreads();  // stage i is in S[i & 1]; every wavefront is done with S[(i + 1) & 1]
        if (i + 1 < nst) store(S[(i + 1) & 1]);
        load(nbeg + (i + 2) * RC);
        const BwdLds& T = S[i & 1];
#pragma unroll 4
        for (int st = 0; st < RC / 4; ++st) {
            const int rl = 4 * st + (lane >> 4);  // this lane's weight row in the stage
            const float aop = T.dy[lane & 15][rl];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = (T.codes[rl][bidx[j]] >> bsh[j]) & 15;
                const float2 c = T.coef[rl][bsub[j]];
                const float wv = c.x * (float)q + c.y;
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop, wv, acc[j], 0, 0, 0);
            }
        }
    }
    // D layout: lane holds column lane%16, rows 4*(lane/16) + r
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = kb * KCOL + 64 * wave + 16 * j + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * (lane >> 4) + r;
            if (m < M) work[((size_t)nc * M + m) * K + k] = acc[j][r];
        }
    }
}

// ---------------------------------------------------------------------------
// Few activation rows (M <= 4): the transposed product as a weight stream.
// A workgroup of RW wavefronts owns a 2048-wide slice of K and a group of
// weight rows; lane l owns the 16-byte code chunk l of the slice (32 weights,
// so 32 output columns), and each wavefront walks its own sub-range of rows,
// one (Q4_K) or two rows per pass with two passes of loads in flight. Per row
// and column the work is one byte conversion and M
// multiply-adds, acc += (dy * a) * q; the b term of w = a*q + b is the same
// for the 16 (or 32) columns of a sub-block, so dy * b is summed once per row
// and sub-block and added at the end. The wavefronts' sums are added in LDS in
// a fixed order, and the per-group partials go to the same workspace and
// reduce as above.
constexpr int RW = 8;        // wavefronts per workgroup
constexpr int KSL = 2048;    // K per workgroup (64 lanes x 32 weights)
constexpr int KPAD = KSL + KSL / 32;  // LDS row of the wave reduction: one pad float per 32

// Rows per pass (two passes in flight): 1 for Q4_K (a header and a code
// chunk per row), 2 otherwise. Measured at 4096 x 14336, M = 1 / 2 / 4 (us):
// Q4_K 14.4 / 17.2 / 24.4 with 1 row, 14.5 / 17.9-19.3 / 25.2 with 2, 16.4 /
// 20.3 / 25.0 with 4; Q4_0 14.5 / 16.7 / 20.5 with 1, 12.6 / 15.0 / 20.6
// with 2, 13.7 / 16.5 / 20.5 with 4; 8 rows was slower still.
template <int FMTB, int MR>
constexpr int rows_per_pass() { return FMTB == 2 ? 1 : 2; }

template <int FMTB, int MR, int RR = rows_per_pass<FMTB, MR>()>
struct RowPass {
    uint4 q[RR];      // the lane's code chunk of each row
    uint4 h[RR];      // Q4_K: the chunk's block header
    uint16_t a[RR], b[RR];  // Q4_0 / affine: raw scale and bias of the chunk's block or group
    float d[RR][MR];  // dY of each row for each activation row
};

template <int FMTB, int G, int MR>
__global__ __launch_bounds__(64 * RW) void backward_rows_kernel(int M, int K, int N, int rows_per_wave,
                                                                const uint8_t* __restrict__ w,
                                                                const uint16_t* __restrict__ wscale,
                                                                const uint16_t* __restrict__ wbias,
                                                                const float* __restrict__ dy,
                                                                float* __restrict__ work) {
    // partial sums of wavefronts 4..7, then of the pairs (w, w + 4); column k at
    // k + k / 32, which spreads a wavefront's 32-float strides over the banks
    __shared__ __attribute__((aligned(16))) float red[4][MR][KPAD];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k0 = blockIdx.x * KSL;
    const int u = k0 / 32 + lane;  // the lane's 32-weight chunk of the row
    const bool uin = u < K / 32;
    const int rg = blockIdx.y;
    const int n0 = (rg * RW + wave) * rows_per_wave;
    const int nrows = max(0, min(rows_per_wave, N - n0));
    const int ngroups = K / G;
    const uint32_t rowbytes = FMTB == 2 ? (uint32_t)(K / 256) * Q4K_BYTES : (uint32_t)(K / 2);

    // the wavefront's own rows: offsets past them read zero
    const __amdgpu_buffer_rsrc_t r_w = rsrc(w + (size_t)min(n0, N) * rowbytes, (uint32_t)nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t r_s =
        rsrc(wscale + (FMTB == 2 ? 0 : (size_t)min(n0, N) * ngroups), FMTB == 2 ? 0u : (uint32_t)nrows * ngroups * 2u);
    const __amdgpu_buffer_rsrc_t r_b =
        rsrc(wbias + (FMTB == 1 ? (size_t)min(n0, N) * ngroups : 0), FMTB == 1 ? (uint32_t)nrows * ngroups * 2u : 0u);
    const __amdgpu_buffer_rsrc_t r_dy = rsrc(dy, (uint32_t)((size_t)M * N * 4));

    // chunk offsets within a row
    const uint32_t qoff = FMTB == 2 ? (uint32_t)(u >> 3) * Q4K_BYTES + 16 + 16 * (u & 7) : 16u * u;
    const uint32_t hoff = (uint32_t)(u >> 3) * Q4K_BYTES;
    const uint32_t soff = 2u * (uint32_t)((32 * u) / G);
    const int c = (u & 7) >> 1;  // Q4_K: 64-weight chunk of the block
    constexpr int RR = rows_per_pass<FMTB, MR>();

    auto load = [&](RowPass<FMTB, MR>& P, int r0) {
#pragma unroll
        for (int i = 0; i < RR; ++i) {
            const int r = r0 + i;
            const bool in = uin && r < nrows;
            const uint32_t rb = (uint32_t)r * rowbytes;
            P.q[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, sel(rb + qoff, in), 0, 0));
            if (FMTB == 2) {
                P.h[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, sel(rb + hoff, in), 0, 0));
            } else {
                const uint32_t so = sel((uint32_t)r * ngroups * 2u + soff, in);
                P.a[i] = __builtin_amdgcn_raw_buffer_load_b16(r_s, so, 0, 0);
                P.b[i] = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, so, 0, 0) : (uint16_t)0;
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const uint32_t o = sel((uint32_t)(((size_t)m * N + n0 + r) * 4), m < M && r < nrows);
                P.d[i][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_dy, o, 0, 0));
            }
        }
    };

    float acc[MR][32], bs[MR][2];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
#pragma unroll
        for (int t = 0; t < 32; ++t) acc[m][t] = 0.0f;
        bs[m][0] = bs[m][1] = 0.0f;
    }

    // Two passes of loads in flight, in two slots that are refilled in place
    // after their compute (a register copy of loads in flight would wait for
    // them); no load is issued for passes past the wavefront's rows.
    auto compute = [&](const RowPass<FMTB, MR>& cur) {
#pragma unroll
        for (int i = 0; i < RR; ++i) {
            // w = a * q + b for the low-nibble (0) and high-nibble (1) halves of the chunk
            float a0, a1, b0, b1;
            if (FMTB == 2) {
                const float dd = half_to_float(cur.h[i].x & 0xFFFFu), dm = half_to_float(cur.h[i].x >> 16);
                const uint64_t lo = ((uint64_t)cur.h[i].z << 32) | cur.h[i].y;  // bits 0..63 of the 6-bit fields
                const uint64_t hi = ((uint64_t)cur.h[i].w << 32) | cur.h[i].z;  // bits 32..95
                const uint32_t sc = (uint32_t)(lo >> (12 * c)) & 0xFFFu;         // sc[2c], sc[2c+1]
                const uint32_t mn = (uint32_t)(hi >> (16 + 12 * c)) & 0xFFFu;    // m[2c], m[2c+1]
                a0 = dd * (float)(sc & 63u);
                a1 = dd * (float)(sc >> 6);
                b0 = -dm * (float)(mn & 63u);
                b1 = -dm * (float)(mn >> 6);
            } else if (FMTB == 0) {
                a0 = a1 = half_to_float(cur.a[i]);
                b0 = b1 = -8.0f * a0;
            } else {
                a0 = a1 = bf16_to_float(cur.a[i]);
                b0 = b1 = bf16_to_float(cur.b[i]);
            }
            const uint4 q = cur.q[i];
            const uint32_t ql[4] = {nibbles_lo(q.x), nibbles_lo(q.y), nibbles_lo(q.z), nibbles_lo(q.w)};
            const uint32_t qh[4] = {nibbles_hi(q.x), nibbles_hi(q.y), nibbles_hi(q.z), nibbles_hi(q.w)};
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float dv = cur.d[i][m];
                const float f0 = dv * a0, f1 = dv * a1;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    acc[m][t] = fmaf(f0, (float)((ql[t >> 2] >> (8 * (t & 3))) & 0xFFu), acc[m][t]);
                    acc[m][16 + t] = fmaf(f1, (float)((qh[t >> 2] >> (8 * (t & 3))) & 0xFFu), acc[m][16 + t]);
                }
                bs[m][0] = fmaf(dv, b0, bs[m][0]);
                bs[m][1] = fmaf(dv, b1, bs[m][1]);
            }
        }
    };
    RowPass<FMTB, MR> pa, pb;
    load(pa, 0);
    if (RR < nrows) load(pb, RR);
    for (int r0 = 0; r0 < nrows; r0 += 2 * RR) {
        compute(pa);
        if (r0 + 2 * RR < nrows) load(pa, r0 + 2 * RR);
        if (r0 + RR < nrows) {
            compute(pb);
            if (r0 + 3 * RR < nrows) load(pb, r0 + 3 * RR);
        }
    }

    // output column of each accumulator within the slice
    auto kcol = [&](int t) {
        const int lo = t & 15, half = t >> 4;
        if (FMTB == 2)  // block u/8, chunk c, l0 = 16 (u % 2): low nibbles at 64c + l0 + t, high at + 32
            return ((u >> 3) * 256 - k0) + 64 * c + 16 * (u & 1) + lo + 32 * half;
        return 32 * lane + 16 * half + lo;  // byte j: low nibble k = 32u + j, high nibble 32u + 16 + j
    };
    // fixed-order reduction of the 8 wavefronts: (w + (w + 4)) for w < 4, then
    // ((0 + 1) + (2 + 3)) of those
    static_assert(RW == 8, "the reduction pairs wavefronts w and w + 4");
    if (wave >= 4) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int t = 0; t < 32; ++t) {
                const int kk = kcol(t);
                red[wave - 4][m][kk + (kk >> 5)] = acc[m][t] + bs[m][t >> 4];
            }
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int t = 0; t < 32; ++t) {
                const int kk = kcol(t);
                float& slot = red[wave][m][kk + (kk >> 5)];
                slot = (acc[m][t] + bs[m][t >> 4]) + slot;
            }
    }
    __syncthreads();
    const int kn = min(KSL, K - k0);
    for (int i = threadIdx.x; i < MR * KSL; i += 64 * RW) {
        const int m = i / KSL, kk = i % KSL, kp = kk + (kk >> 5);
        if (m < M && kk < kn)
            work[((size_t)rg * M + m) * K + k0 + kk] = (red[0][m][kp] + red[1][m][kp]) + (red[2][m][kp] + red[3][m][kp]);
    }
}

// Q4_K input gradient on the f16 matrix cores (more than BWD_ROWS_MAX_M dY
// rows). The same decomposition as backward_partial_kernel (a workgroup owns
// one 256-wide column of K = one super-block, one 16-row tile of dY and one
// range of weight rows, staged 64 rows at a time), with the product
//   dx[m][k] = sum_n dy[m][n] (d[n] sc[n][s] q[n][k] - dmin[n] m[n][s])
// taken as two f16 matrix products into one accumulator, with v_mfma_f32_16x16x32_f16:
//   A = dy[m][n] d[n] * 2^e,    B = sc[n][s] q[n][k]      (exact in f16: <= 63 * 15)
//   A = dy[m][n] dmin[n] * 2^e, B = -m[n][s]              (exact in f16: <= 63)
// Each A enters as hi = f16(a) and lo = f16(a - hi); 2^e is a power of two per
// dY row and stage that brings the row's largest |A| into [2^14, 2^15), so
// hi + lo keep 22 of a's 24 significant bits, every product of a half with a
// B value is exact in f32 and the stage's sum differs from the float32 one by
// rounding only; it is scaled back by 2^-e into float accumulators. The B
// operand holds, per lane, the codes of 8 consecutive weight rows for one
// column k: the staging writes the column's code bytes transposed, [byte][row],
// by 4 x 4 byte transposes (v_perm) of 4 rows x 8 bytes per thread.
constexpr int CT = 72;  // bytes per transposed code row: 64 weight rows + 8 padding
constexpr int AT = 72;  // halves per staged A row: 64 weight rows + 8 padding
typedef _Float16 bv8h __attribute__((ext_vector_type(8)));
typedef _Float16 bv4h __attribute__((ext_vector_type(4)));
typedef _Float16 bv2h __attribute__((ext_vector_type(2)));

struct BwdF16Lds {
    uint8_t codes[128][CT];           // [qs byte j of the column][weight row n]
    _Float16 ahi[16][AT], alo[16][AT];  // dy * d * 2^e as two halves, [m][n]
    _Float16 bhi[16][AT], blo[16][AT];  // dy * dmin * 2^e
    _Float16 sc[8][64], nsc[8][64];     // sc[s][n] and -1024 sc[s][n]
    _Float16 nm[8][64];                 // -m[s][n]
    float inv[16];                      // 2^-e per dY row
};

// Largest magnitude over the 16 lanes of a DPP row (values are magnitudes:
// their bit patterns order as unsigned integers).
__device__ __forceinline__ float row16_max(float f) {
    uint32_t v = __builtin_bit_cast(uint32_t, f);
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
    return __builtin_bit_cast(float, v);
}

// Two codes (bytes 0 and 1 of w, or 2 and 3 when HI) times their rows' sc:
// 0x6400 | q is the half 1024 + q, and fma(1024 + q, sc, -1024 sc) = q sc exactly.
template <bool HI>
__device__ __forceinline__ uint32_t scaled_codes(uint32_t w, uint32_t scp, uint32_t nscp) {
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, w, HI ? 0x04030402u : 0x04010400u);
    const bv2h r = __builtin_elementwise_fma(__builtin_bit_cast(bv2h, h), __builtin_bit_cast(bv2h, scp),
                                             __builtin_bit_cast(bv2h, nscp));
    return __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(BT, 2) void backward_q4k_f16_kernel(int M, int K, int N, int rows_per, int nr,
                                                                 const uint8_t* __restrict__ w,
                                                                 const float* __restrict__ dy,
                                                                 float* __restrict__ work) {
    __shared__ BwdF16Lds S[2];  // stage i in S[i & 1]; the next stage's loads wait in registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroups are dispatched round-robin over the 8 XCDs. The 16 columns of
    // one (row range, dY tile) read neighbouring 144-byte super-blocks of the
    // same rows, whose cache lines they share, so they are mapped to one XCD
    // (one L2): workgroup b runs on XCD b % 8, and the XCD's workgroups take
    // the columns of its row groups x, x + 8, ... in turn.
    const int nkb = K / KCOL, ngrp = nr * (int)((M + 15) / 16);
    const int b = blockIdx.x, xcd = b & 7, t8 = b >> 3;
    const int grp = (t8 / nkb) * 8 + xcd, kb = t8 % nkb;
    if (grp >= ngrp) return;  // padding of the grid to whole rounds of 8
    const int nc = grp % nr, m0 = (grp / nr) * 16;
    const int nbeg = nc * rows_per, nend = min(N, nbeg + rows_per);
    const int nst = nend > nbeg ? (nend - nbeg + RC - 1) / RC : 0;  // 64-row stages of the range
    const int nsb = K / 256;
    const __amdgpu_buffer_rsrc_t r_w = rsrc(w, (uint32_t)((size_t)N * nsb * Q4K_BYTES));
    const __amdgpu_buffer_rsrc_t r_dy = rsrc(dy, (uint32_t)((size_t)M * N * 4));

    // staging roles of a thread within a 64-row stage
    const int crg = tid >> 4, cbg = tid & 15;      // codes: rows 4 crg .. + 3, qs bytes 8 cbg .. + 7
    const int hn = lane, hp = wave;                // header of row hn: 6-bit fields 4 hp .. 4 hp + 3
    const int am = tid >> 4, an = 4 * (tid & 15);  // A operands: dY row am, weight rows an .. an + 3

    // the next stage's loads wait in registers while a stage is computed
    uint2 rc[4];
    uint4 rh;
    float rdy[4];
    uint32_t rdd[4];
    // Offsets are selected against the out-of-range offset with a bit operation
    // (the buffer range check reads zero at offsets of 2^31 and above): with a
    // condition the compiler branches around the load and, at the join, waits
    // for every load in flight, which serialises the prefetch.
    const uint32_t rowb = (uint32_t)nsb * Q4K_BYTES, colb = (uint32_t)kb * Q4K_BYTES;
    const bool dyok = m0 + am < M;
    const uint32_t dyrow = (uint32_t)(m0 + am) * (uint32_t)N * 4u;
    auto load = [&](int r0) {  // rows past the range read zero
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = r0 + 4 * crg + i;
            rc[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  r_w, sel((uint32_t)n * rowb + colb + 16u + 8u * (uint32_t)cbg, n < nend),
                                                  0, 0));
        }
        {
            const int n = r0 + hn;
            rh = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               r_w, sel((uint32_t)n * rowb + colb, n < nend), 0, 0));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = r0 + an + i;
            const bool in = n < nend;
            rdy[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   r_dy, sel(dyrow + 4u * (uint32_t)n, in && dyok), 0, 0));
            rdd[i] = __builtin_amdgcn_raw_buffer_load_b32(r_w, sel((uint32_t)n * rowb + colb, in), 0, 0);
        }
    };
    auto store = [&](BwdF16Lds& T) {
        // codes: byte b of rows 4 crg .. + 3 into one dword of T.codes[8 cbg + b]
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
            const uint32_t w0 = hw ? rc[0].y : rc[0].x, w1 = hw ? rc[1].y : rc[1].x;
            const uint32_t w2 = hw ? rc[2].y : rc[2].x, w3 = hw ? rc[3].y : rc[3].x;
            const uint32_t t01a = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // r1.b1 r0.b1 r1.b0 r0.b0
            const uint32_t t01b = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // r1.b3 r0.b3 r1.b2 r0.b2
            const uint32_t t23a = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
            const uint32_t t23b = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
            const int j0 = 8 * cbg + 4 * hw;
            *reinterpret_cast<uint32_t*>(&T.codes[j0][4 * crg]) = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 1][4 * crg]) = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 2][4 * crg]) = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 3][4 * crg]) = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);
        }
        // the sixteen 6-bit fields of the 96-bit little-endian string in h.y, h.z, h.w:
        // field f < 8 is sc[f], f >= 8 is m[f - 8]
        {
            const uint64_t lo = (uint64_t)rh.y | ((uint64_t)rh.z << 32);  // bits 0..63
            const uint64_t hi = (uint64_t)rh.z | ((uint64_t)rh.w << 32);  // bits 32..95
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 4 * hp + i;
                const uint32_t v = f < 8 ? (uint32_t)(lo >> (6 * f)) & 63u : (uint32_t)(hi >> (6 * f - 32)) & 63u;
                const float fv = (float)v;
                if (f < 8) {
                    T.sc[f][hn] = (_Float16)fv;
                    T.nsc[f][hn] = (_Float16)(-1024.0f * fv);
                } else {
                    T.nm[f - 8][hn] = (_Float16)(-fv);
                }
            }
        }
        // A operands of dY row am and weight rows an .. an + 3
        {
            float va[4], vb[4], mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                va[i] = rdy[i] * half_to_float(rdd[i] & 0xFFFFu);
                vb[i] = rdy[i] * half_to_float(rdd[i] >> 16);
                mx = fmaxf(mx, fmaxf(fabsf(va[i]), fabsf(vb[i])));
            }
            mx = row16_max(mx);  // the 16 threads of dY row am form one DPP row
            const int E = max((int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 126, -111);
            const float sc = __builtin_bit_cast(float, (uint32_t)(127 + 15 - E) << 23);
            if ((tid & 15) == 0) T.inv[am] = __builtin_bit_cast(float, (uint32_t)(127 - 15 + E) << 23);
            bv4h ah, al, bh, bl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xa = va[i] * sc, xb = vb[i] * sc;
                ah[i] = (_Float16)xa;
                al[i] = (_Float16)(xa - (float)ah[i]);
                bh[i] = (_Float16)xb;
                bl[i] = (_Float16)(xb - (float)bh[i]);
            }
            *reinterpret_cast<bv4h*>(&T.ahi[am][an]) = ah;
            *reinterpret_cast<bv4h*>(&T.alo[am][an]) = al;
            *reinterpret_cast<bv4h*>(&T.bhi[am][an]) = bh;
            *reinterpret_cast<bv4h*>(&T.blo[am][an]) = bl;
        }
    };

    // wavefront w owns chunk c = w of the column: qs bytes 32c .. 32c + 31, i.e.
    // k = 64c + 32h + 16tt + col for the low (h = 0, sub-block 2c) and high
    // (h = 1, sub-block 2c + 1) nibbles; tile t = 2h + tt
    const int c = wave, g = lane >> 4, col = lane & 15;
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (nst > 0) {
        load(nbeg);
        store(S[0]);
        load(nbeg + RC);
    }
    auto do_stage = [&](int i, auto par) {
        constexpr int P = decltype(par)::value;  // i & 1
        __syncthreads();  // stage i is in S[P]; every wavefront is done with S[P ^ 1]
        if (i + 1 < nst) store(S[P ^ 1]);
        load(nbeg + (i + 2) * RC);
        const BwdF16Lds& T = S[P];
        v4f D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) D[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            const int nb = 32 * step + 8 * g;  // this lane's 8 weight rows of the 32-row step
            const bv8h Ahi = *reinterpret_cast<const bv8h*>(&T.ahi[col][nb]);
            const bv8h Alo = *reinterpret_cast<const bv8h*>(&T.alo[col][nb]);
            const bv8h Bhi = *reinterpret_cast<const bv8h*>(&T.bhi[col][nb]);
            const bv8h Blo = *reinterpret_cast<const bv8h*>(&T.blo[col][nb]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint2 cb = *reinterpret_cast<const uint2*>(&T.codes[32 * c + 16 * tt + col][nb]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int sbk = 2 * c + h;
                    const uint32_t w0 = h ? (cb.x >> 4) & 0x0F0F0F0Fu : cb.x & 0x0F0F0F0Fu;
                    const uint32_t w1 = h ? (cb.y >> 4) & 0x0F0F0F0Fu : cb.y & 0x0F0F0F0Fu;
                    const uint4 scp = *reinterpret_cast<const uint4*>(&T.sc[sbk][nb]);
                    const uint4 nsp = *reinterpret_cast<const uint4*>(&T.nsc[sbk][nb]);
                    const uint4 q = make_uint4(scaled_codes<false>(w0, scp.x, nsp.x), scaled_codes<true>(w0, scp.y, nsp.y),
                                               scaled_codes<false>(w1, scp.z, nsp.z), scaled_codes<true>(w1, scp.w, nsp.w));
                    const bv8h Bq = __builtin_bit_cast(bv8h, q);
                    const bv8h Bm = *reinterpret_cast<const bv8h*>(&T.nm[sbk][nb]);
                    const int t = 2 * h + tt;
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bq, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bq, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Bhi, Bm, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Blo, Bm, D[t], 0, 0, 0);
                }
            }
        }
        // D layout: lane (col, g) holds rows 4g .. 4g + 3 of column col
        const v4f iv = *reinterpret_cast<const v4f*>(&T.inv[4 * g]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(iv[r], D[t][r], acc[t][r]);
    };
    int i = 0;
    for (; i + 1 < nst; i += 2) {
        do_stage(i, std::integral_constant<int, 0>());
        do_stage(i + 1, std::integral_constant<int, 1>());
    }
    if (i < nst) do_stage(i, std::integral_constant<int, 0>());
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = kb * KCOL + 64 * c + 32 * (t >> 1) + 16 * (t & 1) + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * g + r;
            if (m < M) work[((size_t)nc * M + m) * K + k] = acc[t][r];
        }
    }
}

// Q4_0 input gradient on the f16 matrix cores (more than BWD_ROWS_MAX_M dY
// rows), with the decomposition of backward_q4k_f16_kernel (one 256-wide
// column of K = 8 blocks, one 16-row tile of dY, one range of weight rows,
// staged 64 rows at a time). The block scale d varies along K within the
// column, so it goes with the codes: per stage and block column b,
//   B = d[n][b] * 2^-t_b * (q[n][k] - 8),   A = dy[m][n] * 2^e
// where 2^-t_b brings the stage's largest |d| of column b into [2^10, 2^11)
// (|B| < 2^14: no f16 overflow whatever d), and B enters as hi = f16(B) and
// lo = f16(d' (q - 8) - hi), which is exact: d' (q - 8) has at most 15
// significant bits. A is the dY tile as hi/lo halves with a power of two per
// dY row and stage, as in the Q4_K kernel. Each (tile, 32-row step) is four
// products (hi.hi, hi.lo, lo.hi, lo.lo) into one accumulator, scaled back by
// 2^-e * 2^t_b (exact) into the float sums.
struct BwdQ0Lds {
    uint8_t codes[128][CT];             // [code byte j of the column][weight row n]
    _Float16 ahi[16][AT], alo[16][AT];  // dy * 2^e as two halves, [m][n]
    _Float16 dd[8][64];                 // d[n][b] * 2^-t_b, [b][n]
    float tb[8];                        // 2^t_b
    float inv[16];                      // 2^-e per dY row
};

// Largest magnitude over the 64 lanes of a wavefront (non-negative values:
// their bit patterns order as unsigned integers); every lane receives it.
__device__ __forceinline__ float wave64_max(float f) {
    uint32_t v = __builtin_bit_cast(uint32_t, row16_max(f));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return __builtin_bit_cast(float, max(max(r0, r1), max(r2, r3)));
}

// Two codes (bytes 0 and 1 of w, or 2 and 3 when HI) as the f16 pair q - 8:
// 0x6400 | q is the half 1024 + q.
template <bool HI>
__device__ __forceinline__ bv2h codes_m8(uint32_t w) {
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, w, HI ? 0x04030402u : 0x04010400u);
    return __builtin_bit_cast(bv2h, h) - bv2h{(_Float16)1032.0f, (_Float16)1032.0f};
}

__global__ __launch_bounds__(BT, 2) void backward_q4_0_f16_kernel(int M, int K, int N, int rows_per, int nr,
                                                                  const uint8_t* __restrict__ w,
                                                                  const uint16_t* __restrict__ wscale,
                                                                  const float* __restrict__ dy,
                                                                  float* __restrict__ work) {
    __shared__ BwdQ0Lds S[2];  // stage i in S[i & 1]; the next stage's loads wait in registers
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD mapping as in backward_q4k_f16_kernel: the 16 columns of one (row
    // range, dY tile) share cache lines of the same rows and run on one XCD
    const int nkb = K / KCOL, ngrp = nr * (int)((M + 15) / 16);
    const int b = blockIdx.x, xcd = b & 7, t8 = b >> 3;
    const int grp = (t8 / nkb) * 8 + xcd, kb = t8 % nkb;
    if (grp >= ngrp) return;  // padding of the grid to whole rounds of 8
    const int nc = grp % nr, m0 = (grp / nr) * 16;
    const int nbeg = nc * rows_per, nend = min(N, nbeg + rows_per);
    const int nst = nend > nbeg ? (nend - nbeg + RC - 1) / RC : 0;  // 64-row stages of the range
    const int ng = K / 32;
    const __amdgpu_buffer_rsrc_t r_w = rsrc(w, (uint32_t)((size_t)N * (K / 2)));
    const __amdgpu_buffer_rsrc_t r_s = rsrc(wscale, (uint32_t)((size_t)N * ng * 2));
    const __amdgpu_buffer_rsrc_t r_dy = rsrc(dy, (uint32_t)((size_t)M * N * 4));

    // staging roles of a thread within a 64-row stage
    const int crg = tid >> 4, cbg = tid & 15;      // codes: rows 4 crg .. + 3, bytes 8 cbg .. + 7
    const int hn = lane, hp = wave;                // scales: row hn, blocks 2 hp, 2 hp + 1
    const int am = tid >> 4, an = 4 * (tid & 15);  // A operands: dY row am, weight rows an .. an + 3

    uint2 rc[4];
    uint32_t rd[2];
    float rdy[4];
    // offsets selected against the out-of-range offset with a bit operation
    // (no branch around a load, so no wait at a join)
    const uint32_t rowb = (uint32_t)(K / 2), colb = (uint32_t)kb * 128u;
    const bool dyok = m0 + am < M;
    const uint32_t dyrow = (uint32_t)(m0 + am) * (uint32_t)N * 4u;
    auto load = [&](int r0) {  // rows past the range read zero
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = r0 + 4 * crg + i;
            rc[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  r_w, sel((uint32_t)n * rowb + colb + 8u * (uint32_t)cbg, n < nend),
                                                  0, 0));
        }
        {
            const int n = r0 + hn;
            const uint32_t o = sel(2u * ((uint32_t)n * (uint32_t)ng + 8u * (uint32_t)kb + 2u * (uint32_t)hp), n < nend);
            rd[0] = __builtin_amdgcn_raw_buffer_load_b16(r_s, o, 0, 0);
            rd[1] = __builtin_amdgcn_raw_buffer_load_b16(r_s, o + 2u, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = r0 + an + i;
            rdy[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   r_dy, sel(dyrow + 4u * (uint32_t)n, n < nend && dyok), 0, 0));
        }
    };
    auto store = [&](BwdQ0Lds& T) {
        // codes: byte b of rows 4 crg .. + 3 into one dword of T.codes[8 cbg + b]
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
            const uint32_t w0 = hw ? rc[0].y : rc[0].x, w1 = hw ? rc[1].y : rc[1].x;
            const uint32_t w2 = hw ? rc[2].y : rc[2].x, w3 = hw ? rc[3].y : rc[3].x;
            const uint32_t t01a = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
            const uint32_t t01b = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
            const uint32_t t23a = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
            const uint32_t t23b = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
            const int j0 = 8 * cbg + 4 * hw;
            *reinterpret_cast<uint32_t*>(&T.codes[j0][4 * crg]) = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 1][4 * crg]) = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 2][4 * crg]) = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);
            *reinterpret_cast<uint32_t*>(&T.codes[j0 + 3][4 * crg]) = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);
        }
        // block columns 2 hp, 2 hp + 1: the stage's largest |d| of each (this
        // wavefront's 64 lanes are the 64 rows) into [2^10, 2^11)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float dv = half_to_float(rd[i]);
            const float mx = wave64_max(fabsf(dv));
            const int E = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 127;  // mx = 1.f * 2^E
            const int t = max(E - 10, -100);  // an all-zero column keeps finite scales
            const float down = __builtin_bit_cast(float, (uint32_t)(127 - t) << 23);
            T.dd[2 * hp + i][hn] = (_Float16)(dv * down);
            if (lane == 0) T.tb[2 * hp + i] = __builtin_bit_cast(float, (uint32_t)(127 + t) << 23);
        }
        // A operands of dY row am and weight rows an .. an + 3
        {
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(rdy[i]));
            mx = row16_max(mx);  // the 16 threads of dY row am form one DPP row
            const int E = max((int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 126, -111);
            const float sc = __builtin_bit_cast(float, (uint32_t)(127 + 15 - E) << 23);
            if ((tid & 15) == 0) T.inv[am] = __builtin_bit_cast(float, (uint32_t)(127 - 15 + E) << 23);
            bv4h ah, al;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xa = rdy[i] * sc;
                ah[i] = (_Float16)xa;
                al[i] = (_Float16)(xa - (float)ah[i]);
            }
            *reinterpret_cast<bv4h*>(&T.ahi[am][an]) = ah;
            *reinterpret_cast<bv4h*>(&T.alo[am][an]) = al;
        }
    };

    // wavefront w owns blocks 2w and 2w + 1 of the column: k = 64w + 32bb + 16h
    // + col for block 2w + bb and nibble plane h (bytes 16 (2w + bb) + col);
    // tile t = 2 bb + h
    const int c = wave, g = lane >> 4, col = lane & 15;
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (nst > 0) {
        load(nbeg);
        store(S[0]);
        load(nbeg + RC);
    }
    auto do_stage = [&](int i, auto par) {
        constexpr int P = decltype(par)::value;  // i & 1
        __syncthreads();  // stage i is in S[P]; every wavefront is done with S[P ^ 1]
        if (i + 1 < nst) store(S[P ^ 1]);
        load(nbeg + (i + 2) * RC);
        const BwdQ0Lds& T = S[P];
        v4f D[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) D[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int step = 0; step < 2; ++step) {
            const int nb = 32 * step + 8 * g;  // this lane's 8 weight rows of the 32-row step
            const bv8h Ahi = *reinterpret_cast<const bv8h*>(&T.ahi[col][nb]);
            const bv8h Alo = *reinterpret_cast<const bv8h*>(&T.alo[col][nb]);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int blk = 2 * c + bb;
                const uint2 cb = *reinterpret_cast<const uint2*>(&T.codes[16 * blk + col][nb]);
                const uint4 dq = *reinterpret_cast<const uint4*>(&T.dd[blk][nb]);
                const bv2h d2[4] = {__builtin_bit_cast(bv2h, dq.x), __builtin_bit_cast(bv2h, dq.y),
                                    __builtin_bit_cast(bv2h, dq.z), __builtin_bit_cast(bv2h, dq.w)};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t w0 = h ? (cb.x >> 4) & 0x0F0F0F0Fu : cb.x & 0x0F0F0F0Fu;
                    const uint32_t w1 = h ? (cb.y >> 4) & 0x0F0F0F0Fu : cb.y & 0x0F0F0F0Fu;
                    const bv2h q2[4] = {codes_m8<false>(w0), codes_m8<true>(w0), codes_m8<false>(w1), codes_m8<true>(w1)};
                    bv8h Bhi, Blo;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const bv2h hi = d2[p] * q2[p];
                        const bv2h lo = __builtin_elementwise_fma(d2[p], q2[p], -hi);
                        Bhi[2 * p] = hi[0], Bhi[2 * p + 1] = hi[1];
                        Blo[2 * p] = lo[0], Blo[2 * p + 1] = lo[1];
                    }
                    const int t = 2 * bb + h;
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Bhi, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, Blo, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Bhi, D[t], 0, 0, 0);
                    D[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, Blo, D[t], 0, 0, 0);
                }
            }
        }
        // D layout: lane (col, g) holds rows 4g .. 4g + 3 of column col
        const v4f iv = *reinterpret_cast<const v4f*>(&T.inv[4 * g]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float up = T.tb[2 * c + (t >> 1)];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(iv[r] * up, D[t][r], acc[t][r]);
        }
    };
    int i = 0;
    for (; i + 1 < nst; i += 2) {
        do_stage(i, std::integral_constant<int, 0>());
        do_stage(i + 1, std::integral_constant<int, 1>());
    }
    if (i < nst) do_stage(i, std::integral_constant<int, 0>());
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = kb * KCOL + 64 * c + 32 * (t >> 1) + 16 * (t & 1) + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * g + r;
            if (m < M) work[((size_t)nc * M + m) * K + k] = acc[t][r];
        }
    }
}

// dx[m][k] = sum over ranges c of work[c][m][k] in a fixed order: a workgroup
// of 8 wavefronts takes 64 consecutive outputs; wavefront w sums ranges
// w, w + 8, w + 16, ... in order (loads issued 16 at a time), and the eight
// sums are added as ((0 + 1) + (2 + 3)) + ((4 + 5) + (6 + 7)).
constexpr int RED_W = 8;
__global__ __launch_bounds__(64 * RED_W) void backward_reduce_kernel(long long total, int nranges,
                                                                     const float* __restrict__ work,
                                                                     float* __restrict__ dx) {
    __shared__ float part[RED_W][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long i = (long long)blockIdx.x * 64 + lane;
    const bool in = i < total;
    constexpr int U16 = 16;
    float s = 0.0f;
    int c = wave;
    for (; c + RED_W * (U16 - 1) < nranges; c += RED_W * U16) {
        float v[U16];
#pragma unroll
        for (int j = 0; j < U16; ++j) v[j] = in ? work[(size_t)(c + RED_W * j) * total + i] : 0.0f;
#pragma unroll
        for (int j = 0; j < U16; ++j) s += v[j];
    }
    for (; c < nranges; c += RED_W) s += in ? work[(size_t)c * total + i] : 0.0f;
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && in) {
        const float a = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
        const float b = (part[4][lane] + part[5][lane]) + (part[6][lane] + part[7][lane]);
        dx[i] = a + b;
    }
}

template <int FMTB, int G, int MR>
hipError_t launch_rows(int M, int K, int N, const uint8_t* w, const void* ws, const void* wb, const float* dy,
                       float* dx, float* work, hipStream_t stream) {
    const int ng = backward_ranges(M, K, N);
    const int rpw = (N + ng * RW - 1) / (ng * RW);
    const dim3 grid((K + KSL - 1) / KSL, ng);
    hipLaunchKernelGGL((backward_rows_kernel<FMTB, G, MR>), grid, dim3(64 * RW), 0, stream, M, K, N, rpw, w,
                       static_cast<const uint16_t*>(ws), static_cast<const uint16_t*>(wb), dy, work);
    const long long total = (long long)M * K;
    hipLaunchKernelGGL(backward_reduce_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64 * RED_W), 0, stream, total,
                       ng, work, dx);
    return hipGetLastError();
}

template <int FMTB, int G>
hipError_t launch_b(int M, int K, int N, const uint8_t* w, const void* ws, const void* wb, const float* dy, float* dx,
                    float* work, hipStream_t stream) {
    if (M == 1) return launch_rows<FMTB, G, 1>(M, K, N, w, ws, wb, dy, dx, work, stream);
    if (M == 2) return launch_rows<FMTB, G, 2>(M, K, N, w, ws, wb, dy, dx, work, stream);
    if (M <= BWD_ROWS_MAX_M) return launch_rows<FMTB, G, 4>(M, K, N, w, ws, wb, dy, dx, work, stream);
    const int nr = backward_ranges(M, K, N);
    const int rows_per = (N + nr - 1) / nr;
    const dim3 grid(K / KCOL, nr, (M + 15) / 16);
    if (FMTB == 2 || FMTB == 0) {
        const long long ngrp = (long long)nr * ((M + 15) / 16);
        const unsigned nwg = (unsigned)(((ngrp + 7) / 8) * 8 * (K / KCOL));
        if (FMTB == 2)
            hipLaunchKernelGGL(backward_q4k_f16_kernel, dim3(nwg), dim3(BT), 0, stream, M, K, N, rows_per, nr, w, dy,
                               work);
        else
            hipLaunchKernelGGL(backward_q4_0_f16_kernel, dim3(nwg), dim3(BT), 0, stream, M, K, N, rows_per, nr, w,
                               static_cast<const uint16_t*>(ws), dy, work);
    } else
        hipLaunchKernelGGL((backward_partial_kernel<FMTB, G>), grid, dim3(BT), 0, stream, M, K, N, rows_per, w,
                           static_cast<const uint16_t*>(ws), static_cast<const uint16_t*>(wb), dy, work);
    const long long total = (long long)M * K;
    hipLaunchKernelGGL(backward_reduce_kernel, dim3((unsigned)((total + 63) / 64)), dim3(64 * RED_W), 0, stream, total,
                       nr, work, dx);
    return hipGetLastError();
}

}  // namespace

// Weight-row ranges. Up to BWD_ROWS_MAX_M activation rows: row groups of the
// weight-stream kernel, for about 2048 wavefronts and at least 4 rows per
// wavefront. Otherwise: enough workgroups to fill the chip (about 512), ranges
// of at least 64 rows.
int backward_ranges(int M, int K, int N) {
    if (M <= BWD_ROWS_MAX_M) {
        const long long slices = (K + KSL - 1) / KSL;
        long long ng = (2048 / RW + slices - 1) / slices;
        const long long max_ng = (N + 4 * RW - 1) / (4 * RW);
        if (ng > max_ng) ng = max_ng;
        if (ng < 1) ng = 1;
        return (int)ng;
    }
    const long long cols = (long long)(K / KCOL) * ((M + 15) / 16);
    long long nr = (512 + cols - 1) / cols;
    const long long max_nr = (N + RC - 1) / RC;
    if (nr > max_nr) nr = max_nr;
    if (nr < 1) nr = 1;
    return (int)nr;
}

hipError_t launch_backward(int M, int K, int N, int fmt, int bs, const uint8_t* w, const void* wscale,
                           const void* wbias, const float* dy, float* dx, float* work, hipStream_t stream) {
    if (fmt == 2) return launch_b<2, 256>(M, K, N, w, nullptr, nullptr, dy, dx, work, stream);
    if (fmt == 0) return launch_b<0, 32>(M, K, N, w, wscale, nullptr, dy, dx, work, stream);
    if (bs == 64) return launch_b<1, 64>(M, K, N, w, wscale, wbias, dy, dx, work, stream);
    if (bs == 128) return launch_b<1, 128>(M, K, N, w, wscale, wbias, dy, dx, work, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
