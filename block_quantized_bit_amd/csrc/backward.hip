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
            o = in ? (uint32_t)(((size_t)n * (K / 256) + kb) * Q4K_BYTES + 16 + 32 * part) : OUT;
            rh = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               r_w, in ? (uint32_t)(((size_t)n * (K / 256) + kb) * Q4K_BYTES) : OUT, 0, 0));
        } else {
            o = in ? (uint32_t)((size_t)n * (K / 2) + (size_t)kb * 128 + 32 * part) : OUT;
            const int g0 = (kb * 256 + 32 * s0) / G, g1 = (kb * 256 + 32 * (s0 + 1)) / G;
            // the group offsets differ between lanes: per-lane offsets (a scalar offset
            // that varies over the wavefront makes the compiler loop over its values)
            const uint32_t ob = (uint32_t)((size_t)n * ngroups * 2);
            const uint32_t o0 = in ? ob + 2u * g0 : OUT, o1 = in ? ob + 2u * g1 : OUT;
            ra0 = __builtin_amdgcn_raw_buffer_load_b16(r_s, o0, 0, 0);
            ra1 = __builtin_amdgcn_raw_buffer_load_b16(r_s, o1, 0, 0);
            rb0 = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, o0, 0, 0) : 0u;
            rb1 = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, o1, 0, 0) : 0u;
        }
        // Q4_K blocks are 144 bytes: 16-byte aligned offsets (144 = 9 * 16), so 128-bit loads
        rc0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o, 0, 0));
        rc1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, o == OUT ? OUT : o + 16, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + BT * i, m = idx >> 6, r = idx & 63, nn = r0 + r;
            const uint32_t od = (m0 + m < M && nn < nend) ? (uint32_t)(((size_t)(m0 + m) * N + nn) * 4) : OUT;
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
// 4 per pass (2 with four activation rows) with the next pass's loads in
// flight. Per row and column the work is one byte conversion and M
// multiply-adds, acc += (dy * a) * q; the b term of w = a*q + b is the same
// for the 16 (or 32) columns of a sub-block, so dy * b is summed once per row
// and sub-block and added at the end. The wavefronts' sums are added in LDS in
// a fixed order, and the per-group partials go to the same workspace and
// reduce as above.
constexpr int RW = 8;        // wavefronts per workgroup
constexpr int KSL = 2048;    // K per workgroup (64 lanes x 32 weights)
constexpr int KPAD = KSL + KSL / 32;  // LDS row of the wave reduction: one pad float per 32

// rows per pass: 4, or 2 with four activation rows (registers)
template <int MR>
constexpr int rows_per_pass() { return MR >= 4 ? 2 : 4; }

template <int FMTB, int MR, int RR = rows_per_pass<MR>()>
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
    constexpr int RR = rows_per_pass<MR>();

    auto load = [&](RowPass<FMTB, MR>& P, int r0) {
#pragma unroll
        for (int i = 0; i < RR; ++i) {
            const int r = r0 + i;
            const bool in = uin && r < nrows;
            const uint32_t rb = (uint32_t)r * rowbytes;
            P.q[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, in ? rb + qoff : OUT, 0, 0));
            if (FMTB == 2) {
                P.h[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, in ? rb + hoff : OUT, 0, 0));
            } else {
                const uint32_t so = in ? (uint32_t)r * ngroups * 2u + soff : OUT;
                P.a[i] = __builtin_amdgcn_raw_buffer_load_b16(r_s, so, 0, 0);
                P.b[i] = FMTB == 1 ? __builtin_amdgcn_raw_buffer_load_b16(r_b, so, 0, 0) : (uint16_t)0;
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const uint32_t o = (m < M && r < nrows) ? (uint32_t)(((size_t)m * N + n0 + r) * 4) : OUT;
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

    RowPass<FMTB, MR> cur;
    load(cur, 0);
    for (int r0 = 0; r0 < nrows; r0 += RR) {
        RowPass<FMTB, MR> nxt;
        if (r0 + RR < nrows) load(nxt, r0 + RR);
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
        cur = nxt;
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
