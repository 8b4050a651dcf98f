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
// of a wavefront reads 1 KiB of contiguous codes with 128-bit loads.
// Every load is a buffer load with no branch around it: a wavefront's buffer
// range covers only its own rows, and an offset past the end reads zero, so
// rows past N and chunks past K need no bounds branches (a branch around a
// load makes the compiler wait for it at the branch's end, which serialised
// the passes). Scales stay raw 16-bit values until they are used.
// Order of a launch: the fused variant first issues the loads of its
// activations, then the first pass of code and scale loads, and quantizes x
// into LDS while those are in flight (block maxima and sums combine over 8 or
// 16 lanes with DPP row operations); a large workgroup (16 wavefronts) shares
// that work. Each pass then prefetches the next pass's loads before its own
// arithmetic. The plain variant reads each chunk's codes straight from global
// memory (or, as a tuning option, copies them to LDS first). Each lane reads
// its chunk's 32 codes once and reuses them for all R rows.
// The two nibble planes of a chunk pair with the two 16-byte halves of the
// activation block, so the unpack is one AND (low) and one shift + AND (high)
// per dword with no byte shuffles; eight v_dot4_i32_i8 give the block's
// integer dot. Float partial sums are reduced across the wavefront with DPP
// row operations and lane reads.
#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int RSRC_WORD3 = 0x00020000;
constexpr uint32_t OUT = 0x80000000u;  // beyond every buffer range: reads as zero
constexpr int W_AUX = 2;               // non-temporal weight loads: each weight byte is read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

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

// Activations per thread while quantizing: the G / EPT lanes of a block then
// span 8 or 16 lanes, inside one DPP row.
template <int G>
constexpr int ept() { return G == 128 ? 8 : 4; }
constexpr int XPRE = 16;  // activations per thread loaded ahead of the weights

// Maximum / sum over aligned groups of L lanes (L = 8 or 16) by DPP: two quad
// permutes, a half-row mirror and, for 16, a row mirror. Every lane of the
// group receives the result.
template <int L>
__device__ __forceinline__ float group_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    if (L == 16)
        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    return v;
}
template <int L>
__device__ __forceinline__ int group_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    if (L == 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    return v;
}

// EPT consecutive activations of item u (elements EPT*u ...), float32 or
// bfloat16; an item beyond the row reads as zeros.
template <int EPT, bool XBF16>
__device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t r_x, int u, bool in, float (&v)[EPT]) {
    if (XBF16) {
        uint32_t p[EPT / 2];
        if (EPT == 4) {
            const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r_x, in ? 8u * u : OUT, 0, 0));
            p[0] = t.x; p[1] = t.y;
        } else {
            const uint4 t = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_x, in ? 16u * u : OUT, 0, 0));
            p[0] = t.x; p[1] = t.y; p[2 % (EPT / 2)] = t.z; p[3 % (EPT / 2)] = t.w;
        }
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            v[2 * i] = bf16_to_float(p[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_float(p[i] >> 16);
        }
    } else {
#pragma unroll
        for (int h = 0; h < EPT / 4; ++h) {
            const float4 t = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            r_x, in ? 4u * (EPT * u + 4 * h) : OUT, 0, 0));
            v[4 * h] = t.x; v[4 * h + 1] = t.y; v[4 * h + 2] = t.z; v[4 * h + 3] = t.w;
        }
    }
}

// Quantize item u: all lanes take part (the exchanges need every lane of a
// block); the stores are made only for items inside the row.
template <int G, int EPT>
__device__ __forceinline__ void quantize_item(int u, bool in, const float (&v)[EPT], bool out, int8_t* xq_l,
                                              float* xs_l, int32_t* xsum_l, int8_t* xq_out, float* xs_out,
                                              int32_t* xsum_out) {
    constexpr int L = G / EPT;  // lanes per block
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<L>(amax);
    const float s = amax / 127.0f;
    const float inv = act_inverse(s);
    uint32_t pk[EPT / 4];
    int sum = 0;
    // act_code for the EPT values: quotients by the reciprocal, then one branch
    // (rarely taken) to the exact quotients of values near a rounding tie
    float rq[EPT];
    bool near = inv == 0.0f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        rq[i] = v[i] * inv;
        near |= fabsf((rq[i] - floorf(rq[i])) - 0.5f) < 0x1p-12f;
    }
    if (near) {
#pragma unroll
        for (int i = 0; i < EPT; ++i)
            if (inv == 0.0f || fabsf((rq[i] - floorf(rq[i])) - 0.5f) < 0x1p-12f) rq[i] = v[i] / s;
    }
#pragma unroll
    for (int h = 0; h < EPT / 4; ++h) {
        pk[h] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = (amax != 0.0f) ? min(127, max(-127, (int)rintf(rq[4 * h + i]))) : 0;
            sum += c;
            pk[h] |= (uint32_t)(c & 0xFF) << (8 * i);
        }
    }
    sum = group_sum<L>(sum);
    if (in) {
        if (EPT == 4) {
            reinterpret_cast<uint32_t*>(xq_l)[u] = pk[0];
            if (out) reinterpret_cast<uint32_t*>(xq_out)[u] = pk[0];
        } else {
            reinterpret_cast<uint2*>(xq_l)[u] = make_uint2(pk[0], pk[(EPT / 4) - 1]);
            if (out) reinterpret_cast<uint2*>(xq_out)[u] = make_uint2(pk[0], pk[(EPT / 4) - 1]);
        }
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
}

// One pass of weight loads: lane l takes chunks c0 + l + 64 u of each of its
// R rows (16 bytes of codes each) and the raw 16-bit scale (and bias) of the
// chunk's block. Out-of-range chunks and rows read as zero.
template <int FMT, int G, int R, bool PARTIALS>
struct Pass {
    uint4 w[R][U];
    uint16_t s[R][U], b[R][U];  // raw fp16 / bf16 bits, converted where used

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r_w, __amdgpu_buffer_rsrc_t r_s,
                                         __amdgpu_buffer_rsrc_t r_b, int c0, int lane, int nchunks, int ngroups,
                                         uint32_t rowbytes) {
        constexpr int CPG = G / 32;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + lane + 64 * u;
                const bool in = c < nchunks;
                w[r][u] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(r_w, in ? r * rowbytes + 16u * c : OUT, 0, W_AUX));
                if (!PARTIALS) {
                    const uint32_t so = in ? 2u * (r * ngroups + c / CPG) : OUT;
                    s[r][u] = __builtin_amdgcn_raw_buffer_load_b16(r_s, so, 0, 0);
                    if (FMT == 1) b[r][u] = __builtin_amdgcn_raw_buffer_load_b16(r_b, so, 0, 0);
                }
            }
    }
};

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
    constexpr int NT = 64 * WAVES;
    constexpr int EPT = ept<G>();
    constexpr int NPRE = XPRE / EPT;  // items per thread loaded ahead
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    int8_t* xq_l = lds;                                           // K bytes
    float* xs_l = reinterpret_cast<float*>(lds + K);             // K/G floats
    int32_t* xsum_l = reinterpret_cast<int32_t*>(xs_l + K / G);  // K/G ints

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = (blockIdx.x * WAVES + wave) * R;
    const int nrows = max(0, min(R, N - row0));
    const int nchunks = K >> 5;
    const int ngroups = K / G;
    const uint32_t rowbytes = (uint32_t)(K >> 1);

    // the wave's own rows: a range of nrows rows, so that rows past N read zero
    const __amdgpu_buffer_rsrc_t r_w = rsrc(wq + (size_t)row0 * rowbytes, nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t r_s = rsrc(wscale + (size_t)row0 * ngroups, PARTIALS ? 0u : nrows * ngroups * 2u);
    const __amdgpu_buffer_rsrc_t r_b =
        rsrc(wbias + (size_t)row0 * ngroups, (PARTIALS || FMT == 0) ? 0u : nrows * ngroups * 2u);

    // fused: the activations go out first, so that their quantization below
    // overlaps the weight stream
    const int nitems = K / EPT;
    float xv[NPRE][EPT];
    const __amdgpu_buffer_rsrc_t r_x = rsrc(x, FUSED ? (uint32_t)K * (XBF16 ? 2u : 4u) : 0u);
    if (FUSED) {
#pragma unroll
        for (int i = 0; i < NPRE; ++i) {
            const int u = tid + i * NT;
            if (i * NT < nitems) load_x<EPT, XBF16>(r_x, u, u < nitems, xv[i]);
        }
    }

    Pass<FMT, G, R, PARTIALS> cur;
    cur.load(r_w, r_s, r_b, 0, lane, nchunks, ngroups, rowbytes);

    if (LDS_ACT) {
        if (FUSED) {
            const bool out = xq_out != nullptr && blockIdx.x == 0;
#pragma unroll
            for (int i = 0; i < NPRE; ++i) {
                const int u = tid + i * NT;
                if (i * NT + wave * 64 < nitems)
                    quantize_item<G, EPT>(u, u < nitems, xv[i], out, xq_l, xs_l, xsum_l, xq_out, xs_out, xsum_out);
            }
            for (int ub = NPRE * NT + wave * 64; ub < nitems; ub += NT) {
                const int u = ub + lane;
                float v[EPT];
                load_x<EPT, XBF16>(r_x, u, u < nitems, v);
                quantize_item<G, EPT>(u, u < nitems, v, out, xq_l, xs_l, xsum_l, xq_out, xs_out, xsum_out);
            }
        } else {
            for (int u = tid; u < (K >> 4); u += NT)
                reinterpret_cast<uint4*>(xq_l)[u] = reinterpret_cast<const uint4*>(xq)[u];
            for (int g = tid; g < ngroups; g += NT) {
                if (xs) xs_l[g] = xs[g];
                xsum_l[g] = xsum[g];
            }
        }
        __syncthreads();
    }

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    for (int c0 = 0; c0 < nchunks; c0 += 64 * U) {
        Pass<FMT, G, R, PARTIALS> nxt;
        if (c0 + 64 * U < nchunks) nxt.load(r_w, r_s, r_b, c0 + 64 * U, lane, nchunks, ngroups, rowbytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
            const int cc = min(c, nchunks - 1);  // a chunk past the row has zero codes and scales
            const int gi = cc / CPG;
            uint4 xa, xb;
            float a = 0.0f;
            int s;
            if (LDS_ACT) {
                xa = *reinterpret_cast<const uint4*>(xq_l + 32 * cc);
                xb = *reinterpret_cast<const uint4*>(xq_l + 32 * cc + 16);
                if (!PARTIALS) a = xs_l[gi];
                s = xsum_l[gi];
            } else {
                xa = *reinterpret_cast<const uint4*>(xq + 32 * cc);
                xb = *reinterpret_cast<const uint4*>(xq + 32 * cc + 16);
                if (!PARTIALS) a = xs[gi];
                s = xsum[gi];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int dot = dot_chunk(cur.w[r][u], xa, xb);
                if (PARTIALS) {
                    int p = dot;
                    if (FMT == 0) {
                        p = dot - 8 * s;
                    } else {
#pragma unroll
                        for (int off = 1; off < CPG; off <<= 1) p += __shfl_xor(p, off, 64);
                    }
                    if (c < nchunks && r < nrows && (c % CPG) == 0)
                        partials[(size_t)(row0 + r) * ngroups + c / CPG] = p;
                } else if (FMT == 0) {
                    const int p = dot - 8 * s;  // sum (q - 8) * xq over the block
                    acc[r] += (half_to_float(cur.s[r][u]) * a) * (float)p;
                } else {
                    acc[r] += a * (bf16_to_float(cur.s[r][u]) * (float)dot);
                    const float bt = a * (bf16_to_float(cur.b[r][u]) * (float)s);  // bias * dequantized sum x
                    acc[r] += ((c % CPG) == 0) ? bt : 0.0f;
                }
            }
        }
        cur = nxt;
    }
    if (!PARTIALS) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float t = wave_sum(acc[r]);
            if (lane == 0 && r < nrows) y[row0 + r] = t;
        }
    }
}

// Few-row variant (1 or 2 activation rows, 4-bit codes): the GEMV's
// weight stream and chunk mapping, with each pass's activation codes and
// scales of all MR rows loaded into registers, so every unpacked weight chunk
// feeds MR integer dots. A wavefront owns R consecutive weight rows.
template <int FMT, int G, int MR, int R, bool PARTIALS>
__global__ __launch_bounds__(256) void gemv_rows_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                        const uint16_t* __restrict__ wscale,
                                                        const uint16_t* __restrict__ wbias,
                                                        const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                        const int32_t* __restrict__ xsum, float* __restrict__ y,
                                                        int32_t* __restrict__ partials) {
    constexpr int CPG = G / 32;  // chunks per block / group
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * 4 + wave) * R;
    const int nrows = max(0, min(R, N - row0));
    if (nrows == 0) return;
    const int nchunks = K >> 5;
    const int ngroups = K / G;
    const uint32_t rowbytes = (uint32_t)(K >> 1);

    const __amdgpu_buffer_rsrc_t r_w = rsrc(wq + (size_t)row0 * rowbytes, nrows * rowbytes);
    const __amdgpu_buffer_rsrc_t r_s = rsrc(wscale + (size_t)row0 * ngroups, PARTIALS ? 0u : nrows * ngroups * 2u);
    const __amdgpu_buffer_rsrc_t r_b =
        rsrc(wbias + (size_t)row0 * ngroups, (PARTIALS || FMT == 0) ? 0u : nrows * ngroups * 2u);
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)M * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t r_xs = rsrc(xs, PARTIALS ? 0u : (uint32_t)M * ngroups * 4u);
    const __amdgpu_buffer_rsrc_t r_xsum = rsrc(xsum, (uint32_t)M * ngroups * 4u);

    float acc[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = 0.0f;

    Pass<FMT, G, R, PARTIALS> cur;
    cur.load(r_w, r_s, r_b, 0, lane, nchunks, ngroups, rowbytes);
    for (int c0 = 0; c0 < nchunks; c0 += 64 * U) {
        // this pass's activation codes, scales and code sums; rows past M and
        // chunks past K read zero
        uint4 xa[MR][U], xb[MR][U];
        float a[MR][U];
        int sx[MR][U];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + lane + 64 * u;
                const bool in = c < nchunks && m < M;
                const uint32_t o = in ? (uint32_t)m * (uint32_t)K + 32u * c : OUT;
                xa[m][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, o, 0, 0));
                xb[m][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, in ? o + 16 : OUT, 0, 0));
                const uint32_t og = in ? 4u * (uint32_t)(m * ngroups + c / CPG) : OUT;
                a[m][u] = PARTIALS ? 0.0f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_xs, og, 0, 0));
                sx[m][u] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_xsum, og, 0, 0);
            }
        Pass<FMT, G, R, PARTIALS> nxt;
        if (c0 + 64 * U < nchunks) nxt.load(r_w, r_s, r_b, c0 + 64 * U, lane, nchunks, ngroups, rowbytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + lane + 64 * u;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint4 w = cur.w[r][u];
                const uint32_t lo[4] = {lo_nibbles(w.x), lo_nibbles(w.y), lo_nibbles(w.z), lo_nibbles(w.w)};
                const uint32_t hi[4] = {hi_nibbles(w.x), hi_nibbles(w.y), hi_nibbles(w.z), hi_nibbles(w.w)};
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    int dot = 0;
                    dot = __builtin_amdgcn_sdot4((int)lo[0], (int)xa[m][u].x, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)lo[1], (int)xa[m][u].y, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)lo[2], (int)xa[m][u].z, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)lo[3], (int)xa[m][u].w, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)hi[0], (int)xb[m][u].x, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)hi[1], (int)xb[m][u].y, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)hi[2], (int)xb[m][u].z, dot, false);
                    dot = __builtin_amdgcn_sdot4((int)hi[3], (int)xb[m][u].w, dot, false);
                    if (PARTIALS) {
                        int p = dot;
                        if (FMT == 0) {
                            p = dot - 8 * sx[m][u];
                        } else {
#pragma unroll
                            for (int off = 1; off < CPG; off <<= 1) p += __shfl_xor(p, off, 64);
                        }
                        if (c < nchunks && r < nrows && m < M && (c % CPG) == 0)
                            partials[((size_t)m * N + row0 + r) * ngroups + c / CPG] = p;
                    } else if (FMT == 0) {
                        const int p = dot - 8 * sx[m][u];  // sum (q - 8) * xq over the block
                        acc[r][m] += (half_to_float(cur.s[r][u]) * a[m][u]) * (float)p;
                    } else {
                        acc[r][m] += a[m][u] * (bf16_to_float(cur.s[r][u]) * (float)dot);
                        const float bt = a[m][u] * (bf16_to_float(cur.b[r][u]) * (float)sx[m][u]);
                        acc[r][m] += ((c % CPG) == 0) ? bt : 0.0f;
                    }
                }
            }
        }
        cur = nxt;
    }
    if (!PARTIALS) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float t = wave_sum(acc[r][m]);
                if (lane == 0 && r < nrows && m < M) y[(size_t)m * N + row0 + r] = t;
            }
    }
}

// Launch shapes. Plain GEMV (codes given): one row per wavefront, 8 wavefronts
// per workgroup, codes read from global memory. Fused: one row per wavefront,
// 16 wavefronts per workgroup sharing the quantization of x into LDS. The
// partials views run these same shapes with the partials store switched on.
constexpr int PLAIN_WAVES = 8;
constexpr int FUSED_WAVES = 16;

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

template <int FMT, int G>
hipError_t launch_fmt(int K, int N, const uint8_t* wq, const void* wscale, const void* wbias, const int8_t* xq,
                      const float* xs, const int32_t* xsum, float* y, int32_t* partials, hipStream_t stream) {
    if (partials)
        return launch_one<FMT, G, 1, PLAIN_WAVES, false, false, false, true>(K, N, wq, wscale, wbias, nullptr, xq, xs,
                                                                            xsum, y, partials, nullptr, nullptr,
                                                                            nullptr, stream);
    return launch_one<FMT, G, 1, PLAIN_WAVES, false, false, false, false>(K, N, wq, wscale, wbias, nullptr, xq, xs,
                                                                         xsum, y, nullptr, nullptr, nullptr, nullptr,
                                                                         stream);
}

template <int FMT, int G, bool PARTIALS>
hipError_t launch_fused_fmt(int K, int N, bool xbf16, const void* x, const uint8_t* wq, const void* wscale,
                            const void* wbias, float* y, int32_t* partials, int8_t* xq_out, float* xs_out,
                            int32_t* xsum_out, hipStream_t stream) {
    if (xbf16)
        return launch_one<FMT, G, 1, FUSED_WAVES, true, true, true, PARTIALS>(
            K, N, wq, wscale, wbias, x, nullptr, nullptr, nullptr, y, partials, xq_out, xs_out, xsum_out, stream);
    return launch_one<FMT, G, 1, FUSED_WAVES, true, true, false, PARTIALS>(
        K, N, wq, wscale, wbias, x, nullptr, nullptr, nullptr, y, partials, xq_out, xs_out, xsum_out, stream);
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
        return launch_fused_fmt<0, 32, false>(K, N, xbf16, x, wq, wscale, wbias, y, nullptr, xq_out, xs_out,
                                              xsum_out, stream);
    if (bs == 64)
        return launch_fused_fmt<1, 64, false>(K, N, xbf16, x, wq, wscale, wbias, y, nullptr, xq_out, xs_out,
                                              xsum_out, stream);
    if (bs == 128)
        return launch_fused_fmt<1, 128, false>(K, N, xbf16, x, wq, wscale, wbias, y, nullptr, xq_out, xs_out,
                                               xsum_out, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemv_fused_partials(int K, int N, int bs, int fmt, bool xbf16, const void* x, const uint8_t* wq,
                                      int32_t* partials, hipStream_t stream) {
    if (fmt == 0)
        return launch_fused_fmt<0, 32, true>(K, N, xbf16, x, wq, nullptr, nullptr, nullptr, partials, nullptr,
                                             nullptr, nullptr, stream);
    if (bs == 64)
        return launch_fused_fmt<1, 64, true>(K, N, xbf16, x, wq, nullptr, nullptr, nullptr, partials, nullptr,
                                             nullptr, nullptr, stream);
    if (bs == 128)
        return launch_fused_fmt<1, 128, true>(K, N, xbf16, x, wq, nullptr, nullptr, nullptr, partials, nullptr,
                                              nullptr, nullptr, stream);
    return hipErrorInvalidValue;
}

namespace {

template <int FMT, int G, int MR, bool PARTIALS>
hipError_t launch_rows_mr(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                          const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                          hipStream_t stream) {
    constexpr int R = 2;  // weight rows per wavefront (4 was slower)
    const dim3 grid((unsigned)((N + 4 * R - 1) / (4 * R))), block(256);
    hipLaunchKernelGGL((gemv_rows_kernel<FMT, G, MR, R, PARTIALS>), grid, block, 0, stream, M, K, N, wq,
                       static_cast<const uint16_t*>(wscale), static_cast<const uint16_t*>(wbias), xq, xs, xsum, y,
                       partials);
    return hipGetLastError();
}

template <int FMT, int G, bool PARTIALS>
hipError_t launch_rows_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                           const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                           hipStream_t stream) {
    if (M == 1)
        return launch_rows_mr<FMT, G, 1, PARTIALS>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return launch_rows_mr<FMT, G, 2, PARTIALS>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
}


template <int FMT, int G>
hipError_t launch_rows_p(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                         const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                         hipStream_t stream) {
    if (partials)
        return launch_rows_fmt<FMT, G, true>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return launch_rows_fmt<FMT, G, false>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
}

}  // namespace

bool gemv_rows_fits(int M, int K, int bits) { return bits == 4 && M >= 1 && M <= GEMV_ROWS_MAX_M && K >= 32; }

hipError_t launch_gemv_rows(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                            const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                            int32_t* partials, hipStream_t stream) {
    if (M < 1 || M > GEMV_ROWS_MAX_M) return hipErrorInvalidValue;
    if (fmt == 0) return launch_rows_p<0, 32>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 64) return launch_rows_p<1, 64>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_rows_p<1, 128>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
