// W4A8 GEMM for a few activation rows (M <= 64): the regime between the
// decode GEMV (M = 1) and the tiled prefill GEMM. q4_gemm takes it up to 32
// rows, and for 33..64 rows when N <= 8192 (each workgroup reads all M x K
// activation codes, so wider products go to the tiled kernel).
//
// tract PR #2432 (follow-up decode measurements): the weights dominate the
// traffic of a decode-sized product, so they must be streamed once.
// MLX PR #4802: below M = 32 its int8 path is not taken and x is dequantized
// instead; here the int8 path covers every M.
//
// One or two rows with 4-bit codes go to the GEMV-shaped kernel in gemv.hip
// (activation codes of all rows in registers, 8 v_dot4 per row and block),
// and 3 to 32 rows with 4-bit codes to the weight-streaming matrix-core kernel
// in rows_mfma.hip, which are faster there; the kernel below covers 6- and
// 8-bit codes and 33 to 64 rows.
//
// A workgroup owns 16 output columns and all M rows, so every weight block is
// read once for all rows. K is walked in chunks (2048, 1024 or 512 wide, see
// chunk_k): the workgroup copies the chunk's packed codes (16 rows), activation
// codes (M rows) and activation scales into LDS with coalesced 128-bit loads
// (the next chunk's loads are in flight while this one is computed), then its
// 8 wavefronts split the chunk's K steps; each runs v_mfma_i32_16x16x32_i8
// (16 rows x 16 columns x one 32-weight block) per step, with one, two or
// four 16-row tiles. The wavefronts' float partial sums are added in LDS in a
// fixed order (no atomics, so results do not depend on scheduling).
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
// The activation scales (and xs * xsum) of a chunk are staged with its codes.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int SW = 8;          // wavefronts per workgroup
constexpr int SNT = 64 * SW;   // threads per workgroup
constexpr int SN = 16;         // output columns per workgroup
// K per chunk staged in LDS: 2048 with one 16-row tile, 1024 with two, 512
// with four (1024 for 128-weight groups: a wavefront's share of a chunk holds
// whole groups). The activation codes of a chunk and two chunks of loads in
// flight then stay within the register and LDS budget.
template <int MT, int G>
constexpr int chunk_k() { return MT == 1 ? 2048 : (MT == 2 || G == 128) ? 1024 : 512; }
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data format
constexpr uint32_t OUT = 0x80000000u;   // beyond every buffer range: reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

// Code bytes per weight row and chunk: the main part (nibbles, or bytes for
// 8-bit codes) and, for 6-bit codes, the high 2-bit plane after it.
template <int MT, int G, int BITS>
constexpr int main_bytes() { return BITS == 8 ? chunk_k<MT, G>() : chunk_k<MT, G>() / 2; }
template <int MT, int G, int BITS>
constexpr int plane_bytes() { return BITS == 6 ? chunk_k<MT, G>() / 4 : 0; }

template <int G, int MT, int BITS>
struct SmallLds {
    static constexpr int KC = chunk_k<MT, G>();
    static constexpr int GPC = KC / G;  // groups per chunk
    uint8_t w[SN][main_bytes<MT, G, BITS>() + plane_bytes<MT, G, BITS>() + 16];  // codes (16 bytes of padding per row)
    uint8_t a[16 * MT][KC + 16];        // activation codes of the chunk
    float xs[GPC][16 * MT];             // activation scales, group-major
    float xb[GPC][16 * MT];             // xs * xsum (affine)
    float red[SW][MT][256];             // per-wavefront partial sums
};

// BITS: affine code width, 4, 6 or 8 (layouts as in the tiled GEMM); 8-bit
// codes enter the MFMA as q - 128 with 128 * s added to the group's bias.
template <int FMT, int G, int MT, bool PARTIALS, int BITS>
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
    using L = SmallLds<G, MT, BITS>;
    constexpr int MB = main_bytes<MT, G, BITS>(), PB = plane_bytes<MT, G, BITS>();
    constexpr int KC = L::KC;
    constexpr int GPC = L::GPC;
    constexpr int SPW = KC / 32 / SW;  // MFMA steps per wavefront per chunk
    static_assert(SPW % SPG == 0, "a wavefront's share of a chunk holds whole groups");
    static_assert((16 * MT * KC / 16) % SNT == 0, "activation staging covers the chunk exactly");
    constexpr int W_CH = (SN * MB / 16 + SNT - 1) / SNT;  // 16-byte code loads per thread per chunk (rounded up)
    constexpr int P_CH = (SN * PB / 16 + SNT - 1) / SNT;  // 16-byte high-plane loads (6 bits)
    constexpr int CPS = BITS == 8 ? 16 : 32;           // codes per 16 bytes of the main part
    constexpr int A_CH = MR * KC / 16 / SNT;           // 16-byte activation loads per thread per chunk (4 / 8)
    constexpr int S_CH = (MR * GPC + SNT - 1) / SNT;   // scale values per thread per chunk
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    L& S = *reinterpret_cast<L*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * SN;
    const int ngroups = K / G;
    const int nchunks = (K + KC - 1) / KC;

    const __amdgpu_buffer_rsrc_t r_b = rsrc(wq, (uint32_t)((size_t)N * K * BITS / 8));
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)((size_t)M * K));
    const __amdgpu_buffer_rsrc_t r_xs = rsrc(xs, PARTIALS ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_xsum = rsrc(xsum, (PARTIALS || !AFF) ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, PARTIALS ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    const __amdgpu_buffer_rsrc_t r_wb =
        rsrc(wbias, (PARTIALS || !AFF) ? 0u : (uint32_t)((size_t)N * ngroups * 2));

    // Chunk staging, coalesced: consecutive threads read consecutive 16 bytes of
    // one weight row (KC/2 bytes per row) or one activation row (KC bytes). Two
    // register sets: the loads of chunks ch + 1 and ch + 2 are in flight while
    // chunk ch is computed. Each lane also fetches the weight scales (and
    // biases) of its column for the groups its wavefront will rescale.
    constexpr int GPW = SPW / SPG;  // groups per wavefront per chunk
    const uint32_t os = (n0 + c < N) ? (uint32_t)((n0 + c) * ngroups * 2) : OUT;  // this lane's weight-scale row
    uint4 rw[2][W_CH], rpl[2][P_CH > 0 ? P_CH : 1], ra[2][A_CH];
    float rxs[2][S_CH], rxb[2][S_CH];
    uint32_t rws[2][GPW], rwb[2][GPW];
    auto load_chunk = [&](int ch, auto setc) {
        constexpr int B = decltype(setc)::value;
        const int k0 = ch * KC;
#pragma unroll
        for (int i = 0; i < W_CH; ++i) {
            const int idx = tid + SNT * i, r = idx / (MB / 16), seg = idx % (MB / 16);  // 16-byte segment
            const bool in = idx < SN * MB / 16 && n0 + r < N && k0 + CPS * seg < K;
            const uint32_t rowb = BITS == 8 ? (uint32_t)K : (uint32_t)(K / 2);
            rw[B][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                r_b, in ? (uint32_t)((n0 + r) * rowb + 16 * seg) : OUT, BITS == 8 ? k0 : k0 / 2, 0));
        }
#pragma unroll
        for (int i = 0; i < P_CH; ++i) {  // 16 bytes of the high plane hold 64 codes
            const int idx = tid + SNT * i, r = idx / (PB / 16), seg = idx % (PB / 16);
            const bool in = idx < SN * PB / 16 && n0 + r < N && k0 + 64 * seg < K;
            const uint32_t o = (uint32_t)((size_t)N * (K / 2) + (size_t)(n0 + r) * (K / 4) + 16 * seg);
            rpl[B][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_b, in ? o : OUT, k0 / 4, 0));
        }
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int idx = tid + SNT * i, r = idx / (KC / 16), seg = idx % (KC / 16);
            const bool in = r < M && k0 + 16 * seg < K;
            ra[B][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                r_a, in ? (uint32_t)(r * K + 16 * seg) : OUT, k0, 0));
        }
        if (!PARTIALS) {
            const int g0 = k0 / G;
#pragma unroll
            for (int i = 0; i < S_CH; ++i) {
                const int idx = tid + SNT * i, r = idx / GPC, gi = idx % GPC;
                const bool in = idx < MR * GPC && r < M && g0 + gi < ngroups;
                const uint32_t o = in ? (uint32_t)((r * ngroups + gi) * 4) : OUT;
                rxs[B][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_xs, o, g0 * 4, 0));
                rxb[B][i] = AFF ? (float)(int)__builtin_amdgcn_raw_buffer_load_b32(r_xsum, o, g0 * 4, 0) : 0.0f;
            }
            const int gw0 = ch * GPC + wave * GPW;
#pragma unroll
            for (int u = 0; u < GPW; ++u) {
                // The group depends on the wavefront index, which the compiler does not
                // know to be uniform, so as a scalar offset it is looped over lane by
                // lane. Affine takes it as a per-lane offset (g128 16x4096x4096: 7.6 ->
                // 7.0 us); Q4_0 keeps the scalar offset, with which it measured 5-9%
                // faster (8.5 against 9.2 us at 16x4096x4096).
                if (AFF) {
                    const uint32_t o = (gw0 + u < ngroups && os != OUT) ? os + (uint32_t)(gw0 + u) * 2u : OUT;
                    rws[B][u] = __builtin_amdgcn_raw_buffer_load_b16(r_ws, o, 0, 0);
                    rwb[B][u] = __builtin_amdgcn_raw_buffer_load_b16(r_wb, o, 0, 0);
                } else {
                    const uint32_t o = (gw0 + u < ngroups) ? os : OUT;
                    rws[B][u] = __builtin_amdgcn_raw_buffer_load_b16(r_ws, o, (gw0 + u) * 2, 0);
                    rwb[B][u] = 0u;
                }
            }
        }
    };
    auto store_chunk = [&](auto setc) {
        constexpr int B = decltype(setc)::value;
#pragma unroll
        for (int i = 0; i < W_CH; ++i) {
            const int idx = tid + SNT * i, r = idx / (MB / 16), seg = idx % (MB / 16);
            if (idx < SN * MB / 16) *reinterpret_cast<uint4*>(&S.w[r][16 * seg]) = rw[B][i];
        }
#pragma unroll
        for (int i = 0; i < P_CH; ++i) {
            const int idx = tid + SNT * i, r = idx / (PB / 16), seg = idx % (PB / 16);
            if (idx < SN * PB / 16) *reinterpret_cast<uint4*>(&S.w[r][MB + 16 * seg]) = rpl[B][i];
        }
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int idx = tid + SNT * i, r = idx / (KC / 16), seg = idx % (KC / 16);
            *reinterpret_cast<uint4*>(&S.a[r][16 * seg]) = ra[B][i];
        }
        if (!PARTIALS) {
#pragma unroll
            for (int i = 0; i < S_CH; ++i) {
                const int idx = tid + SNT * i, r = idx / GPC, gi = idx % GPC;
                if (idx < MR * GPC) {
                    S.xs[gi][r] = rxs[B][i];
                    if (AFF) S.xb[gi][r] = rxs[B][i] * rxb[B][i];
                }
            }
        }
    };

    const int shift = 4 * (q >> 1);

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    // One chunk: stage it from register set B, refill B with chunk ch + 2, compute.
    auto do_chunk = [&](int ch, auto setc) {
        constexpr int B = decltype(setc)::value;
        __syncthreads();  // the previous chunk is consumed
        store_chunk(setc);
        uint32_t wsb[GPW], wbb[GPW];
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            wsb[u] = rws[B][u];
            wbb[u] = rwb[B][u];
        }
        __syncthreads();
        if (ch + 2 < nchunks) load_chunk(ch + 2, setc);
        const int gw0 = ch * GPC + wave * GPW;  // first group of this wavefront
#pragma unroll
        for (int u = 0; u < GPW; ++u) {
            const int g = gw0 + u;
            v4i P[MT];
#pragma unroll
            for (int e = 0; e < SPG; ++e) {
                const int sl = wave * SPW + u * SPG + e;  // step within the chunk
                uint32_t lo, hi;
                if (BITS == 8) {  // this lane's 8 codes are bytes 8q .. 8q+7 of the step: q - 128
                    const uint2 wv = *reinterpret_cast<const uint2*>(&S.w[c][32 * sl + 8 * q]);
                    lo = wv.x ^ 0x80808080u;
                    hi = wv.y ^ 0x80808080u;
                } else {
                    const uint2 wv = *reinterpret_cast<const uint2*>(&S.w[c][16 * sl + 8 * (q & 1)]);
                    lo = (wv.x >> shift) & 0x0F0F0F0Fu;
                    hi = (wv.y >> shift) & 0x0F0F0F0Fu;
                    if (FMT == 0) {
                        lo = minus8_bytes(lo);
                        hi = minus8_bytes(hi);
                    }
                    if (BITS == 6) {  // word q / 2 of the step's plane; codes 8(q&1) .. +7 take bit pairs 2(q&1), +1
                        const uint32_t pw = *reinterpret_cast<const uint32_t*>(&S.w[c][MB + 8 * sl + 4 * (q >> 1)]);
                        lo |= two_bits_high(pw, 2 * (q & 1));
                        hi |= two_bits_high(pw, 2 * (q & 1) + 1);
                    }
                }
                const long bop = (long)(((uint64_t)hi << 32) | lo);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const uint2 av = *reinterpret_cast<const uint2*>(&S.a[16 * t + c][32 * sl + 8 * q]);
                    const long aop = (long)(((uint64_t)av.y << 32) | av.x);
                    const v4i z = {0, 0, 0, 0};
                    P[t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, e == 0 ? z : P[t], 0, 0, 0);
                }
            }
            if (PARTIALS) {
                const int n = n0 + c;
                if (g < ngroups && n < N) {
#pragma unroll
                    for (int t = 0; t < MT; ++t)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = 16 * t + 4 * q + r;
                            // 8 bits: the MFMA summed (q - 128) * xq; the reported partial is sum q * xq
                            if (m < M)
                                partials[((size_t)m * N + n) * ngroups + g] =
                                    P[t][r] + (BITS == 8 ? 128 * xsum[(size_t)m * ngroups + g] : 0);
                        }
                }
                continue;
            }
            // groups past K have zero codes and zero scales and biases
            const int gi = wave * GPW + u;  // group within the chunk
            const float w = AFF ? bf16_to_float(wsb[u]) : half_to_float(wsb[u]);
            const float b = AFF ? bf16_to_float(wbb[u]) + (BITS == 8 ? 128.0f * w : 0.0f) : 0.0f;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float4 xv = *reinterpret_cast<const float4*>(&S.xs[gi][16 * t + 4 * q]);
                acc[t][0] += xv.x * (w * (float)P[t][0]);
                acc[t][1] += xv.y * (w * (float)P[t][1]);
                acc[t][2] += xv.z * (w * (float)P[t][2]);
                acc[t][3] += xv.w * (w * (float)P[t][3]);
                if (AFF) {
                    const float4 bv = *reinterpret_cast<const float4*>(&S.xb[gi][16 * t + 4 * q]);
                    acc[t][0] += bv.x * b;
                    acc[t][1] += bv.y * b;
                    acc[t][2] += bv.z * b;
                    acc[t][3] += bv.w * b;
                }
            }
        }
    };

    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    load_chunk(0, C0());
    if (nchunks > 1) load_chunk(1, C1());
    int ch = 0;
    for (; ch + 1 < nchunks; ch += 2) {
        do_chunk(ch, C0());
        do_chunk(ch + 1, C1());
    }
    if (ch < nchunks) do_chunk(ch, C0());
    if (PARTIALS) return;

    // combine the wavefronts' partial sums in wavefront order
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) S.red[wave][t][(4 * q + r) * 16 + c] = acc[t][r];
    __syncthreads();
    for (int o = tid; o < MT * 256; o += SNT) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < SW; ++w) s += S.red[w][o >> 8][o & 255];
        const int m = 16 * (o >> 8) + ((o >> 4) & 15), nn = n0 + (o & 15);
        if (m < M && nn < N) y[(size_t)m * N + nn] = s;
    }
}

template <int FMT, int G, int MT, int BITS>
hipError_t launch_mt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                     const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                     hipStream_t stream) {
    const size_t lds = sizeof(SmallLds<G, MT, BITS>);
    auto k = partials ? gemm_small_kernel<FMT, G, MT, true, BITS> : gemm_small_kernel<FMT, G, MT, false, BITS>;
    if (lds > 64 * 1024) {
        const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(k), lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, dim3((N + SN - 1) / SN), dim3(SNT), lds, stream, M, K, N, wq,
                       static_cast<const uint16_t*>(wscale), static_cast<const uint16_t*>(wbias), xq, xs, xsum, y,
                       partials);
    return hipGetLastError();
}

template <int FMT, int G, int BITS = 4>
hipError_t launch_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    if (M <= 16) return launch_mt<FMT, G, 1, BITS>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (M <= 32) return launch_mt<FMT, G, 2, BITS>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return launch_mt<FMT, G, 4, BITS>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
}

template <int G>
hipError_t launch_affine_bits(int bits, int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                              const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                              hipStream_t stream) {
    if (bits == 4) return launch_fmt<1, G, 4>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bits == 6) return launch_fmt<1, G, 6>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bits == 8) return launch_fmt<1, G, 8>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_small(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                             const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                             int32_t* partials, hipStream_t stream) {
    if (M < 1 || M > GEMM_SMALL_MAX_M) return hipErrorInvalidValue;
    if (gemv_rows_fits(M, K, bits))  // 1 or 2 rows of 4-bit codes: the GEMV-shaped kernel (gemv.hip)
        return launch_gemv_rows(M, K, N, bs, fmt, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (rows_mfma_fits(M, K, fmt == 0 ? 32 : bs, fmt, bits))  // up to 32 rows of 4-bit codes (rows_mfma.hip)
        return launch_rows_mfma(M, K, N, bs, fmt, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (fmt == 0) {
        if (bits != 4) return hipErrorInvalidValue;
        return launch_fmt<0, 32>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    }
    if (bs == 64) return launch_affine_bits<64>(bits, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_affine_bits<128>(bits, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
