// W4A8 prefill GEMM on the gfx950 int8 matrix cores.
//
// tract PR #2432 ("The kernel"): the integer dot of every 32-weight block is
// exact and each block's integer is rescaled in float before accumulation.
// MLX PR #4802: with affine weights the int8 x int8 MMA runs on the original
// codes and the per-group scale and bias are applied inside the kernel.
//
// Tiling: a workgroup of 2 x 2 wavefronts computes a 128 x 128 tile of Y; each
// wavefront owns 2 x 2 tiles of v_mfma_i32_32x32x32_i8 (32 x 32 outputs; one
// 32-wide K step is one Q4_0 block). Two workgroups share a CU (registers are
// held under 256 per lane and LDS under 80 KB per workgroup); they are not
// synchronised with each other, so one's matrix work overlaps the other's
// float rescale on every SIMD.
//
// K is walked in 128-wide stages through two LDS buffers. The stage's global
// loads are buffer loads with a per-lane offset fixed for the whole kernel
// and the stage offset in a scalar register; rows past M or N read as zero
// (the buffer range check), so the staging needs no masks. After the one
// barrier of a stage, the registers holding stage s+1 are written to the free
// buffer (weight nibbles unpacked on the way: q - 8 as signed bytes for Q4_0,
// q for affine), the loads of stage s+2 are issued, and stage s is computed.
// LDS rows are 128 bytes with the 16-byte chunk index XORed with bits of the
// row index, so the MFMA fragment reads (32 rows at one K offset) hit all banks.
//
// Per block (Q4_0) or group (affine, 64 / 128 weights = 2 / 4 MFMA steps) the
// int32 tile is rescaled into float accumulators:
//   Q4_0:   acc += xs[m] * (d[n] * P)                 3 VALU ops per output
//   affine: acc += xs[m] * (s[n] * A)                 3 VALU ops per output
//           acc += sum_g (xs * xsum)[m, g] * b[n, g]  on the f32 matrix core
// The affine bias term is a rank-(K/g) product, so it runs as
// v_mfma_f32_32x32x2_f32 with two groups in its two K slots instead of a
// fourth VALU op per output.
//
// Workgroups are mapped to tiles so that the workgroups resident on one XCD
// (dispatch is round-robin over the 8 XCDs) take neighbouring tiles, grouped
// GROUP_M row tiles at a time, which keeps their shared A and B panels in
// that XCD's L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q4 {

namespace {

constexpr int BM = 128, BN = 128;    // workgroup tile
constexpr int KS = 128;              // K per stage
constexpr int NT = 256;              // threads per workgroup
constexpr int GROUP_M = 8;           // row tiles per tile group
constexpr int NXCD = 8;
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data format

template <int G, int FMT>
struct Stage {
    static constexpr int GPS = KS / G;
    static constexpr int NB = (FMT == 1) ? GPS : 1;  // affine keeps the bias operands too
    uint4 a[BM * KS / 16];
    uint4 b[BN * KS / 16];
    float xs[GPS][BM];
    float ws[GPS][BN];
    float xb[NB][BM];
    float wb[NB][BN];
};

// 16-byte chunk c (0..7) of LDS row r. The chunk index is XORed with
// (r & 7) ^ ((r >> 3) & 1): any 8 consecutive aligned rows use 8 different
// chunk positions, and any 16 consecutive aligned rows use 16 different
// 16-byte slots of a 256-byte bank line (even and odd rows fill its two
// halves), so a 32-row fragment read at one K offset is conflict-free whether
// the banks serve 8 or 16 lanes of a 128-bit read per cycle.
__device__ __forceinline__ int swz(int r, int c) { return r * (KS / 16) + (c ^ (r & 7) ^ ((r >> 3) & 1)); }

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    // consecutive workgroup ids go to different XCDs: give each XCD a contiguous range of tiles
    int t = bid;
    if (total % NXCD == 0) t = (bid % NXCD) * (total / NXCD) + bid / NXCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = t / per_group;
    const int first_m = group * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int r = t - group * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

template <int FMT, int G, bool PARTIALS>
__global__ __launch_bounds__(NT, 2) void gemm_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wscale,
                                                      const uint16_t* __restrict__ wbias,
                                                      const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int32_t* __restrict__ xsum, float* __restrict__ y,
                                                      int32_t* __restrict__ partials) {
    constexpr int GPS = KS / G;  // blocks or groups per stage
    constexpr int SPG = G / 32;  // MFMA K steps per block or group
    constexpr int A_CH = BM * (KS / 16) / NT;  // 16-byte activation chunks per thread per stage (4)
    constexpr int B_CH = BN * (KS / 32) / NT;  // 16-byte packed weight chunks per thread per stage (2)
    constexpr bool AFF = FMT == 1;
    constexpr bool BIAS_MFMA = AFF && !PARTIALS;
    static_assert(A_CH * NT == BM * (KS / 16) && B_CH * NT == BN * (KS / 32), "tile / thread mismatch");

    using St = Stage<G, FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    St* stage_buf = reinterpret_cast<St*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int ngroups = K / G;
    const int nstages = (K + KS - 1) / KS;
    const int half = lane >> 5, l32 = lane & 31;

    // ---------------------------------------------------------------- staging
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)((size_t)M * K));
    const __amdgpu_buffer_rsrc_t r_b = rsrc(wq, (uint32_t)((size_t)N * (K / 2)));
    const __amdgpu_buffer_rsrc_t r_xs = rsrc(xs, PARTIALS ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_xsum = rsrc(xsum, PARTIALS ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, PARTIALS ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    const __amdgpu_buffer_rsrc_t r_wb =
        rsrc(wbias, (PARTIALS || !AFF) ? 0u : (uint32_t)((size_t)N * ngroups * 2));
    constexpr uint32_t OUT = 0x80000000u;  // beyond every buffer range: reads as zero

    // per-lane offsets, fixed for the whole kernel (each stage adds a scalar offset)
    uint32_t off_a[A_CH], off_b[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int idx = tid + NT * i, r = idx >> 3, c16 = idx & 7;
        off_a[i] = (m0 + r < M) ? (uint32_t)((m0 + r) * K + c16 * 16) : OUT;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int idx = tid + NT * i, c = idx >> 2, b = idx & 3;
        off_b[i] = (n0 + c < N) ? (uint32_t)((n0 + c) * (K / 2) + b * 16) : OUT;
    }
    // scale staging: the thread covers (gi, r) = divmod(tid + NT*i, BM), GPS*BM values
    constexpr int SC_N = (GPS * BM + NT - 1) / NT;
    uint32_t off_xs[SC_N], off_ws[SC_N];
#pragma unroll
    for (int i = 0; i < SC_N; ++i) {
        const int idx = tid + NT * i, gi = idx / BM, r = idx % BM;
        const bool used = idx < GPS * BM;
        off_xs[i] = (used && m0 + r < M) ? (uint32_t)(((m0 + r) * ngroups + gi) * 4) : OUT;
        off_ws[i] = (used && n0 + r < N) ? (uint32_t)(((n0 + r) * ngroups + gi) * 2) : OUT;
    }

    uint4 ra[A_CH], rb[B_CH];
    float rxs[SC_N];
    int32_t rxsum[SC_N];
    uint32_t rws[SC_N], rwb[SC_N];

    // Every load that is not needed (rows past M or N, K past the end of the
    // row in the last stage) gets an out-of-range lane offset, so it reads zero
    // without touching memory whether or not the range check counts the
    // scalar offset.
    auto load_stage = [&](int st) {
        const int k0 = st * KS;
        const int ks = min(KS, K - k0);
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int c16 = (tid + NT * i) & 7;
            const uint32_t o = (c16 * 16 < ks) ? off_a[i] : OUT;
            ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_a, o, k0, 0));
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int b = (tid + NT * i) & 3;
            const uint32_t o = (b * 32 < ks) ? off_b[i] : OUT;
            rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_b, o, k0 >> 1, 0));
        }
        if (!PARTIALS) {
            const int g0 = k0 / G;
#pragma unroll
            for (int i = 0; i < SC_N; ++i) {
                const int gi = (tid + NT * i) / BM;
                const bool in = gi * G < ks;
                const uint32_t ox = in ? off_xs[i] : OUT, ow = in ? off_ws[i] : OUT;
                rxs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_xs, ox, g0 * 4, 0));
                if (AFF) rxsum[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_xsum, ox, g0 * 4, 0);
                rws[i] = __builtin_amdgcn_raw_buffer_load_b16(r_ws, ow, g0 * 2, 0);
                if (AFF) rwb[i] = __builtin_amdgcn_raw_buffer_load_b16(r_wb, ow, g0 * 2, 0);
            }
        }
    };

    auto store_stage = [&](St& S) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int idx = tid + NT * i, r = idx >> 3, c16 = idx & 7;
            S.a[swz(r, c16)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int idx = tid + NT * i, c = idx >> 2, b = idx & 3;
            uint4 lo = make_uint4(lo_nibbles(rb[i].x), lo_nibbles(rb[i].y), lo_nibbles(rb[i].z), lo_nibbles(rb[i].w));
            uint4 hi = make_uint4(hi_nibbles(rb[i].x), hi_nibbles(rb[i].y), hi_nibbles(rb[i].z), hi_nibbles(rb[i].w));
            if (FMT == 0) {
                lo = make_uint4(minus8_bytes(lo.x), minus8_bytes(lo.y), minus8_bytes(lo.z), minus8_bytes(lo.w));
                hi = make_uint4(minus8_bytes(hi.x), minus8_bytes(hi.y), minus8_bytes(hi.z), minus8_bytes(hi.w));
            }
            S.b[swz(c, 2 * b)] = lo;      // k = 32b .. 32b+15
            S.b[swz(c, 2 * b + 1)] = hi;  // k = 32b+16 .. 32b+31
        }
        if (!PARTIALS) {
#pragma unroll
            for (int i = 0; i < SC_N; ++i) {
                const int idx = tid + NT * i;
                if (idx < GPS * BM) {
                    const int gi = idx / BM, r = idx % BM;
                    S.xs[gi][r] = rxs[i];
                    S.ws[gi][r] = AFF ? bf16_to_float(rws[i]) : half_to_float(rws[i]);
                    if (AFF) {
                        S.xb[gi][r] = rxs[i] * (float)rxsum[i];
                        S.wb[gi][r] = bf16_to_float(rwb[i]);
                    }
                }
            }
        }
    };

    // ---------------------------------------------------------------- compute
    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int arow0 = wm * 64 + l32, brow0 = wn * 64 + l32;
    float bva[2] = {0.0f, 0.0f}, bvb[2] = {0.0f, 0.0f};  // bias operands of a pending slot-0 group
    bool bias_pending = false;

    auto do_stage = [&](int st, auto par) {
        constexpr int P = decltype(par)::value;
        __syncthreads();
        if (st + 1 < nstages) store_stage(stage_buf[P ^ 1]);
        if (st + 2 < nstages) load_stage(st + 2);
        const St& S = stage_buf[P];
        const int k0 = st * KS;
        const int ks = min(KS, K - k0);
#pragma unroll
        for (int gi = 0; gi < GPS; ++gi) {
            if (gi * G >= ks) break;
            v16i pi[2][2];
#pragma unroll
            for (int s = 0; s < SPG; ++s) {
                const int chunk = gi * (G / 16) + 2 * s + half;
                v4i af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) af[i] = __builtin_bit_cast(v4i, S.a[swz(arow0 + 32 * i, chunk)]);
#pragma unroll
                for (int j = 0; j < 2; ++j) bf[j] = __builtin_bit_cast(v4i, S.b[swz(brow0 + 32 * j, chunk)]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        if (s == 0) {
                            const v16i z = {};
                            pi[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], z, 0, 0, 0);
                        } else {
                            pi[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], pi[i][j], 0, 0, 0);
                        }
                    }
            }
            // D layout of the 32x32 MFMA: lane holds column l32, rows 8*(r/4) + 4*half + r%4.
            if (PARTIALS) {
                const int g = k0 / G + gi;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                            if (m < M && n < N) partials[((size_t)m * N + n) * ngroups + g] = pi[i][j][r];
                        }
                    }
                continue;
            }
            float wsv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) wsv[j] = S.ws[gi][wn * 64 + 32 * j + l32];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float xsv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(&S.xs[gi][wm * 64 + 32 * i + 8 * q + 4 * half]);
                    xsv[4 * q] = v.x; xsv[4 * q + 1] = v.y; xsv[4 * q + 2] = v.z; xsv[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += xsv[r] * (wsv[j] * (float)pi[i][j][r]);
            }
            if (BIAS_MFMA) {
                // two groups per f32 MFMA: lanes of half h supply group slot h
                float va[2], vb[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) va[i] = S.xb[gi][wm * 64 + 32 * i + l32];
#pragma unroll
                for (int j = 0; j < 2; ++j) vb[j] = S.wb[gi][wn * 64 + 32 * j + l32];
                if (bias_pending) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) va[i] = half ? va[i] : bva[i];
#pragma unroll
                    for (int j = 0; j < 2; ++j) vb[j] = half ? vb[j] : bvb[j];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[i], vb[j], acc[i][j], 0, 0, 0);
                    bias_pending = false;
                } else {
                    bva[0] = va[0]; bva[1] = va[1];
                    bvb[0] = vb[0]; bvb[1] = vb[1];
                    bias_pending = true;
                }
            }
        }
    };

    load_stage(0);
    store_stage(stage_buf[0]);
    if (nstages > 1) load_stage(1);
    for (int st = 0; st < nstages; st += 2) {
        do_stage(st, std::integral_constant<int, 0>());
        if (st + 1 < nstages) do_stage(st + 1, std::integral_constant<int, 1>());
    }
    if (!PARTIALS) {
        if (BIAS_MFMA && bias_pending) {
            float va[2], vb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) va[i] = half ? 0.0f : bva[i];
#pragma unroll
            for (int j = 0; j < 2; ++j) vb[j] = half ? 0.0f : bvb[j];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[i], vb[j], acc[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (m < M && n < N) y[(size_t)m * N + n] = acc[i][j][r];
                }
            }
    }
}

template <int FMT, int G>
hipError_t launch_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    const unsigned tiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
    const size_t lds = 2 * sizeof(Stage<G, FMT>);
    const uint16_t* ws = static_cast<const uint16_t*>(wscale);
    const uint16_t* wb = static_cast<const uint16_t*>(wbias);
    if (partials) {
        auto k = gemm_kernel<FMT, G, true>;
        static bool attr = false;
        if (!attr) {
            hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            attr = true;
        }
        hipLaunchKernelGGL(k, dim3(tiles), dim3(NT), lds, stream, M, K, N, wq, ws, wb, xq, xs, xsum, y, partials);
    } else {
        auto k = gemm_kernel<FMT, G, false>;
        static bool attr = false;
        if (!attr) {
            hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            attr = true;
        }
        hipLaunchKernelGGL(k, dim3(tiles), dim3(NT), lds, stream, M, K, N, wq, ws, wb, xq, xs, xsum, y, partials);
    }
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
