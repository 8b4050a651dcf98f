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
// held under 256 per lane and LDS under 80 KB per workgroup).
//
// K is walked in 128-wide stages through two LDS tile buffers. The stage's
// global loads are buffer loads with a per-lane offset fixed for the whole
// kernel and the stage offset in a scalar register; rows past M or N read as
// zero (the buffer range check), so the staging needs no masks. After the one
// barrier of a stage, the registers holding stage s+1 are written to the free
// buffer (weight nibbles unpacked on the way: q - 8 as signed bytes for Q4_0,
// q for affine), the loads of stage s+2 are issued, and stage s is computed.
// LDS rows are 128 bytes with the 16-byte chunk index XORed with bits of the
// row index, so the MFMA fragment reads (32 rows at one K offset) hit all banks.
//
// Per block (Q4_0) or group (affine, 64 / 128 weights = 2 / 4 MFMA steps) the
// int32 tile is rescaled into float accumulators:
//   Q4_0:   acc += xs[m] * (d[n] * P)                 2 VALU ops per output
//   affine: acc += xs[m] * (s[n] * A)                 2 VALU ops per output
//           acc += sum_g (xs * xsum)[m, g] * b[n, g]  on the f32 matrix core
// The integer-to-float conversion costs no instruction: each group's MFMA
// chain starts from the integer 0x4B400000 (the bits of C = 1.5 * 2^23)
// instead of zero. Every block or group sum P or A lies within +-2^22, so the
// chain ends on the bits of the float C + P exactly, and one FMA with the
// exact constant -d * C (d has at most 11 significant bits) gives d * P
// rounded once, as a conversion and a multiply would. The limit this puts on
// the weight scales: d * C must stay finite, |d| < 2^104. (8-bit codes stage
// twice the code bytes per thread and keep the conversion: the 16 registers
// holding the start value do not fit beside them.)
// The affine bias term is a rank-(K/g) product, so it runs as
// v_mfma_f32_32x32x2_f32 with two groups in its two K slots instead of a
// fourth VALU op per output.
//
// The rescale is VALU work of the same order as the matrix work, so the two
// are software-pipelined inside each wavefront: while the matrix core runs
// the MFMA chain of one of the wavefront's four tiles for group g, the VALU
// rescales the tile before it, whose integers are complete. Two int32 tiles
// are live at a time instead of four, which pays for the registers the
// overlap needs. Because the last tile's rescale trails its group into the
// next stage, the per-stage scales sit in a ring of three LDS slots rather
// than in the double-buffered tile memory.
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

constexpr int KS = 128;              // K per stage
constexpr int BM = 128, BN = 128;    // workgroup tile
constexpr int NT = 256;              // threads per workgroup (2 x 2 wavefronts)
constexpr int GROUP_M = 8;           // row tiles per tile group
constexpr int NXCD = 8;
constexpr int RING = 3;              // scale slots
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer descriptor: 32-bit data format
constexpr int CHAIN_BIAS = 0x4B400000;  // bits of the float 1.5 * 2^23
constexpr float CHAIN_BIAS_F = 12582912.0f;

struct Tiles {
    uint4 a[BM * KS / 16];  // int8 activation codes, swizzled 128-byte rows
    uint4 b[BN * KS / 16];  // unpacked weight codes, swizzled 128-byte rows
};

// Scales of one stage. The staging threads cover SR = max(GPS, NT / 128) rows
// of each array; rows past GPS only receive the zeros of threads with no
// scale to stage, so the staging stores need no branch.
template <int G, int FMT>
struct Scales {
    static constexpr int GPS = KS / G;
    static constexpr int SR = (GPS > NT / BM) ? GPS : NT / BM;
    static constexpr int NB = (FMT == 1) ? SR : 1;  // affine keeps the bias operands too
    float xs[SR][BM];
    float ws[SR][BN];
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

// PACKED: wq, wscale and wbias point into a packed weight buffer (one 8 KB
// block of codes per 128-column tile and stage, rows in order; scales and
// biases as [tile][group][128]) and xs, xsum are group-major, [K/G][M]. Every
// staging load of the stage is then contiguous across the workgroup's threads.
// BITS: affine code width (MLX PR #4802 serves 4, 6 and 8 bits): 4 -> the
// nibble planes; 6 -> the nibble planes of the low 4 bits, then at N*K/2 a
// plane of the high 2 bits (8 bytes per 32-code block: word h holds code
// 16h + c in byte c % 4, bits 2 * (c / 4)); 8 -> one byte per code, staged as
// q - 128 (signed for the MFMA) with 128 * s added to the group's bias.
// KSP: K split inside the workgroup. With KSP = 2 the workgroup has two groups
// of 2 x 2 wavefronts; group h takes the h-th half of the K stages with its own
// LDS tiles and scales, and at the end group 1's accumulators are added to
// group 0's through LDS (for tile counts too small to put two workgroups on
// every CU: twice the wavefronts per SIMD, half the stages each).
template <int FMT, int G, bool PARTIALS, bool PACKED, int BITS, int KSP>
__global__ __launch_bounds__(NT * KSP, KSP == 1 ? 2 : 1) void gemm_kernel(int M, int K, int N, const uint8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ wscale,
                                                      const uint16_t* __restrict__ wbias,
                                                      const int8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      const int32_t* __restrict__ xsum, float* __restrict__ y,
                                                      int32_t* __restrict__ partials) {
    constexpr int GPS = KS / G;  // blocks or groups per stage
    constexpr int SPG = G / 32;  // MFMA K steps per block or group
    constexpr int A_CH = BM * (KS / 16) / NT;  // 16-byte activation chunks per thread per stage (4)
    constexpr int B_CH = BN * (KS / (BITS == 8 ? 16 : 32)) / NT;  // 16-byte code chunks per thread per stage (2 / 4)
    static_assert(BITS == 4 || (FMT == 1 && !PACKED && (BITS == 6 || BITS == 8)), "code width");
    constexpr bool AFF = FMT == 1;
    constexpr bool BIAS_MFMA = AFF && !PARTIALS;
    using Sc = Scales<G, FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // K half of this thread's wavefront group, and the thread index within the group
    const int kh = KSP == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
    uint8_t* hmem = smem + (size_t)kh * (2 * sizeof(Tiles) + RING * sizeof(Sc));
    Tiles* tiles = reinterpret_cast<Tiles*>(hmem);
    Sc* ring = reinterpret_cast<Sc*>(hmem + 2 * sizeof(Tiles));

    const int tid = (int)threadIdx.x - kh * NT, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int ngroups = K / G;
    const int nstages = (K + KS - 1) / KS;
    // this group's stages: [st_begin, st_begin + nst); stages past the end of K read zero
    const int nst = (nstages + KSP - 1) / KSP;
    const int st_begin = kh * nst;
    const int half = lane >> 5, l32 = lane & 31;

    // ---------------------------------------------------------------- staging
    const __amdgpu_buffer_rsrc_t r_a = rsrc(xq, (uint32_t)((size_t)M * K));
    const int ntn = (N + BN - 1) / BN;  // column tiles
    const size_t wrows = PACKED ? (size_t)ntn * BN : (size_t)N;  // weight rows as stored
    const __amdgpu_buffer_rsrc_t r_b =
        rsrc(wq, (uint32_t)(PACKED ? (size_t)ntn * nstages * (BN * KS / 2) : (size_t)N * K * BITS / 8));
    const __amdgpu_buffer_rsrc_t r_xs = rsrc(xs, PARTIALS ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_xsum = rsrc(xsum, PARTIALS ? 0u : (uint32_t)((size_t)M * ngroups * 4));
    const __amdgpu_buffer_rsrc_t r_ws = rsrc(wscale, PARTIALS ? 0u : (uint32_t)(wrows * ngroups * 2));
    const __amdgpu_buffer_rsrc_t r_wb = rsrc(wbias, (PARTIALS || !AFF) ? 0u : (uint32_t)(wrows * ngroups * 2));
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
        if (BITS == 8) {  // row c = idx / 8, 16-byte chunk idx % 8 of the stage's 128 codes
            const int idx = tid + NT * i, c = idx >> 3, c16 = idx & 7;
            off_b[i] = (n0 + c < N) ? (uint32_t)((n0 + c) * K + c16 * 16) : OUT;
        } else {
            const int idx = tid + NT * i, c = idx >> 2, b = idx & 3;
            // packed: row c's 64 bytes of the stage sit at c * 64 of the tile's block
            off_b[i] = PACKED ? (uint32_t)(idx * 16) : (n0 + c < N) ? (uint32_t)((n0 + c) * (K / 2) + b * 16) : OUT;
        }
    }
    // 6 bits: the high 2-bit plane of each 32-code block, 8 bytes per block
    uint32_t off_p[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int idx = tid + NT * i, c = idx >> 2, b = idx & 3;
        off_p[i] = (BITS == 6 && n0 + c < N) ? (uint32_t)((size_t)N * (K / 2) + (n0 + c) * (K / 4) + b * 8) : OUT;
    }
    // scale staging: the thread covers (gi, r) = divmod(tid + NT*i, 128) of the
    // GPS*128 activation scales and of the GPS*128 weight scales
    static_assert(BM == BN, "scale staging assumes a square tile");
    constexpr int SC_N = (GPS * BM + NT - 1) / NT;
    static_assert(SC_N * NT <= Sc::SR * BM, "scale staging overruns its rows");
    uint32_t off_xs[SC_N], off_ws[SC_N];
#pragma unroll
    for (int i = 0; i < SC_N; ++i) {
        const int idx = tid + NT * i, gi = idx / BM, r = idx % BM;
        const bool used = idx < GPS * BM;
        if (PACKED) {
            off_xs[i] = (used && m0 + r < M) ? (uint32_t)((gi * M + m0 + r) * 4) : OUT;
            off_ws[i] = used ? (uint32_t)((gi * BN + r) * 2) : OUT;
        } else {
            off_xs[i] = (used && m0 + r < M) ? (uint32_t)(((m0 + r) * ngroups + gi) * 4) : OUT;
            off_ws[i] = (used && n0 + r < N) ? (uint32_t)(((n0 + r) * ngroups + gi) * 2) : OUT;
        }
    }

    uint4 ra[A_CH], rb[B_CH];
    uint2 rp[BITS == 6 ? B_CH : 1];
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
            // the chunk's first k within the stage: 16 * (idx % 8) for 8 bits, 32 * (idx % 4) otherwise
            const int kc = BITS == 8 ? 16 * ((tid + NT * i) & 7) : 32 * ((tid + NT * i) & 3);
            const uint32_t o = (kc < ks) ? off_b[i] : OUT;
            const int sb = PACKED ? (tn * nstages + st) * (BN * KS / 2) : (BITS == 8 ? k0 : (k0 >> 1));
            rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r_b, o, sb, 0));
            if (BITS == 6)
                rp[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r_b, (kc < ks) ? off_p[i] : OUT,
                                                                                        k0 >> 2, 0));
        }
        if (!PARTIALS) {
            const int g0 = k0 / G;
            const int sx = PACKED ? g0 * M * 4 : g0 * 4;
            const int sw = PACKED ? (tn * ngroups + g0) * (BN * 2) : g0 * 2;
#pragma unroll
            for (int i = 0; i < SC_N; ++i) {
                const int gi = (tid + NT * i) / BM;
                const bool in = gi * G < ks;
                const uint32_t ox = in ? off_xs[i] : OUT, ow = in ? off_ws[i] : OUT;
                rxs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_xs, ox, sx, 0));
                if (AFF) rxsum[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(r_xsum, ox, sx, 0);
                rws[i] = __builtin_amdgcn_raw_buffer_load_b16(r_ws, ow, sw, 0);
                if (AFF) rwb[i] = __builtin_amdgcn_raw_buffer_load_b16(r_wb, ow, sw, 0);
            }
        }
    };

    auto store_stage = [&](Tiles& T, Sc& S) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int idx = tid + NT * i, r = idx >> 3, c16 = idx & 7;
            T.a[swz(r, c16)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            if (BITS == 8) {  // codes q - 128 as signed bytes: flip bit 7 of every byte
                const int idx = tid + NT * i, c = idx >> 3, c16 = idx & 7;
                const uint4 v = rb[i];
                T.b[swz(c, c16)] = make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u,
                                              v.w ^ 0x80808080u);
                continue;
            }
            const int idx = tid + NT * i, c = idx >> 2, b = idx & 3;
            uint4 lo = make_uint4(lo_nibbles(rb[i].x), lo_nibbles(rb[i].y), lo_nibbles(rb[i].z), lo_nibbles(rb[i].w));
            uint4 hi = make_uint4(hi_nibbles(rb[i].x), hi_nibbles(rb[i].y), hi_nibbles(rb[i].z), hi_nibbles(rb[i].w));
            if (FMT == 0) {
                lo = make_uint4(minus8_bytes(lo.x), minus8_bytes(lo.y), minus8_bytes(lo.z), minus8_bytes(lo.w));
                hi = make_uint4(minus8_bytes(hi.x), minus8_bytes(hi.y), minus8_bytes(hi.z), minus8_bytes(hi.w));
            }
            if (BITS == 6) {  // word j of a half takes bits 2j, 2j+1 of every byte of its plane word
                lo = make_uint4(lo.x | two_bits_high(rp[i].x, 0), lo.y | two_bits_high(rp[i].x, 1),
                                lo.z | two_bits_high(rp[i].x, 2), lo.w | two_bits_high(rp[i].x, 3));
                hi = make_uint4(hi.x | two_bits_high(rp[i].y, 0), hi.y | two_bits_high(rp[i].y, 1),
                                hi.z | two_bits_high(rp[i].y, 2), hi.w | two_bits_high(rp[i].y, 3));
            }
            T.b[swz(c, 2 * b)] = lo;      // k = 32b .. 32b+15
            T.b[swz(c, 2 * b + 1)] = hi;  // k = 32b+16 .. 32b+31
        }
        if (!PARTIALS) {
#pragma unroll
            for (int i = 0; i < SC_N; ++i) {
                const int idx = tid + NT * i, gi = idx / BM, r = idx % BM;
                S.xs[gi][r] = rxs[i];
                S.ws[gi][r] = AFF ? bf16_to_float(rws[i]) : half_to_float(rws[i]);
                if (AFF) {
                    S.xb[gi][r] = rxs[i] * (float)rxsum[i];
                    // 8 bits: the MFMA sees q - 128, so the bias term carries 128 * s
                    S.wb[gi][r] = bf16_to_float(rwb[i]) + (BITS == 8 ? 128.0f * bf16_to_float(rws[i]) : 0.0f);
                }
            }
        }
    };

    // ---------------------------------------------------------------- compute
    // The wavefront's four 32 x 32 tiles (i, j) -- rows wm*64 + 32i, columns
    // wn*64 + 32j -- are visited in the order (0,0) (0,1) (1,1) (1,0), so that
    // consecutive tiles share a fragment. Phase t of a group runs tile t's MFMA
    // chain into pi[t & 1] while the VALU rescales tile t - 1 from pi[(t+1) & 1].
    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    v16i pi[2];

    const int arow = wm * 64 + l32;       // fragment row of A (+ 32i); also the bias row of xb
    const int brow = wn * 64 + l32;       // fragment row of B (+ 32j): this lane's output column
    const int xrow = wm * 64 + 4 * half;  // first output row of this lane (+ 32i + 8q + r)

    auto frag = [&](const uint4* base, int row, int gi, int s) {
        return __builtin_bit_cast(v4i, base[swz(row, gi * (G / 16) + 2 * s + half)]);
    };

    // Start value of every MFMA chain: the bits of 1.5 * 2^23, or zero for
    // 8-bit codes (the empty asm keeps the 16 registers live instead of
    // rebuilding them before each chain). The partials view runs the same
    // chain and reports its integer minus the start value.
    constexpr bool BIASED = BITS != 8;
    v16i chain0;
#pragma unroll
    for (int r = 0; r < 16; ++r) chain0[r] = BIASED ? CHAIN_BIAS : 0;
    if (BIASED) asm("" : "+v"(chain0));

    // MFMA chain of one group for one tile.
    auto mfma_tile = [&](v16i& d, const v4i (&fa)[SPG], const v4i (&fb)[SPG]) {
        d = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[0], fb[0], chain0, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < SPG; ++s) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s], fb[s], d, 0, 0, 0);
    };

    // Activation scales of this lane's 16 rows in strip i (slot gi of S); the
    // two tiles of a strip share them.
    auto read_xs = [&](float (&xsv)[16], const Sc& S, int gi, int i) {
        if (PARTIALS) return;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&S.xs[gi][xrow + 32 * i + 8 * q]);
            xsv[4 * q] = v.x; xsv[4 * q + 1] = v.y; xsv[4 * q + 2] = v.z; xsv[4 * q + 3] = v.w;
        }
    };

    // Rescale tile (i, j)'s integers of group g (slot gi of scale set S, xsv
    // from read_xs) into acc, or store them as partials. D layout of the 32x32
    // MFMA: lane holds column l32, rows 8*(r/4) + 4*half + r%4.
    auto rescale_tile = [&](const v16i& d, const float (&xsv)[16], const Sc& S, int gi, int i, int j, int g) {
        if (PARTIALS) {
            // row r of the lane's 16 sits (8*(r/4) + r%4) rows below its first row;
            // the row stride is wave-uniform, so the offsets stay in scalar registers
            const int n = n0 + brow + 32 * j;
            const int mb = m0 + xrow + 32 * i;
            const size_t rstride = (size_t)__builtin_amdgcn_readfirstlane(N * ngroups);
            int32_t* pb = partials + ((size_t)mb * N + n) * ngroups + g;
            const size_t sstride = (size_t)__builtin_amdgcn_readfirstlane(ngroups);
            const int32_t* sb = xsum + (size_t)mb * ngroups + g;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = 8 * (r >> 2) + (r & 3);
                if (mb + dr < M && n < N && g < ngroups) {
                    // 8 bits: the MFMA summed (q - 128) * xq; the reported partial is sum q * xq
                    const int fix = BITS == 8 ? 128 * sb[dr * sstride] : 0;
                    pb[dr * rstride] = (d[r] - (BIASED ? CHAIN_BIAS : 0)) + fix;
                }
            }
            return;
        }
        const float w = S.ws[gi][brow + 32 * j];
        if (!BIASED) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] += xsv[r] * (w * (float)d[r]);
            return;
        }
        const float wc = w * -CHAIN_BIAS_F;  // exact
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // copy the element first: clang's bit_cast of a vector element
            // subscript reads element 0 whatever the index
            const int e = d[r];
            acc[i][j][r] += xsv[r] * fmaf(w, __builtin_bit_cast(float, e), wc);
        }
    };

    // Affine bias of two groups on the f32 matrix core for tile (i, j): lanes
    // of half 0 supply group slot 0 (S0, gi0), lanes of half 1 group slot 1
    // (S1, gi1), or zero when that slot is empty.
    auto bias_tile = [&](const Sc& S0, int gi0, const Sc& S1, int gi1, int i, int j, bool second) {
        const Sc& S = half ? S1 : S0;
        const int gi = half ? gi1 : gi0;
        const bool on = !half || second;
        const float va = on ? S.xb[gi][arow + 32 * i] : 0.0f;
        const float vb = on ? S.wb[gi][brow + 32 * j] : 0.0f;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, vb, acc[i][j], 0, 0, 0);
    };

    const int g_begin = st_begin * GPS;
    int g = g_begin;  // global index of the next group
    int rs = 0, rs_prev = RING - 1;  // ring slots of the current and the previous stage
    // The first phase rescales tile (1,0) of a group "-1": its integers are zero
    // and the scale slot standing for stage -1 is zeroed, so it adds exactly zero
    // and the pipeline needs no branch.
    pi[1] = v16i{};
    float xs0[16], xs1[16];  // activation scales of strip 0 (current group) and strip 1 (held into the next group)
#pragma unroll
    for (int r = 0; r < 16; ++r) xs1[r] = 0.0f;
    if (!PARTIALS) {
        float* z = reinterpret_cast<float*>(&ring[RING - 1]);
        for (int i = tid; i < (int)(sizeof(Sc) / 4); i += NT) z[i] = 0.0f;
    }

    // One stage. The stage is straight-line code: stages and groups past the
    // end of K are staged and computed like the others, from loads that read
    // zero (codes and scales alike), so they add exactly zero.
    auto do_stage = [&](int st, auto par) {
        constexpr int P = decltype(par)::value;
        __syncthreads();
        const int rs_next = (rs + 1 == RING) ? 0 : rs + 1;
        store_stage(tiles[P ^ 1], ring[rs_next]);
        load_stage(st + 2);
        const Tiles& T = tiles[P];
        const Sc& S = ring[rs];
        const Sc& Sp = ring[rs_prev];
#pragma unroll
        for (int gi = 0; gi < GPS; ++gi) {
            // group g - 1: earlier in this stage, or the last group of the previous stage
            const Sc& S1 = gi == 0 ? Sp : S;
            const int gi1 = gi == 0 ? GPS - 1 : gi - 1;
            // bias groups pair up as (g - 1, g) for odd g = st*GPS + gi; stages alternate P
            const bool odd = (GPS == 1) ? (P == 1) : ((gi & 1) == 1);
            v4i fa0[SPG], fa1[SPG], fb0[SPG], fb1[SPG];
#pragma unroll
            for (int s2 = 0; s2 < SPG; ++s2) {
                fa0[s2] = frag(T.a, arow, gi, s2);
                fb0[s2] = frag(T.b, brow, gi, s2);
            }
            // phase 0: tile (0,0) of group g; rescale tile (1,0) of group g - 1
            mfma_tile(pi[0], fa0, fb0);
            if (BIAS_MFMA && odd) bias_tile(S1, gi1, S, gi, 0, 0, true);
            if (!PARTIALS || g > g_begin) rescale_tile(pi[1], xs1, S1, gi1, 1, 0, g - 1);
            __builtin_amdgcn_sched_barrier(0);
            // phase 1: tile (0,1); rescale tile (0,0)
#pragma unroll
            for (int s2 = 0; s2 < SPG; ++s2) fb1[s2] = frag(T.b, brow + 32, gi, s2);
            mfma_tile(pi[1], fa0, fb1);
            if (BIAS_MFMA && odd) bias_tile(S1, gi1, S, gi, 0, 1, true);
            read_xs(xs0, S, gi, 0);
            rescale_tile(pi[0], xs0, S, gi, 0, 0, g);
            __builtin_amdgcn_sched_barrier(0);
            // phase 2: tile (1,1); rescale tile (0,1)
#pragma unroll
            for (int s2 = 0; s2 < SPG; ++s2) fa1[s2] = frag(T.a, arow + 32, gi, s2);
            mfma_tile(pi[0], fa1, fb1);
            if (BIAS_MFMA && odd) bias_tile(S1, gi1, S, gi, 1, 1, true);
            rescale_tile(pi[1], xs0, S, gi, 0, 1, g);
            __builtin_amdgcn_sched_barrier(0);
            // phase 3: tile (1,0); rescale tile (1,1)
            mfma_tile(pi[1], fa1, fb0);
            if (BIAS_MFMA && odd) bias_tile(S1, gi1, S, gi, 1, 0, true);
            read_xs(xs1, S, gi, 1);
            rescale_tile(pi[0], xs1, S, gi, 1, 1, g);
            __builtin_amdgcn_sched_barrier(0);
            ++g;
        }
        rs_prev = rs;
        rs = rs_next;
    };

    load_stage(st_begin);
    store_stage(tiles[0], ring[0]);
    load_stage(st_begin + 1);
    const int st_end = st_begin + nst;  // the same count in both groups (the barriers pair up)
    int st = st_begin;
    for (; st + 1 < st_end; st += 2) {
        do_stage(st, std::integral_constant<int, 0>());
        do_stage(st + 1, std::integral_constant<int, 1>());
    }
    if (st < st_end) do_stage(st, std::integral_constant<int, 0>());
    // tile (1,0) of the last group of the last stage (whose scales are in that
    // stage's slot); with one group per stage and an odd stage count the last
    // group's bias has no partner group
    {
        const Sc& Sl = ring[rs_prev];
        const int gl = st_end * GPS - 1;
        rescale_tile(pi[1], xs1, Sl, GPS - 1, 1, 0, gl);
        if (BIAS_MFMA && GPS == 1 && (nst & 1)) {
            const int gil = GPS - 1;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) bias_tile(Sl, gil, Sl, gil, i, j, false);
        }
    }
    if (!PARTIALS && KSP == 2) {
        // group 1's accumulators into group 0's, through group 1's tile memory
        __syncthreads();
        float* part = reinterpret_cast<float*>(smem + 2 * sizeof(Tiles) + RING * sizeof(Sc));
        if (kh == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    *reinterpret_cast<v16f*>(&part[(((2 * i + j) * NT) + tid) * 16]) = acc[i][j];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] += *reinterpret_cast<const v16f*>(&part[(((2 * i + j) * NT) + tid) * 16]);
    }
    if (!PARTIALS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + brow + 32 * j;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + xrow + 32 * i + 8 * (r >> 2) + (r & 3);
                    if (m < M && n < N) y[(size_t)m * N + n] = acc[i][j][r];
                }
            }
    }
}

template <int FMT, int G, bool PACKED, int BITS, int KSP>
hipError_t launch_ksp(unsigned ntiles, int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    const size_t lds = KSP * (2 * sizeof(Tiles) + RING * sizeof(Scales<G, FMT>));
    const uint16_t* ws = static_cast<const uint16_t*>(wscale);
    const uint16_t* wb = static_cast<const uint16_t*>(wbias);
    auto k = partials ? gemm_kernel<FMT, G, true, PACKED, BITS, KSP> : gemm_kernel<FMT, G, false, PACKED, BITS, KSP>;
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(k), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(ntiles), dim3(NT * KSP), lds, stream, M, K, N, wq, ws, wb, xq, xs, xsum, y, partials);
    return hipGetLastError();
}

// Up to one tile per CU (and at least KSPLIT_STAGES K stages), K is split over
// two wavefront groups per workgroup. Measured on affine g64 1024 x 4096 x 4096
// (256 tiles): packed 74.4 -> 60.3 us, unpacked 72.0 -> 70.1 us; at 512 tiles
// (one workgroup per CU then, for the split's LDS) it is slower.
constexpr unsigned KSPLIT_TILES = 256;
constexpr int KSPLIT_STAGES = 8;

template <int FMT, int G, bool PACKED, int BITS = 4>
hipError_t launch_fmt(int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                      const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                      hipStream_t stream) {
    const unsigned ntiles = (unsigned)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
    if (ntiles <= KSPLIT_TILES && (K + KS - 1) / KS >= KSPLIT_STAGES)
        return launch_ksp<FMT, G, PACKED, BITS, 2>(ntiles, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials,
                                                   stream);
    return launch_ksp<FMT, G, PACKED, BITS, 1>(ntiles, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
}

// Packed weights: copy row r's bytes of stage s into block (t, s) and the
// scales (and biases) into [tile][group][128]; rows past N are zero, so the
// GEMM's staging of a packed tile needs no row masks.
__global__ __launch_bounds__(256) void pack_codes_kernel(int N, int K, const uint8_t* __restrict__ wq,
                                                         uint8_t* __restrict__ out, long long nchunks) {
    const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte chunk of the output
    if (j >= nchunks) return;
    const int nstages = (K + KS - 1) / KS;
    const long long blk = j / (BN * KS / 32);
    const int within = (int)(j - blk * (BN * KS / 32));
    const int t = (int)(blk / nstages), st = (int)(blk - (long long)t * nstages);
    const int r = within >> 2, b = within & 3;
    const int n = t * BN + r, kb = st * (KS / 2) + 16 * b;  // byte offset in the row
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N && kb < K / 2) v = *reinterpret_cast<const uint4*>(wq + (size_t)n * (K / 2) + kb);
    reinterpret_cast<uint4*>(out)[j] = v;
}

__global__ __launch_bounds__(256) void pack_scales_kernel(int N, int ngroups, const uint16_t* __restrict__ ws,
                                                          uint16_t* __restrict__ out, long long count) {
    const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // (tile, group, row)
    if (j >= count) return;
    const int r = (int)(j % BN);
    const long long tg = j / BN;
    const int g = (int)(tg % ngroups), t = (int)(tg / ngroups);
    const int n = t * BN + r;
    out[j] = (n < N) ? ws[(size_t)n * ngroups + g] : (uint16_t)0;
}

}  // namespace

template <int G>
hipError_t launch_affine_bits(int bits, int M, int K, int N, const uint8_t* wq, const void* wscale, const void* wbias,
                              const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                              hipStream_t stream) {
    if (bits == 4) return launch_fmt<1, G, false, 4>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bits == 6) return launch_fmt<1, G, false, 6>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bits == 8) return launch_fmt<1, G, false, 8>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                       const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                       int32_t* partials, hipStream_t stream) {
    if (fmt == 0) {
        if (bits != 4) return hipErrorInvalidValue;
        return launch_fmt<0, 32, false>(M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    }
    if (bs == 64) return launch_affine_bits<64>(bits, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    if (bs == 128) return launch_affine_bits<128>(bits, M, K, N, wq, wscale, wbias, xq, xs, xsum, y, partials, stream);
    return hipErrorInvalidValue;
}

size_t packed_code_bytes(int K, int N) {
    return (size_t)((N + BN - 1) / BN) * ((K + KS - 1) / KS) * (BN * KS / 2);
}

size_t packed_scale_bytes(int K, int N, int bs) { return (size_t)((N + BN - 1) / BN) * (K / bs) * BN * 2; }

hipError_t launch_pack_weights(int N, int K, int bs, int fmt, const uint8_t* wq, const void* wscale,
                               const void* wbias, uint8_t* packed, hipStream_t stream) {
    const size_t cb = packed_code_bytes(K, N), sb = packed_scale_bytes(K, N, bs);
    const long long nchunks = (long long)(cb / 16);
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream, N, K, wq,
                       packed, nchunks);
    const long long count = (long long)(sb / 2);
    const unsigned grid = (unsigned)((count + 255) / 256);
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid), dim3(256), 0, stream, N, K / bs,
                       static_cast<const uint16_t*>(wscale), reinterpret_cast<uint16_t*>(packed + cb), count);
    if (fmt == 1)
        hipLaunchKernelGGL(pack_scales_kernel, dim3(grid), dim3(256), 0, stream, N, K / bs,
                           static_cast<const uint16_t*>(wbias), reinterpret_cast<uint16_t*>(packed + cb + sb), count);
    return hipGetLastError();
}

hipError_t launch_gemm_packed(int M, int K, int N, int bs, int fmt, const uint8_t* packed, const int8_t* xq,
                              const float* xs_gm, const int32_t* xsum_gm, float* y, hipStream_t stream) {
    const size_t cb = packed_code_bytes(K, N), sb = packed_scale_bytes(K, N, bs);
    const void* ws = packed + cb;
    const void* wb = packed + cb + sb;
    if (fmt == 0) return launch_fmt<0, 32, true>(M, K, N, packed, ws, nullptr, xq, xs_gm, xsum_gm, y, nullptr, stream);
    if (bs == 64) return launch_fmt<1, 64, true>(M, K, N, packed, ws, wb, xq, xs_gm, xsum_gm, y, nullptr, stream);
    if (bs == 128) return launch_fmt<1, 128, true>(M, K, N, packed, ws, wb, xq, xs_gm, xsum_gm, y, nullptr, stream);
    return hipErrorInvalidValue;
}

}  // namespace q4
