/*
 * q4.h -- C ABI of the gfx950 (MI355X) block-quantized 4-bit matmul library.
 *
 * The library computes matrix products with 4-bit block-quantized weights:
 *   - W4A8: Q4_0 weights (32-weight blocks, one fp16 scale d each, value
 *     d * (q - 8)) or affine 4-bit weights (groups of 64 or 128 weights with a
 *     bf16 scale s and bias b, value s * q + b), times activations quantized
 *     per block to int8. Each block's dot product is an exact integer; the
 *     per-block float rescale (and, for affine weights, bias * sum x) is
 *     applied in the kernel; the output is float32.
 *     (tract PR #2432 "WIP: W4A8 (Q4_0 int8-dot) path for block_quant",
 *     section "The kernel" and its pipeline figure; MLX PR #4802, mx.qqmm with
 *     mode="affine": int8 x int8 MMA over the original codes with per-group
 *     scales and biases applied in the kernel.)
 *   - Q4_K: 256-weight super-blocks times float32 activations with the
 *     dequantization fused into the multiply-add (C-Kernel-Engine
 *     gemm_kernels_q4k.c: gemv_q4_k_ref, gemm_q4_k_ref, gemm_nt_q4_k).
 *
 * Conventions for every entry point
 *   - Shapes: X is [M][K], W is [N][K], Y is [M][N], all row-major (the
 *     gemm_nt_q4_k convention: A [M x K] activations, B [N x K] weights,
 *     C [M x N] output). M, N >= 1; K a positive multiple of the block size.
 *   - Memory: every pointer is a DEVICE pointer owned by the caller. The
 *     library never allocates or frees memory and keeps no per-call state.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream). Each
 *     call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns; results are valid once the caller synchronizes
 *     the stream. Calls are deterministic (no float atomics).
 *   - Errors: an invalid call returns a nonzero q4_status and enqueues
 *     nothing. Q4_ERR_HIP reports a failed kernel launch. q4_status_string()
 *     names a status.
 *   - Bit width: `bits` is the code width. Q4_0 codes are 4 bits. Affine
 *     codes may be 4, 6 or 8 bits wide (MLX PR #4802 serves all three on its
 *     int8 path) in q4_gemm, q4_debug_partials (GEMM paths) and
 *     q4_quantize_weights; every other entry point decodes 4-bit codes only.
 *     A width an entry point does not decode is rejected with Q4_ERR_FORMAT
 *     before any launch: a decoder handed another width reads the bytes
 *     wrongly without any other sign (meTile PR #29, "Measure the int8
 *     multi-row headroom, and keep the four-bit guard that was protecting us").
 *
 * Code layout (shared by Q4_0 and affine)
 *   4 bits: wq [N][K/2] bytes. Block b (32 weights) of row n is the 16 bytes
 *   at wq + n*K/2 + 16*b; byte j holds the code of k = 32*b + j in its low
 *   nibble and of k = 32*b + 16 + j in its high nibble. An affine group of g
 *   weights is g/32 consecutive blocks.
 *   8 bits (affine): wq [N][K] bytes, byte k of row n is the code of k.
 *   6 bits (affine): N*K*3/4 bytes. The low 4 bits of every code in the
 *   4-bit layout (N*K/2 bytes), then the high 2 bits: N*K/4 bytes, row n at
 *   N*K/2 + n*K/4, block b at 8*b within it as two little-endian 32-bit
 *   words; word h holds code 32*b + 16*h + c (c = 0..15) in byte c % 4, bits
 *   2*(c/4) and 2*(c/4) + 1.
 *   Affine codes of width B run 0 .. 2^B - 1; the weight is s*q + b.
 *
 * Q4_K block layout (144 bytes, 4.5 bits per weight)
 *   { fp16 d; fp16 dmin; uint8 scales[12]; uint8 qs[128]; }, blocks [N][K/256].
 *   scales holds sixteen 6-bit fields, little-endian, field f at bits
 *   [6f, 6f+6): f < 8 is the scale sc[f] of sub-block f, f >= 8 the min
 *   m[f-8]. Chunk c (0..3) of 64 weights uses qs[32c .. 32c+31]: weight
 *   64c + l is the low nibble of qs[32c + l] (sub-block 2c), weight
 *   64c + 32 + l its high nibble (sub-block 2c+1). Weight value
 *   d * sc[s] * q - dmin * m[s].
 *   The packing of the sixteen 6-bit fields is this library's own (the
 *   C-Kernel-Engine page calls an unpack routine whose body it does not
 *   show). llama.cpp-style Q4_K blocks store the high bits of the scales and
 *   mins of sub-blocks 4..7 differently, so such blocks cannot be exchanged
 *   with these: repack them with q4k_quantize_weights from float weights.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,     /* a required pointer is NULL */
    Q4_ERR_DIM = 2,      /* M, N or K out of range (<= 0, or an entry point's limit) */
    Q4_ERR_BLOCK = 3,    /* K not a multiple of the block size, or block size invalid for the format */
    Q4_ERR_FORMAT = 4,   /* unknown format or dtype, or a code width the entry point does not decode */
    Q4_ERR_ALIGN = 5,    /* a pointer is not aligned as its argument requires */
    Q4_ERR_HIP = 6,      /* a kernel launch failed */
    Q4_ERR_RANGE = 7,    /* row range [m0, m1) outside [0, M] or empty */
    Q4_ERR_SCRATCH = 8   /* the call needs more scratch than the library's static per-device buffer (16 MiB) */
} q4_status;

enum { Q4_DT_F32 = 0, Q4_DT_BF16 = 1 };
enum {
    Q4_FMT_Q4_0 = 0,     /* bs = 32; wscale fp16 [N][K/32]; wbias unused (may be NULL) */
    Q4_FMT_AFFINE = 1    /* bs = g in {64, 128}; wscale, wbias bf16 [N][K/g] */
};
enum { Q4_PATH_GEMV = 0, Q4_PATH_GEMM = 1, Q4_PATH_SMALL = 2 };

/*
 * Per-block int8 quantization of activations (tract PR #2432: "activation ->
 * int8, per-block"; MLX PR #4802: "x is quantized to int8").
 * For every row m and block b of bs consecutive k:
 *   amax = max |x|;  xs = amax / 127 (float32, correctly rounded);
 *   xq = clamp(round_half_even(x / xs), -127, 127) with a correctly rounded
 *   float32 quotient (all codes 0 and xs = 0 when amax == 0);
 *   xsum = sum of the block's codes.
 * x     [M][K], float32 (xdtype Q4_DT_F32) or bfloat16 (Q4_DT_BF16); 16-byte aligned.
 * xq    [M][K] int8, 16-byte aligned.   xs [M][K/bs] float32.   xsum [M][K/bs] int32.
 * bs in {32, 64, 128}.
 */
int q4_quantize_act(int M, int K, int bs, int xdtype, const void* x,
                     int8_t* xq, float* xs, int32_t* xsum, void* stream);

/*
 * Decode GEMV (M must be 1): y[n] = sum over blocks b of the rescaled exact
 * integer dot of weight row n with the int8 activation codes.
 *   Q4_0:   y += d[n,b] * xs[b] * sum_{k in b} (q - 8) * xq
 *   affine: y += xs[g] * (s[n,g] * sum_{k in g} q * xq + b[n,g] * xsum[g])
 * The weight codes are streamed with 128-bit loads and the dots use the
 * int8 dot-product instruction; one wavefront reduces each output.
 * wq [N][K/2] (16-byte aligned), wscale/wbias as in the format enum,
 * xq [1][K] (16-byte aligned), xs, xsum [1][K/bs] from q4_quantize_act,
 * y [1][N] float32. K <= 32768 (the activation codes are staged in LDS).
 */
int q4_gemv(int M, int K, int N, int bs, int fmt, int bits,
            const uint8_t* wq, const void* wscale, const void* wbias,
            const int8_t* xq, const float* xs, const int32_t* xsum,
            float* y, void* stream);

/*
 * Fused decode step (M must be 1): q4_quantize_act of x followed by q4_gemv,
 * in one launch. Every workgroup quantizes x into LDS while its weight loads
 * are in flight (tract PR #2432 measures the per-call activation
 * re-quantization as overhead of the decode op; here it costs no extra pass
 * over memory and no extra launch). The codes are bit-identical to those of
 * q4_quantize_act. x [1][K] float32 or bfloat16 (xdtype), 16-byte aligned.
 * xq_out [1][K], xs_out, xsum_out [1][K/bs]: either all NULL or all set; when
 * set they receive the activation codes the kernel used (xq_out 16-byte
 * aligned). Other arguments as q4_gemv.
 */
int q4_gemv_fused(int M, int K, int N, int bs, int fmt, int bits, int xdtype, const void* x,
                  const uint8_t* wq, const void* wscale, const void* wbias, float* y,
                  int8_t* xq_out, float* xs_out, int32_t* xsum_out, void* stream);

/*
 * Prefill GEMM, any M >= 1: Y[m][n] as q4_gemv for every row m, computed on
 * the int8 matrix cores (int32 accumulation within a block or group, float
 * rescale per block). Same arguments as q4_gemv with xq [M][K], xs, xsum
 * [M][K/bs], y [M][N]; affine codes may be 4, 6 or 8 bits (bits; 8-bit codes
 * enter the matrix cores as q - 128 with 128*s folded into the bias term).
 * M*K and N*K*bits/8 must be below 2^31.
 * Four kernels, chosen by M, N (and the code width):
 *   M <= 2 with 4-bit codes: the decode GEMV's weight stream, each weight
 *     chunk unpacked once and dotted (v_dot4) with the codes of every row,
 *     which are held in registers.
 *   3 <= M <= 32 with 4-bit codes: the same kind of weight stream on the
 *     int8 matrix cores: a workgroup of 16 wavefronts (8 above 16 rows) owns
 *     16 weight rows, its wavefronts take 128-weight stretches of them in
 *     turn, and each 32-weight block is one 16x16x32 int8 MFMA per 16
 *     activation rows.
 *     Its float rescale uses the same exponent bias as the tiled kernel
 *     below (|weight scale| < 2^104).
 *   other M <= 32, and 33 <= M <= 64 with N <= 8192: every weight block is
 *     read once for all rows (16x16x32 int8 MFMA on one, two or four 16-row
 *     tiles, 16 output columns per workgroup, K chunks staged in LDS and
 *     split over its wavefronts; each workgroup reads all M x K activation
 *     codes, which is why wide N goes to the tiled kernel above 32 rows).
 *     tract PR #2432 measures decode-sized products as weight streams; MLX
 *     PR #4802 leaves its int8 path below M = 32.
 *   otherwise: 128 x 128 output tiles on 32x32x32 int8 MFMA, one 32-weight
 *     block per K step. For 4- and 6-bit codes this kernel takes each
 *     block's integer sum into float through an exponent bias, which needs
 *     |weight scale| < 2^104 (d * 1.5 * 2^23 must stay finite); larger
 *     scales give infinities instead of the finite result.
 */
int q4_gemm(int M, int K, int N, int bs, int fmt, int bits,
            const uint8_t* wq, const void* wscale, const void* wbias,
            const int8_t* xq, const float* xs, const int32_t* xsum,
            float* y, void* stream);

/*
 * Debug view of the exact integer partials computed inside q4_gemv
 * (path Q4_PATH_GEMV, needs M == 1) or q4_gemm (Q4_PATH_GEMM: the tiled
 * kernel, any row count; Q4_PATH_SMALL: the few-row kernels, which q4_gemm
 * takes as described there, for m1 - m0 <= 64 rows at any N, else
 * Q4_ERR_RANGE): the same kernels at the same launch shapes, compiled with
 * the partials store in place of the float epilogue. The tiled kernel's
 * integer chains start from the same exponent bias as in q4_gemm (the bits
 * of 1.5 * 2^23 for 4- and 6-bit codes) and report the chain's integer minus
 * that start value.
 * partials [(m1-m0)][N][K/bs] int32 for rows m0 <= m < m1:
 *   Q4_0:   sum_{k in b} (q - 8) * xq[m][k]
 *   affine: sum_{k in g} q * xq[m][k]
 * xsum is read by the Q4_0 GEMV (which forms sum q*xq - 8*xsum); it must be
 * the xsum of xq.
 */
int q4_debug_partials(int path, int M, int K, int N, int bs, int fmt, int bits,
                      const uint8_t* wq, const int8_t* xq, const int32_t* xsum,
                      int m0, int m1, int32_t* partials, void* stream);

/*
 * Debug view of the exact integer partials inside q4_gemv_fused: the fused
 * decode kernel itself (every workgroup quantizes x into LDS and dots the
 * weight codes against its own copy of the codes), compiled with the partials
 * store in place of the float epilogue (tract PR #2432, "The kernel": the
 * integer dot of every block is exact). x [1][K] float32 or bfloat16 (xdtype),
 * 16-byte aligned; wq as q4_gemv; partials [N][K/bs] int32 as
 * q4_debug_partials (Q4_0: sum (q - 8) * xq; affine: sum q * xq), where xq are
 * the codes q4_quantize_act gives for x. K <= 32768.
 */
int q4_debug_partials_fused(int K, int N, int bs, int fmt, int bits, int xdtype, const void* x,
                            const uint8_t* wq, int32_t* partials, void* stream);

/*
 * Q4_K fused-dequant GEMV (M must be 1) and GEMM (any M >= 1) with float32
 * activations (C-Kernel-Engine gemm_kernels_q4k.c: gemv_q4_k_ref computes
 * sum_k (d*sc*q - dmin*m) * x per output row; gemm_q4_k_ref is one GEMV per
 * activation row). Dequantized weights live only in registers. q4k_gemm
 * takes sum_k q * x per 32-weight sub-block on the f16 matrix cores: codes
 * are exact f16, activations enter as two f16 halves of x scaled by a power
 * of two per row and 256-weight super-block, so the result is the float32
 * one up to rounding (for finite activations; a row whose largest magnitude
 * in a super-block is below 2^-112 loses relative precision there).
 * blocks [N][K/256] x 144 bytes (16-byte aligned), x [M][K] float32
 * (16-byte aligned), y [M][N] float32. K must be a multiple of 256. The
 * kernels address blocks and x with 32-bit byte offsets: N*(K/256)*144 and
 * 4*M*K must be below 2^31 (else Q4_ERR_DIM).
 */
int q4k_gemv(int M, int K, int N, const void* blocks, const float* x, float* y,
             void* stream);
int q4k_gemm(int M, int K, int N, const void* blocks, const float* x, float* y,
             void* stream);

/*
 * q4k_gemm with a caller workspace: the activations are split into the f16
 * halves the matrix cores take (with the per-row, per-super-block power of
 * two, the sub-block sums and the inverse scales) once per call by a first
 * launch, and the GEMM copies the split tiles instead of forming them in
 * every workgroup. Same arithmetic and results as q4k_gemm (bit-identical).
 * work: caller-owned, 16-byte aligned, q4k_gemm_work_bytes(M, K) bytes
 * (17 KB per 16 activation rows and 256 columns of K; 0 for invalid shapes);
 * it holds the split tiles when the stream completes. Two launches on stream.
 */
size_t q4k_gemm_work_bytes(int M, int K);
int q4k_gemm_work(int M, int K, int N, const void* blocks, const float* x, float* y,
                  void* work, void* stream);

/*
 * Weight quantization on the GPU (model preparation, not the hot path).
 * q4_quantize_weights: w [N][K] float32 or bfloat16 (wdtype) ->
 *   Q4_0 (bs 32):  i = first index of the largest |w| in the block,
 *                  d = fp16(w[i] / -8), q = clamp(round_half_even(w / d) + 8, 0, 15)
 *                  (q = 8 when d == 0);
 *   affine (bs g): s = bf16((max - min) / (2^bits - 1)), b = bf16(min),
 *                  q = clamp(round_half_even((w - b) / s), 0, 2^bits - 1) (q = 0 when s == 0),
 *                  bits 4, 6 or 8 (codes in the layout above);
 *   every step in float32. wq as above (16-byte aligned); wscale, wbias as in
 *   the format enum (wbias unused for Q4_0).
 * q4k_quantize_weights: w [N][K] float32 -> Q4_K blocks. For each 32-weight
 *   sub-block: lo = min(0, min w), hi = max w, a = (hi - lo) / 15, c = -lo;
 *   d = fp16(max a / 63), dmin = fp16(max c / 63); sc = round_half_even(a / d),
 *   m = round_half_even(c / dmin), clamped to 0..63 (0 when the divisor is 0);
 *   q = clamp(round_half_even((w + dmin*m) / (d*sc)), 0, 15) (0 when d*sc == 0).
 */
int q4_quantize_weights(int N, int K, int bs, int fmt, int bits, int wdtype,
                        const void* w, uint8_t* wq, void* wscale, void* wbias,
                        void* stream);
int q4k_quantize_weights(int N, int K, const float* w, void* blocks, void* stream);

/*
 * Weight pre-pack for the tiled GEMM, and the fused quantize + GEMM on packed
 * weights (tract PR #2432, production direction: a pre-packed weight layout
 * and fusing the activation quantization into the matmul remove per-call
 * overhead). The arithmetic is that of q4_quantize_act followed by q4_gemm.
 *
 * Packed layout, T = ceil(N/128) column tiles, S = ceil(K/128) K stages,
 * ng = K/bs groups, three sections back to back:
 *   codes   T*S blocks of 8192 bytes; block (t, s) holds, for r = 0..127 at
 *           offset 64*r, bytes 64*s .. 64*s + 63 of row 128*t + r of wq (the
 *           codes of that row's weights 128*s .. 128*s + 127); rows past N
 *           and bytes past K/2 are zero.
 *   scales  T*ng*128 16-bit values, (t, g, r) at index (t*ng + g)*128 + r:
 *           wscale[128*t + r][g], zero for rows past N.
 *   biases  (affine only) the same from wbias.
 * q4_packed_bytes returns the size (0 for invalid arguments; the code and
 * scale sections must each be below 2^31 bytes). q4_pack_weights writes the
 * packed buffer (16-byte aligned, caller-owned) from wq, wscale, wbias as
 * q4_quantize_weights makes them.
 *
 * q4_gemm_packed: x [M][K] float32 or bfloat16 (xdtype, 16-byte aligned),
 * packed as above, y [M][N] float32. work: caller-owned scratch of
 * q4_gemm_packed_work_bytes(M, K, bs) bytes (16-byte aligned). After the
 * stream completes, work holds the activation codes used: xq [M][K] at
 * offset 0, then at offset A = align256(M*K) xs as [K/bs][M] float32
 * (group-major, the transpose of q4_quantize_act's xs), then at offset
 * A + align256(4*M*K/bs) xsum as [K/bs][M] int32. Two launches on stream:
 * the quantizer, then the tiled 32x32x32 int8 MFMA GEMM (for every M),
 * with the weight-scale limit stated at q4_gemm. M*K must be below 2^31.
 */
size_t q4_packed_bytes(int K, int N, int bs, int fmt);
int q4_pack_weights(int N, int K, int bs, int fmt, int bits, const uint8_t* wq,
                    const void* wscale, const void* wbias, uint8_t* packed, void* stream);
size_t q4_gemm_packed_work_bytes(int M, int K, int bs);
int q4_gemm_packed(int M, int K, int N, int bs, int fmt, int bits, int xdtype, const void* x,
                   const uint8_t* packed, float* y, void* work, void* stream);

/*
 * Input gradient with frozen weights (C-Kernel-Engine gemm_kernels_q4k.c,
 * section "Backward Pass: Gradient w.r.t. Input": dL/dX = W^T . dL/dY with the
 * weights dequantized on the fly, no weight gradient; the batched form is one
 * such product per activation row). With W [N][K] as in the forward calls:
 *   dx[m][k] = sum_n dy[m][n] * w^[n][k],  dy [M][N], dx [M][K] float32,
 * w^ the dequantized weight (Q4_K: d*sc*q - dmin*m; Q4_0: d*(q - 8);
 * affine: s*q + b). K must be a multiple of 256 (else Q4_ERR_BLOCK).
 * work: caller-owned scratch of q4_backward_work_bytes(M, K, N) bytes
 * (4-byte aligned) for per-row-range partial sums, which a second launch adds
 * in a fixed order (results do not depend on scheduling).
 * q4_backward_work_bytes returns 0 for invalid shapes.
 */
size_t q4_backward_work_bytes(int M, int K, int N);
int q4k_gemm_backward(int M, int K, int N, const void* blocks, const float* dy, float* dx,
                      void* work, void* stream);
int q4_gemm_backward(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq,
                     const void* wscale, const void* wbias, const float* dy, float* dx,
                     void* work, void* stream);

/*
 * q4k_gemm_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The partial sums live in a static
 * device buffer of the library, one per GPU, of 16 MiB (16777216 bytes),
 * held until the process ends; the call allocates nothing. A shape
 * whose q4_backward_work_bytes(M, K, N) exceeds the capacity is rejected with
 * Q4_ERR_SCRATCH before any launch (at K = 4096 and N = 14336 every M up to
 * 256 fits). Calls on one GPU share its buffer: calls that overlap on one GPU
 * (other streams or host threads) race and must be serialized by the caller.
 * Other arguments, results and errors as q4k_gemm_backward.
 */
int q4k_gemm_backward_noalloc(int M, int K, int N, const void* blocks, const float* dy, float* dx,
                              void* stream);

/* Static name of a q4_status value ("unknown status" otherwise). */
const char* q4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
