// Internal launchers of the gfx950 kernels. Arguments are validated by the
// C-ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (device, kernel, size); safe to call from several host threads.
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

hipError_t launch_quantize_act(int M, int K, int bs, bool bf16, const void* x, int8_t* xq, float* xs,
                               int32_t* xsum, hipStream_t stream);
// Same codes, with xs and xsum written group-major: [K/bs][M].
hipError_t launch_quantize_act_gm(int M, int K, int bs, bool bf16, const void* x, int8_t* xq, float* xs,
                                  int32_t* xsum, hipStream_t stream);

// fmt: 0 = Q4_0 (bs 32), 1 = affine (bs 64 / 128). partials != nullptr selects
// the integer-partials store in place of the float epilogue.
hipError_t launch_gemv(int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale, const void* wbias,
                       const int8_t* xq, const float* xs, const int32_t* xsum, float* y, int32_t* partials,
                       hipStream_t stream);

// Decode GEMV that quantizes x itself; the optional *_out pointers receive the
// activation codes it used (written by one workgroup).
hipError_t launch_gemv_fused(int K, int N, int bs, int fmt, bool xbf16, const void* x, const uint8_t* wq,
                             const void* wscale, const void* wbias, float* y, int8_t* xq_out, float* xs_out,
                             int32_t* xsum_out, hipStream_t stream);
// The same fused kernel with the integer-partials store in place of the float
// epilogue (partials [N][K/bs], from the codes the kernel quantizes itself).
hipError_t launch_gemv_fused_partials(int K, int N, int bs, int fmt, bool xbf16, const void* x, const uint8_t* wq,
                                      int32_t* partials, hipStream_t stream);

// bits: code width of affine weights (4, 6 or 8; Q4_0 is 4-bit only).
hipError_t launch_gemm(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                       const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                       int32_t* partials, hipStream_t stream);

// Few-row GEMM (1 <= M <= GEMM_SMALL_MAX_M): every weight block is read once
// for all rows (16x16x32 int8 MFMA, K chunks staged in LDS and split over the
// wavefronts of a workgroup). Same arguments as launch_gemm.
constexpr int GEMM_SMALL_MAX_M = 64;
// Which kernel q4_gemm takes: the few-row kernel up to 32 rows, and up to 64
// rows while N <= 8192. Each of its workgroups (16 columns) reads all M x K
// activation codes, so for 33..64 rows and wide N the tiled kernel is faster
// (measured at K = 4096: N = 4096 few-row 11.6-15.3 us against tiled 31-52 us;
// N = 14336 few-row 39-53 us against tiled 32-45 us).
constexpr int GEMM_SMALL_WIDE_N = 8192;
inline bool gemm_small_preferred(int M, int N) {
    return M <= 32 || (M <= GEMM_SMALL_MAX_M && N <= GEMM_SMALL_WIDE_N);
}
hipError_t launch_gemm_small(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                             const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                             int32_t* partials, hipStream_t stream);

// Few-row GEMV (1 <= M <= GEMV_ROWS_MAX_M, 4-bit codes): the decode GEMV's
// weight stream with the activation codes of all rows in registers. Taken by
// launch_gemm_small where gemv_rows_fits (Q4_0 at M = 2, cold weights: 4.7 us
// at 4096 x 4096, 9.7 us at N = 14336, 10.8 us at K = 14336, against 4.9,
// 12.1 and 13.2 us for the matrix-core kernel below; from 3 rows on that one
// is as fast or faster). Same arguments as launch_gemm.
constexpr int GEMV_ROWS_MAX_M = 2;
bool gemv_rows_fits(int M, int K, int bits);
hipError_t launch_gemv_rows(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                            const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                            int32_t* partials, hipStream_t stream);

// Few-row product on the int8 matrix cores with the decode GEMV's weight
// stream (rows_mfma.hip): 4-bit Q4_0 or affine codes, M <= ROWS_MFMA_MAX_M,
// a workgroup of 16 wavefronts per 16 weight rows. launch_gemm_small takes it
// for GEMV_ROWS_MAX_M < M <= ROWS_MFMA_MAX_M. Same arguments as launch_gemm.
constexpr int ROWS_MFMA_MAX_M = 32;
bool rows_mfma_fits(int M, int K, int bs, int fmt, int bits);
hipError_t launch_rows_mfma(int M, int K, int N, int bs, int fmt, const uint8_t* wq, const void* wscale,
                            const void* wbias, const int8_t* xq, const float* xs, const int32_t* xsum, float* y,
                            int32_t* partials, hipStream_t stream);


// Packed weights for the tiled GEMM (layout in include/q4.h, q4_pack_weights).
size_t packed_code_bytes(int K, int N);
size_t packed_scale_bytes(int K, int N, int bs);
hipError_t launch_pack_weights(int N, int K, int bs, int fmt, const uint8_t* wq, const void* wscale,
                               const void* wbias, uint8_t* packed, hipStream_t stream);
// Tiled GEMM on packed weights with group-major activation scales ([K/bs][M]).
hipError_t launch_gemm_packed(int M, int K, int N, int bs, int fmt, const uint8_t* packed, const int8_t* xq,
                              const float* xs_gm, const int32_t* xsum_gm, float* y, hipStream_t stream);

// Input gradient with frozen weights, dx = dy . dequant(W); fmt 0 Q4_0, 1 affine
// (bs 64 / 128), 2 Q4_K. K % 256 == 0. work: backward_ranges(M, K, N) * M * K floats.
// Up to BWD_ROWS_MAX_M rows take the weight-stream kernel, more rows the
// matrix-core kernel.
constexpr int BWD_ROWS_MAX_M = 4;
int backward_ranges(int M, int K, int N);
hipError_t launch_backward(int M, int K, int N, int fmt, int bs, const uint8_t* w, const void* wscale,
                           const void* wbias, const float* dy, float* dx, float* work, hipStream_t stream);

hipError_t launch_q4k_gemv(int K, int N, const void* blocks, const float* x, float* y, hipStream_t stream);
hipError_t launch_q4k_gemm(int M, int K, int N, const void* blocks, const float* x, float* y, hipStream_t stream);
// q4k_gemm with the activations split once per call into a workspace of
// q4k_gemm_work_bytes(M, K) bytes (a split kernel, then the GEMM copying the
// split tiles instead of forming them in every workgroup).
size_t q4k_gemm_work_bytes(int M, int K);
hipError_t launch_q4k_gemm_work(int M, int K, int N, const void* blocks, const float* x, float* y, void* work,
                                hipStream_t stream);

hipError_t launch_quantize_weights(int N, int K, int bs, int fmt, int bits, bool bf16, const void* w, uint8_t* wq,
                                   void* wscale, void* wbias, hipStream_t stream);
hipError_t launch_q4k_quantize_weights(int N, int K, const float* w, void* blocks, hipStream_t stream);

}  // namespace q4
