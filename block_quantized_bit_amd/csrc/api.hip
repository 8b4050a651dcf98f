// C-ABI entry points: host-side argument validation, then kernel launches.
// Validation is pure host code and runs before any HIP call, so an invalid
// call returns its status without touching the device.
#include <stdint.h>

#include <mutex>
#include <set>
#include <tuple>

#include "q4.h"
#include "kernels.h"

namespace q4 {

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
    static std::mutex mu;
    static std::set<std::tuple<int, const void*, size_t>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const auto key = std::make_tuple(dev, kernel, bytes);
    std::lock_guard<std::mutex> lock(mu);
    if (done.count(key)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done.insert(key);
    return e;
}

}  // namespace q4

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int block_status(int K, int bs, int fmt) {
    if (fmt == Q4_FMT_Q4_0) {
        if (bs != 32) return Q4_ERR_BLOCK;
    } else if (fmt == Q4_FMT_AFFINE) {
        if (bs != 64 && bs != 128) return Q4_ERR_BLOCK;
    } else {
        return Q4_ERR_FORMAT;
    }
    if (K % bs != 0) return Q4_ERR_BLOCK;
    return Q4_OK;
}

// Code widths: Q4_0 is 4-bit only; affine codes may be 4, 6 or 8 bits wide
// (MLX PR #4802) where an entry point decodes them. A decoder handed a width
// it does not decode must refuse it rather than misread the bytes (meTile
// PR #29: a four-bit decoder fed eight-bit data fails silently).
bool bits_ok(int fmt, int bits, bool wide_ok) {
    if (bits == 4) return true;
    return wide_ok && fmt == Q4_FMT_AFFINE && (bits == 6 || bits == 8);
}

// Common checks of the W4A8 matmul entry points (pointers checked by callers).
// wide_ok: the entry point decodes 6- and 8-bit affine codes.
int matmul_status(int M, int K, int N, int bs, int fmt, int bits, bool wide_ok = false) {
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE) return Q4_ERR_FORMAT;
    if (!bits_ok(fmt, bits, wide_ok)) return Q4_ERR_FORMAT;
    if (M <= 0 || N <= 0 || K <= 0) return Q4_ERR_DIM;
    return block_status(K, bs, fmt);
}

int hip_status(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_HIP; }

constexpr int Q4_GEMV_MAX_K = 32768;  // activation codes staged in LDS

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Status of a packed-weight shape: the tiled layout is addressed with 32-bit offsets.
int packed_status(int K, int N, int bs, int fmt) {
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE) return Q4_ERR_FORMAT;
    if (N <= 0 || K <= 0) return Q4_ERR_DIM;
    int st = block_status(K, bs, fmt);
    if (st) return st;
    if (q4::packed_code_bytes(K, N) >= (1ull << 31) || q4::packed_scale_bytes(K, N, bs) >= (1ull << 31))
        return Q4_ERR_DIM;
    return Q4_OK;
}

}  // namespace

extern "C" {

const char* q4_status_string(int status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_ERR_NULL: return "a required pointer is NULL";
        case Q4_ERR_DIM: return "M, N or K out of range";
        case Q4_ERR_BLOCK: return "K is not a multiple of the block size, or the block size is invalid for the format";
        case Q4_ERR_FORMAT: return "unknown format or dtype, or a bit width other than 4 (these kernels decode two 4-bit codes per byte)";
        case Q4_ERR_ALIGN: return "a pointer is not aligned as its argument requires";
        case Q4_ERR_HIP: return "a kernel launch failed";
        case Q4_ERR_RANGE: return "row range [m0, m1) is empty or outside [0, M]";
        case Q4_ERR_SCRATCH: return "the call needs more scratch memory than the library's static per-device buffer (16 MiB); use the entry point that takes a workspace";
        default: return "unknown status";
    }
}

int q4_quantize_act(int M, int K, int bs, int xdtype, const void* x, int8_t* xq, float* xs, int32_t* xsum,
                    void* stream) {
    if (!x || !xq || !xs || !xsum) return Q4_ERR_NULL;
    if (xdtype != Q4_DT_F32 && xdtype != Q4_DT_BF16) return Q4_ERR_FORMAT;
    if (M <= 0 || K <= 0) return Q4_ERR_DIM;
    if ((bs != 32 && bs != 64 && bs != 128) || K % bs != 0) return Q4_ERR_BLOCK;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xs, 4) || !aligned(xsum, 4)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_quantize_act(M, K, bs, xdtype == Q4_DT_BF16, x, xq, xs, xsum,
                                              static_cast<hipStream_t>(stream)));
}

static int check_matmul_ptrs(int fmt, const uint8_t* wq, const void* wscale, const void* wbias, const int8_t* xq,
                             const float* xs, const int32_t* xsum, const void* out) {
    if (!wq || !wscale || !xq || !xs || !xsum || !out) return Q4_ERR_NULL;
    if (fmt == Q4_FMT_AFFINE && !wbias) return Q4_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(wscale, 2) || (wbias && !aligned(wbias, 2)) ||
        !aligned(xs, 4) || !aligned(xsum, 4) || !aligned(out, 4))
        return Q4_ERR_ALIGN;
    return Q4_OK;
}

int q4_gemv(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale, const void* wbias,
            const int8_t* xq, const float* xs, const int32_t* xsum, float* y, void* stream) {
    int st = matmul_status(M, K, N, bs, fmt, bits);
    if (st) return st;
    if (M != 1 || K > Q4_GEMV_MAX_K) return Q4_ERR_DIM;
    st = check_matmul_ptrs(fmt, wq, wscale, wbias, xq, xs, xsum, y);
    if (st) return st;
    return hip_status(q4::launch_gemv(K, N, bs, fmt, wq, wscale, wbias, xq, xs, xsum, y, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int q4_gemv_fused(int M, int K, int N, int bs, int fmt, int bits, int xdtype, const void* x, const uint8_t* wq,
                  const void* wscale, const void* wbias, float* y, int8_t* xq_out, float* xs_out, int32_t* xsum_out,
                  void* stream) {
    int st = matmul_status(M, K, N, bs, fmt, bits);
    if (st) return st;
    if (xdtype != Q4_DT_F32 && xdtype != Q4_DT_BF16) return Q4_ERR_FORMAT;
    if (M != 1 || K > Q4_GEMV_MAX_K) return Q4_ERR_DIM;
    if (!x || !wq || !wscale || !y || (fmt == Q4_FMT_AFFINE && !wbias)) return Q4_ERR_NULL;
    const bool any_out = xq_out || xs_out || xsum_out;
    if (any_out && !(xq_out && xs_out && xsum_out)) return Q4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(wscale, 2) || (wbias && !aligned(wbias, 2)) ||
        !aligned(y, 4) || (any_out && (!aligned(xq_out, 16) || !aligned(xs_out, 4) || !aligned(xsum_out, 4))))
        return Q4_ERR_ALIGN;
    return hip_status(q4::launch_gemv_fused(K, N, bs, fmt, xdtype == Q4_DT_BF16, x, wq, wscale, wbias, y, xq_out,
                                            xs_out, xsum_out, static_cast<hipStream_t>(stream)));
}

int q4_gemm(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale, const void* wbias,
            const int8_t* xq, const float* xs, const int32_t* xsum, float* y, void* stream) {
    int st = matmul_status(M, K, N, bs, fmt, bits, true);
    if (st) return st;
    // buffer loads address each operand with 32-bit byte offsets
    if ((long long)M * K >= (1LL << 31) || (long long)N * K * bits / 8 >= (1LL << 31)) return Q4_ERR_DIM;
    st = check_matmul_ptrs(fmt, wq, wscale, wbias, xq, xs, xsum, y);
    if (st) return st;
    // a few rows: stream every weight block once for all of them
    if (q4::gemm_small_preferred(M, N))
        return hip_status(q4::launch_gemm_small(M, K, N, bs, fmt, bits, wq, wscale, wbias, xq, xs, xsum, y, nullptr,
                                                static_cast<hipStream_t>(stream)));
    return hip_status(q4::launch_gemm(M, K, N, bs, fmt, bits, wq, wscale, wbias, xq, xs, xsum, y, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int q4_debug_partials(int path, int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const int8_t* xq,
                      const int32_t* xsum, int m0, int m1, int32_t* partials, void* stream) {
    int st = matmul_status(M, K, N, bs, fmt, bits, path != Q4_PATH_GEMV);
    if (st) return st;
    if (path != Q4_PATH_GEMV && path != Q4_PATH_GEMM && path != Q4_PATH_SMALL) return Q4_ERR_FORMAT;
    if (!wq || !xq || !xsum || !partials) return Q4_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(xq, 16) || !aligned(xsum, 4) || !aligned(partials, 4)) return Q4_ERR_ALIGN;
    if (m0 < 0 || m1 > M || m0 >= m1) return Q4_ERR_RANGE;
    if ((long long)(m1 - m0) * K >= (1LL << 31) || (long long)N * K * bits / 8 >= (1LL << 31)) return Q4_ERR_DIM;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int ng = K / bs;
    const int8_t* xq0 = xq + (size_t)m0 * K;
    const int32_t* xsum0 = xsum + (size_t)m0 * ng;
    if (path == Q4_PATH_GEMV) {
        if (m1 - m0 != 1) return Q4_ERR_RANGE;
        if (K > Q4_GEMV_MAX_K) return Q4_ERR_DIM;
        return hip_status(q4::launch_gemv(K, N, bs, fmt, wq, nullptr, nullptr, xq0, nullptr, xsum0, nullptr,
                                          partials, s));
    }
    if (path == Q4_PATH_SMALL) {
        if (m1 - m0 > q4::GEMM_SMALL_MAX_M) return Q4_ERR_RANGE;
        return hip_status(q4::launch_gemm_small(m1 - m0, K, N, bs, fmt, bits, wq, nullptr, nullptr, xq0, nullptr,
                                                xsum0, nullptr, partials, s));
    }
    return hip_status(q4::launch_gemm(m1 - m0, K, N, bs, fmt, bits, wq, nullptr, nullptr, xq0, nullptr, xsum0,
                                      nullptr, partials, s));
}

int q4_debug_partials_fused(int K, int N, int bs, int fmt, int bits, int xdtype, const void* x, const uint8_t* wq,
                            int32_t* partials, void* stream) {
    int st = matmul_status(1, K, N, bs, fmt, bits);
    if (st) return st;
    if (xdtype != Q4_DT_F32 && xdtype != Q4_DT_BF16) return Q4_ERR_FORMAT;
    if (K > Q4_GEMV_MAX_K) return Q4_ERR_DIM;
    if (!x || !wq || !partials) return Q4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(partials, 4)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_gemv_fused_partials(K, N, bs, fmt, xdtype == Q4_DT_BF16, x, wq, partials,
                                                     static_cast<hipStream_t>(stream)));
}

size_t q4_packed_bytes(int K, int N, int bs, int fmt) {
    if (packed_status(K, N, bs, fmt)) return 0;
    return q4::packed_code_bytes(K, N) + q4::packed_scale_bytes(K, N, bs) * (fmt == Q4_FMT_AFFINE ? 2 : 1);
}

int q4_pack_weights(int N, int K, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                    const void* wbias, uint8_t* packed, void* stream) {
    if (bits != 4) return Q4_ERR_FORMAT;
    int st = packed_status(K, N, bs, fmt);
    if (st) return st;
    if (!wq || !wscale || !packed || (fmt == Q4_FMT_AFFINE && !wbias)) return Q4_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(wscale, 2) || (wbias && !aligned(wbias, 2)) || !aligned(packed, 16))
        return Q4_ERR_ALIGN;
    return hip_status(q4::launch_pack_weights(N, K, bs, fmt, wq, wscale, wbias, packed,
                                              static_cast<hipStream_t>(stream)));
}

size_t q4_gemm_packed_work_bytes(int M, int K, int bs) {
    if (M <= 0 || K <= 0 || (bs != 32 && bs != 64 && bs != 128) || K % bs != 0) return 0;
    return align256((size_t)M * K) + 2 * align256((size_t)M * (K / bs) * 4);
}

int q4_gemm_packed(int M, int K, int N, int bs, int fmt, int bits, int xdtype, const void* x,
                   const uint8_t* packed, float* y, void* work, void* stream) {
    int st = matmul_status(M, K, N, bs, fmt, bits);
    if (st) return st;
    if (xdtype != Q4_DT_F32 && xdtype != Q4_DT_BF16) return Q4_ERR_FORMAT;
    st = packed_status(K, N, bs, fmt);
    if (st) return st;
    if ((long long)M * K >= (1LL << 31)) return Q4_ERR_DIM;
    if (!x || !packed || !y || !work) return Q4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 4) || !aligned(work, 16)) return Q4_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    int8_t* xq = static_cast<int8_t*>(work);
    float* xs = reinterpret_cast<float*>(static_cast<uint8_t*>(work) + align256((size_t)M * K));
    int32_t* xsum = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(xs) + align256((size_t)M * (K / bs) * 4));
    st = hip_status(q4::launch_quantize_act_gm(M, K, bs, xdtype == Q4_DT_BF16, x, xq, xs, xsum, s));
    if (st) return st;
    return hip_status(q4::launch_gemm_packed(M, K, N, bs, fmt, packed, xq, xs, xsum, y, s));
}

// Shapes of the input-gradient entry points: K a multiple of 256, 32-bit buffer offsets.
static int backward_shape(int M, int K, int N, int fmt) {
    if (M <= 0 || N <= 0 || K <= 0) return Q4_ERR_DIM;
    if (K % 256 != 0) return Q4_ERR_BLOCK;
    const long long wbytes = fmt == 2 ? (long long)N * (K / 256) * 144 : (long long)N * (K / 2);
    if (wbytes >= (1LL << 31) || (long long)M * N * 4 >= (1LL << 31)) return Q4_ERR_DIM;
    return Q4_OK;
}

size_t q4_backward_work_bytes(int M, int K, int N) {
    if (backward_shape(M, K, N, 2) || backward_shape(M, K, N, 0)) return 0;
    return (size_t)q4::backward_ranges(M, K, N) * M * K * sizeof(float);
}

int q4k_gemm_backward(int M, int K, int N, const void* blocks, const float* dy, float* dx, void* work, void* stream) {
    int st = backward_shape(M, K, N, 2);
    if (st) return st;
    if (!blocks || !dy || !dx || !work) return Q4_ERR_NULL;
    if (!aligned(blocks, 16) || !aligned(dy, 4) || !aligned(dx, 4) || !aligned(work, 4)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_backward(M, K, N, 2, 256, static_cast<const uint8_t*>(blocks), nullptr, nullptr, dy,
                                          dx, static_cast<float*>(work), static_cast<hipStream_t>(stream)));
}

int q4_gemm_backward(int M, int K, int N, int bs, int fmt, int bits, const uint8_t* wq, const void* wscale,
                     const void* wbias, const float* dy, float* dx, void* work, void* stream) {
    if (bits != 4) return Q4_ERR_FORMAT;
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE) return Q4_ERR_FORMAT;
    int st = block_status(K > 0 ? K : bs, bs, fmt);
    if (st) return st;
    st = backward_shape(M, K, N, fmt);
    if (st) return st;
    if (!wq || !wscale || !dy || !dx || !work || (fmt == Q4_FMT_AFFINE && !wbias)) return Q4_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(wscale, 2) || (wbias && !aligned(wbias, 2)) || !aligned(dy, 4) ||
        !aligned(dx, 4) || !aligned(work, 4))
        return Q4_ERR_ALIGN;
    return hip_status(q4::launch_backward(M, K, N, fmt, bs, wq, wscale, wbias, dy, dx, static_cast<float*>(work),
                                          static_cast<hipStream_t>(stream)));
}

// The Q4_K kernels address blocks and x with 32-bit buffer offsets.
static bool q4k_offsets_too_large(int M, int K, int N) {
    return (long long)N * (K / 256) * 144 >= (1LL << 31) || 4LL * M * K >= (1LL << 31);
}

int q4k_gemv(int M, int K, int N, const void* blocks, const float* x, float* y, void* stream) {
    if (!blocks || !x || !y) return Q4_ERR_NULL;
    if (M != 1 || N <= 0 || K <= 0) return Q4_ERR_DIM;
    if (K % 256 != 0) return Q4_ERR_BLOCK;
    if (q4k_offsets_too_large(M, K, N)) return Q4_ERR_DIM;
    if (!aligned(blocks, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_q4k_gemv(K, N, blocks, x, y, static_cast<hipStream_t>(stream)));
}

int q4k_gemm(int M, int K, int N, const void* blocks, const float* x, float* y, void* stream) {
    if (!blocks || !x || !y) return Q4_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0 || M > (1 << 20)) return Q4_ERR_DIM;  // grid rows of 16
    if (K % 256 != 0) return Q4_ERR_BLOCK;
    if (q4k_offsets_too_large(M, K, N)) return Q4_ERR_DIM;
    if (!aligned(blocks, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_q4k_gemm(M, K, N, blocks, x, y, static_cast<hipStream_t>(stream)));
}

size_t q4k_gemm_work_bytes(int M, int K) {
    if (M <= 0 || K <= 0 || K % 256 != 0 || M > (1 << 20)) return 0;
    return q4::q4k_gemm_work_bytes(M, K);
}

int q4k_gemm_work(int M, int K, int N, const void* blocks, const float* x, float* y, void* work, void* stream) {
    if (!blocks || !x || !y || !work) return Q4_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0 || M > (1 << 20)) return Q4_ERR_DIM;
    if (K % 256 != 0) return Q4_ERR_BLOCK;
    if (q4k_offsets_too_large(M, K, N) || q4::q4k_gemm_work_bytes(M, K) >= (1ull << 31)) return Q4_ERR_DIM;
    if (!aligned(blocks, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(work, 16)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_q4k_gemm_work(M, K, N, blocks, x, y, work, static_cast<hipStream_t>(stream)));
}

int q4_quantize_weights(int N, int K, int bs, int fmt, int bits, int wdtype, const void* w, uint8_t* wq,
                        void* wscale, void* wbias, void* stream) {
    if (fmt != Q4_FMT_Q4_0 && fmt != Q4_FMT_AFFINE) return Q4_ERR_FORMAT;
    if (!bits_ok(fmt, bits, true)) return Q4_ERR_FORMAT;
    if (wdtype != Q4_DT_F32 && wdtype != Q4_DT_BF16) return Q4_ERR_FORMAT;
    if (N <= 0 || K <= 0) return Q4_ERR_DIM;
    int st = block_status(K, bs, fmt);
    if (st) return st;
    if (!w || !wq || !wscale || (fmt == Q4_FMT_AFFINE && !wbias)) return Q4_ERR_NULL;
    if (!aligned(w, wdtype == Q4_DT_F32 ? 4 : 2) || !aligned(wq, 16) || !aligned(wscale, 2) ||
        (wbias && !aligned(wbias, 2)))
        return Q4_ERR_ALIGN;
    return hip_status(q4::launch_quantize_weights(N, K, bs, fmt, bits, wdtype == Q4_DT_BF16, w, wq, wscale, wbias,
                                                  static_cast<hipStream_t>(stream)));
}

int q4k_quantize_weights(int N, int K, const float* w, void* blocks, void* stream) {
    if (!w || !blocks) return Q4_ERR_NULL;
    if (N <= 0 || K <= 0) return Q4_ERR_DIM;
    if (K % 256 != 0) return Q4_ERR_BLOCK;
    if (!aligned(w, 4) || !aligned(blocks, 16)) return Q4_ERR_ALIGN;
    return hip_status(q4::launch_q4k_quantize_weights(N, K, w, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
