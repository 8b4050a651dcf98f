// Input gradient with frozen Q4_K weights for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid allocation): the per-range partial sums that q4k_gemm_backward keeps
// in a caller workspace live here in a static device array instead.
//
// The array is one per GPU the library runs on, held until the process ends.
// Its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; the kernels receive that address as their
// workspace argument. Every call on one GPU shares the array, so calls that
// overlap on one GPU (different streams, or different host threads) race.
// Nothing in it must start at zero: the range kernels write every element
// the reduction reads.
#include <mutex>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "q4.h"

namespace {

constexpr size_t SCRATCH_BYTES = size_t(16) << 20;  // 16 MiB per device
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) float scratch[SCRATCH_BYTES / sizeof(float)];

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[MAX_DEVICES];

// Device address of this device's copy of `scratch` (nullptr on failure).
void* scratch_ptr(int dev) {
    DeviceScratch& s = g_scratch[dev];
    std::call_once(s.once, [&] {
        void* p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s.err == hipSuccess) s.ptr = p;
    });
    return s.ptr;
}

}  // namespace

extern "C" int q4k_gemm_backward_noalloc(int M, int K, int N, const void* blocks, const float* dy, float* dx,
                                         void* stream) {
    const size_t need = q4_backward_work_bytes(M, K, N);
    if (need == 0) return q4k_gemm_backward(M, K, N, blocks, dy, dx, nullptr, stream);  // the shape's status
    if (need > SCRATCH_BYTES) return Q4_ERR_SCRATCH;
    if (!blocks || !dy || !dx) return Q4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(blocks) % 16 || reinterpret_cast<uintptr_t>(dy) % 4 ||
        reinterpret_cast<uintptr_t>(dx) % 4)
        return Q4_ERR_ALIGN;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return Q4_ERR_HIP;
    float* work = static_cast<float*>(scratch_ptr(dev));
    if (!work) return Q4_ERR_HIP;
    return q4k_gemm_backward(M, K, N, blocks, dy, dx, work, stream);
}
