// Measurement kernels: an empty kernel and a read-only stream (q4_measure.h).
// They give the dispatch floor and the streaming ceiling that the decode
// kernels are compared against on the running GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4.h"
#include "q4_measure.h"

namespace {

constexpr int RSRC_WORD3 = 0x00020000;
constexpr int NT_AUX = 2;  // non-temporal loads, as the decode GEMV's weight stream
constexpr int UNROLL = 4;  // 16-byte loads in flight per thread per iteration

__global__ void empty_kernel() {}

// Thread t of the grid reads 16-byte chunks t, t + T, t + 2T, ... (T threads in
// all), UNROLL loads in flight; chunks past the end read zero (buffer range).
__global__ void stream_read_kernel(const void* buf, uint32_t nchunks, uint32_t key, uint32_t* sink) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(buf), (short)0, (int)(nchunks * 16u), RSRC_WORD3);
    const uint32_t T = gridDim.x * blockDim.x;
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (uint32_t c = t; c < nchunks; c += UNROLL * T) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint32_t cc = c + u * T;
            v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, cc < nchunks ? cc * 16u : 0x80000000u, 0, NT_AUX));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == key) sink[0] = acc;
}

bool shape_ok(int grid, int block) { return grid > 0 && block > 0 && block <= 1024 && block % 64 == 0; }

}  // namespace

extern "C" int q4_measure_empty(int grid, int block, void* stream) {
    if (!shape_ok(grid, block)) return Q4_ERR_DIM;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}

extern "C" int q4_measure_stream_read(const void* buf, size_t bytes, int grid, int block, uint32_t key,
                                      uint32_t* sink, void* stream) {
    if (!shape_ok(grid, block)) return Q4_ERR_DIM;
    if (!buf || !sink) return Q4_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || bytes >= (1ull << 31)) return Q4_ERR_DIM;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return Q4_ERR_ALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream), buf,
                       (uint32_t)(bytes / 16), key, sink);
    return hipGetLastError() == hipSuccess ? Q4_OK : Q4_ERR_HIP;
}
