// kda_util.hip -- small fill / copy kernels for the empty-sequence path (kernels rather
// than hipMemsetAsync / hipMemcpyAsync so that a caller may capture the call in a HIP
// graph), and the compute-unit count that sizes the persistent grids.
#include <atomic>

#include "kda_internal.h"

namespace kda {

namespace {

__global__ __launch_bounds__(256) void fill_copy_kernel(float *dst, const float *src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

int device_cu_count() {
    // per device, filled on first use; threads that race to fill it store the same value
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_fill_copy(float *dst, const float *src, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace kda
