// Streaming device-to-device copy with the access pattern of the decode
// kernels' code streams: 16-byte non-temporal loads and stores, one per lane,
// a grid of short workgroups.  Its bandwidth is the attainable reference the
// benchmark reports beside the decode kernel's fraction of the 8 TB/s peak,
// and a copy of known size calibrates the profiler's byte counters.
#include "pace_layout.h"

namespace pace {
namespace {

typedef uint32_t cp_u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_copy_kernel(cp_u32x4 *dst, const cp_u32x4 *src, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (cp_u32x4 *)dst,
                       (const cp_u32x4 *)src, n);
    return hipGetLastError();
}

}  // namespace pace
