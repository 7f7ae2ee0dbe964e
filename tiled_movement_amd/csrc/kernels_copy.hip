// Reference device copy: one 16-byte non-temporal load and store per thread,
// like the tile kernels' global accesses.  It is the read-once / write-once
// bandwidth ceiling the tile kernels are compared with, and the kernel of
// known size HBM byte counters are scaled by.  The shape was picked by a
// sweep on MI355X (64 MiB: one 16-byte vector per thread at 256 threads
// 6.13 TB/s; two or four per thread 5.88-5.89; 512 or 1024 threads 6.00;
// cached accesses 5.4-5.6).
#include "launch.h"

namespace swz {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int64_t kMaxGrid = int64_t(1) << 22;  // workgroups per launch

// Vector i = first + blockIdx.x * 256 + threadIdx.x, for i < n16.
__global__ __launch_bounds__(kCopyThreads) void k_copy(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                                       int64_t n16, int64_t first) {
    const int64_t i = first + static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(&s[i]), &d[i]);
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t blocks = (n16 + kCopyThreads - 1) / kCopyThreads;
    for (int64_t b0 = 0; b0 < blocks; b0 += kMaxGrid) {
        const int64_t nb = blocks - b0 < kMaxGrid ? blocks - b0 : kMaxGrid;
        hipLaunchKernelGGL(k_copy, dim3(static_cast<unsigned>(nb)), dim3(kCopyThreads), 0, stream,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16, b0 * kCopyThreads);
    }
    return hipGetLastError();
}

}  // namespace swz
