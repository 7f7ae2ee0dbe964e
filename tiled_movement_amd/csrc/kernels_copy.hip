// Reference device copy: plain 16-byte vector loads and stores, several in
// flight per thread, non-temporal like the tile kernels' global accesses.
// It is the read-once / write-once bandwidth ceiling the tile kernels are
// compared with, and the kernel of known size HBM byte counters are scaled
// by.
#include "launch.h"

namespace swz {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyChunk = int64_t(kCopyThreads) * kCopyUnroll;  // 16-byte vectors per block step
constexpr int64_t kMaxGrid = int64_t(1) << 22;

__global__ __launch_bounds__(kCopyThreads) void k_copy(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                                       int64_t n16) {
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyChunk + threadIdx.x; base < n16;
         base += static_cast<int64_t>(gridDim.x) * kCopyChunk) {
        if (base + (kCopyUnroll - 1) * kCopyThreads < n16) {
            u32x4 v[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(&s[base + u * kCopyThreads]);
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], &d[base + u * kCopyThreads]);
        } else {
            for (int u = 0; u < kCopyUnroll; ++u) {
                const int64_t i = base + u * kCopyThreads;
                if (i < n16) d[i] = s[i];
            }
        }
    }
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    int64_t blocks = (n16 + kCopyChunk - 1) / kCopyChunk;
    if (blocks > kMaxGrid) blocks = kMaxGrid;
    hipLaunchKernelGGL(k_copy, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

}  // namespace swz
