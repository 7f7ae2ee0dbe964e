// Reference device copy (16-byte vectors, several loads in flight per
// thread) and the resident-grid helper shared by the tile kernels.  The copy
// is the plain kernel against which HBM byte counters are calibrated and
// the practical bandwidth ceiling of a read-once / write-once pass.
#include <map>
#include <mutex>
#include <utility>

#include "launch.h"

namespace swz {

int64_t resident_grid(const void* kernel, int threads, int64_t want) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const auto key = std::make_pair(kernel, dev);
    int64_t cap = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) cap = it->second;
    }
    if (cap == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
            per_cu = 1;
        cap = static_cast<int64_t>(cus) * per_cu;
        std::lock_guard<std::mutex> lock(mu);
        cache[key] = cap;
    }
    return want < cap ? want : cap;
}

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void k_copy(const uint4* __restrict__ s, uint4* __restrict__ d,
                                                       int64_t n16) {
    const int64_t chunk = static_cast<int64_t>(kCopyThreads) * kCopyUnroll;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * chunk + threadIdx.x; base < n16;
         base += static_cast<int64_t>(gridDim.x) * chunk) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * kCopyThreads;
            if (i < n16) v[u] = s[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const int64_t i = base + u * kCopyThreads;
            if (i < n16) d[i] = v[u];
        }
    }
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    const int64_t blocks = (n16 + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
    const int64_t grid = resident_grid(reinterpret_cast<const void*>(k_copy), kCopyThreads, blocks);
    hipLaunchKernelGGL(k_copy, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), 0, stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
    return hipGetLastError();
}

}  // namespace swz
