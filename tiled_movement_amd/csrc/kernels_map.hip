// Elementwise Swizzle<B,M,S> of 32-bit offsets ("CuTe Swizzle 学习手册",
// swizzle formula; "CUDA 013 - Swizzle 的工作原理", section 计算公式).
#include "launch.h"

namespace swz {
namespace {

// No __restrict__: in and out may be the same buffer (in place).
template <bool VEC4>
__global__ __launch_bounds__(256) void k_map(const uint32_t* in, uint32_t* out, int64_t n, uint32_t B, uint32_t M,
                                             int32_t S) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC4) {
        const int64_t n4 = n / 4;
        const uint4* in4 = reinterpret_cast<const uint4*>(in);
        uint4* out4 = reinterpret_cast<uint4*>(out);
        for (int64_t q = i; q < n4; q += stride) {
            uint4 x = in4[q];
            x.x = swizzle(x.x, B, M, S);
            x.y = swizzle(x.y, B, M, S);
            x.z = swizzle(x.z, B, M, S);
            x.w = swizzle(x.w, B, M, S);
            out4[q] = x;
        }
        for (int64_t q = 4 * n4 + i; q < n; q += stride) out[q] = swizzle(in[q], B, M, S);
    } else {
        for (; i < n; i += stride) out[i] = swizzle(in[i], B, M, S);
    }
}

}  // namespace

hipError_t launch_map(const int32_t* in, int32_t* out, int64_t n, swz_params p, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const bool vec4 = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    const int64_t items = vec4 ? (n + 3) / 4 : n;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const auto B = static_cast<uint32_t>(p.B), M = static_cast<uint32_t>(p.M);
    const int32_t S = p.S;
    const auto* ui = reinterpret_cast<const uint32_t*>(in);
    auto* uo = reinterpret_cast<uint32_t*>(out);
    if (vec4)
        hipLaunchKernelGGL(k_map<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ui, uo, n, B, M, S);
    else
        hipLaunchKernelGGL(k_map<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ui, uo, n, B, M, S);
    return hipGetLastError();
}

}  // namespace swz
