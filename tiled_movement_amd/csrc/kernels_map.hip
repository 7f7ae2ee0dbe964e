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

// One input range under many triples: each thread loads its offsets once
// and writes them under T consecutive triples (rows y0 .. y0 + T - 1 of the
// output, y0 = T * blockIdx.y; rows at or past count are skipped).  Four
// triples per thread ran the 125-triple workload 11% faster than one (two:
// 8%, three and five: 5%).  VEC4: 16-byte vectors (pointers 16-byte
// aligned and n a multiple of 4, so every output row starts aligned).
template <bool VEC4, int T>
__global__ __launch_bounds__(256) void k_map_batch(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                   int64_t n, int count, MapParamPack pk) {
    const int y0 = blockIdx.y * T;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (VEC4) {
        typedef uint32_t v4 __attribute__((ext_vector_type(4)));
        const v4* in4 = reinterpret_cast<const v4*>(in);
        for (int64_t q = i; q < n / 4; q += stride) {
            const v4 x = in4[q];
#pragma unroll
            for (int j = 0; j < T; ++j) {
                const int y = y0 + j;
                if (y < count) {
                    const uint32_t B = pk.B[y], M = pk.M[y];
                    const int32_t S = pk.S[y];
                    v4* out4 = reinterpret_cast<v4*>(out + static_cast<int64_t>(y) * n);
                    const v4 o{swizzle(x[0], B, M, S), swizzle(x[1], B, M, S), swizzle(x[2], B, M, S), swizzle(x[3], B, M, S)};
                    __builtin_nontemporal_store(o, out4 + q);
                }
            }
        }
    } else {
        for (int j = 0; j < T; ++j) {
            const int y = y0 + j;
            if (y >= count) break;
            const uint32_t B = pk.B[y], M = pk.M[y];
            const int32_t S = pk.S[y];
            uint32_t* row = out + static_cast<int64_t>(y) * n;
            for (int64_t q = i; q < n; q += stride) row[q] = swizzle(in[q], B, M, S);
        }
    }
}

constexpr int kMapTriplesPerThread = 4;

}  // namespace

hipError_t launch_map_batch(const int32_t* in, int32_t* out, int64_t n, const MapParamPack& pk, int count,
                            hipStream_t stream) {
    if (n == 0 || count == 0) return hipSuccess;
    const bool vec4 = reinterpret_cast<uintptr_t>(in) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0 &&
                      n % 4 == 0;
    const int64_t items = vec4 ? n / 4 : n;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    constexpr int TPB = kMapTriplesPerThread;
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>((count + TPB - 1) / TPB));
    const auto* ui = reinterpret_cast<const uint32_t*>(in);
    auto* uo = reinterpret_cast<uint32_t*>(out);
    if (vec4)
        hipLaunchKernelGGL((k_map_batch<true, TPB>), grid, dim3(256), 0, stream, ui, uo, n, count, pk);
    else
        hipLaunchKernelGGL((k_map_batch<false, TPB>), grid, dim3(256), 0, stream, ui, uo, n, count, pk);
    return hipGetLastError();
}

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
