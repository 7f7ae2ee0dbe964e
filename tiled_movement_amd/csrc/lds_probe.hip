// LDS bank microbenchmark: time programmed per-lane LDS access patterns to
// measure how gfx950 splits a wave's LDS access into bank phases.  The pages
// define a conflict as lanes of one access asking a bank for different words
// ("CuTe Swizzle 学习手册", when conflicts happen; "CUDA 013 - Swizzle 的工作
// 原理", section 什么是 Bank Conflict); this kernel measures what that costs
// for each lane pattern on this hardware.
#include "launch.h"

namespace swz {
namespace {

constexpr uint32_t kWindow = 96 * 1024;  // bytes; more than half of a CU's LDS,
                                         // so one probe workgroup runs per CU
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int W>
struct Vec;
template <>
struct Vec<1> {
    using T = uint32_t;
};
template <>
struct Vec<2> {
    using T = uint32_t;
};
template <>
struct Vec<4> {
    using T = uint32_t;
};
template <>
struct Vec<8> {
    using T = u32x2;
};
template <>
struct Vec<16> {
    using T = u32x4;
};

// Eight back-to-back accesses to the same address, then wait for all of them.
template <int W>
__device__ __forceinline__ uint32_t read8(uint32_t a);
#define SWZ_PROBE_READ8(OP)                                                                                  \
    uint32_t r0, r1, r2, r3, r4, r5, r6, r7;                                                                 \
    asm volatile(OP " %0, %8\n\t" OP " %1, %8\n\t" OP " %2, %8\n\t" OP " %3, %8\n\t" OP " %4, %8\n\t" OP   \
                 " %5, %8\n\t" OP " %6, %8\n\t" OP " %7, %8\n\ts_waitcnt lgkmcnt(0)"                           \
                 : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)     \
                 : "v"(a)                                                                                    \
                 : "memory");                                                                                \
    return r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
template <>
__device__ __forceinline__ uint32_t read8<1>(uint32_t a) {
    SWZ_PROBE_READ8("ds_read_u8")
}
template <>
__device__ __forceinline__ uint32_t read8<2>(uint32_t a) {
    SWZ_PROBE_READ8("ds_read_u16")
}
#undef SWZ_PROBE_READ8
template <>
__device__ __forceinline__ uint32_t read8<4>(uint32_t a) {
    uint32_t r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b32 %0, %8\n\tds_read_b32 %1, %8\n\tds_read_b32 %2, %8\n\tds_read_b32 %3, %8\n\t"
        "ds_read_b32 %4, %8\n\tds_read_b32 %5, %8\n\tds_read_b32 %6, %8\n\tds_read_b32 %7, %8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a)
        : "memory");
    return r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
}
template <>
__device__ __forceinline__ uint32_t read8<8>(uint32_t a) {
    u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64 %0, %8\n\tds_read_b64 %1, %8\n\tds_read_b64 %2, %8\n\tds_read_b64 %3, %8\n\t"
        "ds_read_b64 %4, %8\n\tds_read_b64 %5, %8\n\tds_read_b64 %6, %8\n\tds_read_b64 %7, %8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a)
        : "memory");
    const u32x2 x = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
    return x.x ^ x.y;
}
template <>
__device__ __forceinline__ uint32_t read8<16>(uint32_t a) {
    u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8\n\tds_read_b128 %2, %8\n\tds_read_b128 %3, %8\n\t"
        "ds_read_b128 %4, %8\n\tds_read_b128 %5, %8\n\tds_read_b128 %6, %8\n\tds_read_b128 %7, %8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a)
        : "memory");
    const u32x4 x = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
    return x.x ^ x.y ^ x.z ^ x.w;
}

template <int W>
__device__ __forceinline__ void write8(uint32_t a, typename Vec<W>::T v);
#define SWZ_PROBE_WRITE8(OP)                                                                                 \
    asm volatile(OP " %0, %1\n\t" OP " %0, %1\n\t" OP " %0, %1\n\t" OP " %0, %1\n\t" OP " %0, %1\n\t" OP    \
                 " %0, %1\n\t" OP " %0, %1\n\t" OP " %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(a),                  \
                 "v"(v)                                                                                      \
                 : "memory");
template <>
__device__ __forceinline__ void write8<1>(uint32_t a, uint32_t v) {
    SWZ_PROBE_WRITE8("ds_write_b8")
}
template <>
__device__ __forceinline__ void write8<2>(uint32_t a, uint32_t v) {
    SWZ_PROBE_WRITE8("ds_write_b16")
}
#undef SWZ_PROBE_WRITE8
template <>
__device__ __forceinline__ void write8<4>(uint32_t a, uint32_t v) {
    asm volatile(
        "ds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\t"
        "ds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\tds_write_b32 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)" ::"v"(a),
        "v"(v)
        : "memory");
}
template <>
__device__ __forceinline__ void write8<8>(uint32_t a, u32x2 v) {
    asm volatile(
        "ds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\t"
        "ds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\tds_write_b64 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)" ::"v"(a),
        "v"(v)
        : "memory");
}
template <>
__device__ __forceinline__ void write8<16>(uint32_t a, u32x4 v) {
    asm volatile(
        "ds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\t"
        "ds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\tds_write_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)" ::"v"(a),
        "v"(v)
        : "memory");
}

template <int W, bool WRITE>
__global__ __launch_bounds__(1024) void k_lds_probe(const uint32_t* __restrict__ addrs,
                                                    const uint64_t* __restrict__ masks, int iters,
                                                    uint64_t* __restrict__ cycles) {
    __shared__ u32x4 window[kWindow / 16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.x;
    for (uint32_t i = threadIdx.x; i < kWindow / 16; i += blockDim.x) window[i] = u32x4{i, i + 1, i + 2, i + 3};
    __syncthreads();

    // Byte address inside the window, aligned to the access width.
    // LDS byte offset of the window (only a C-style cast reaches address space 3).
    const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)(window));
    const uint32_t a = base + ((addrs[64 * g + lane] % kWindow) & ~static_cast<uint32_t>(W - 1));
    const bool active = (masks[g] >> lane) & 1ull;
    typename Vec<W>::T v{};
    v = v + static_cast<uint32_t>(lane);
    uint32_t acc = 0;  // the asm statements are volatile, so unused reads stay

    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (active) {
        for (int it = 0; it < iters; ++it) {
            if (WRITE)
                write8<W>(a, v);
            else
                acc ^= read8<W>(a);
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) cycles[static_cast<int64_t>(g) * (blockDim.x / 64) + wave] = t1 - t0;
}

template <int W, bool WRITE>
void launch_one(const uint32_t* addrs, const uint64_t* masks, int n, int iters, int waves, uint64_t* cycles,
                hipStream_t stream) {
    hipLaunchKernelGGL((k_lds_probe<W, WRITE>), dim3(n), dim3(64 * waves), 0, stream, addrs, masks, iters, cycles);
}

}  // namespace

hipError_t launch_lds_probe(const uint32_t* addrs, const uint64_t* masks, int n, int width, bool write, int iters,
                            int waves, uint64_t* cycles, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (width == 1)
        write ? launch_one<1, true>(addrs, masks, n, iters, waves, cycles, stream)
              : launch_one<1, false>(addrs, masks, n, iters, waves, cycles, stream);
    else if (width == 2)
        write ? launch_one<2, true>(addrs, masks, n, iters, waves, cycles, stream)
              : launch_one<2, false>(addrs, masks, n, iters, waves, cycles, stream);
    else if (width == 4)
        write ? launch_one<4, true>(addrs, masks, n, iters, waves, cycles, stream)
              : launch_one<4, false>(addrs, masks, n, iters, waves, cycles, stream);
    else if (width == 8)
        write ? launch_one<8, true>(addrs, masks, n, iters, waves, cycles, stream)
              : launch_one<8, false>(addrs, masks, n, iters, waves, cycles, stream);
    else
        write ? launch_one<16, true>(addrs, masks, n, iters, waves, cycles, stream)
              : launch_one<16, false>(addrs, masks, n, iters, waves, cycles, stream);
    return hipGetLastError();
}

}  // namespace swz
