// Epilogue of the GEMM kernels: a wave's fp32 accumulators out to C as whole
// row runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swz {

typedef float epi_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_f32;

// LDS bytes of one wave's slice: 16 rows of 16*WB_N floats, padded by 4.
template <int WB_N>
constexpr int epilogue_slice_bytes() {
    return 16 * (16 * WB_N + 4) * 4;
}

// Lane l holds rows 4*(l/16) .. +3 of column l%16 of each 16 x 16 block (the
// 16x16x32 instruction's result layout).  One row of blocks at a time, the
// wave writes them into its own LDS slice of 16 rows and reads whole rows
// back, 16 bytes per lane, so every store instruction writes whole 64-byte
// runs of C rows.  The writes go 4 bytes per lane; lanes 16 apart write the
// same columns 4 rows apart, and those two 16-lane groups are served
// together, so the rows are padded by 4 floats: 4 rows then move 16 banks.
// The row reads still cover whole 16-byte-aligned rows, each bank once per
// phase.
template <int WB_M, int WB_N>
__device__ __forceinline__ void store_c_blocks(const epi_f32x4 (&acc)[WB_M][WB_N], lds_f32* slice,
                                               float* __restrict__ c, int64_t n, int64_t bm, int64_t bn, int64_t mb,
                                               int64_t nb, int lane) {
    constexpr int kRowFloats = WB_N * 16, kPitch = kRowFloats + 4;
    const int g = lane / 16, col = lane % 16;
#pragma unroll
    for (int x = 0; x < WB_M; ++x) {
#pragma unroll
        for (int y = 0; y < WB_N; ++y)
#pragma unroll
            for (int i = 0; i < 4; ++i) slice[(4 * g + i) * kPitch + 16 * y + col] = acc[x][y][i];
        if (bm + x < mb) {
            constexpr int kLanesPerRow = kRowFloats / 4;
#pragma unroll
            for (int q = 0; q < 16 * kLanesPerRow / 64; ++q) {
                const int t = q * 64 + lane, r = t / kLanesPerRow, c4 = 4 * (t % kLanesPerRow);
                const epi_f32x4 v =
                    *(__attribute__((address_space(3))) epi_f32x4*)(slice + r * kPitch + c4);
                if (bn + c4 / 16 < nb)
                    __builtin_nontemporal_store(v, reinterpret_cast<epi_f32x4*>(c + (16 * (bm + x) + r) * n + 16 * bn + c4));
            }
        }
    }
}

// bf16 bits of an fp32 value, rounded to nearest with ties to even (the
// low 16 bits decide; a carry into the exponent is the correct rounding up);
// NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The same as store_c_blocks for a bf16 C: each lane reads 8 floats of a
// slice row back (two 16-byte reads), rounds them and stores 16 bytes, so
// every store instruction still writes whole 32-byte runs of C rows.
template <int WB_M, int WB_N>
__device__ __forceinline__ void store_c_blocks_bf16(const epi_f32x4 (&acc)[WB_M][WB_N], lds_f32* slice,
                                                    uint16_t* __restrict__ c, int64_t n, int64_t bm, int64_t bn,
                                                    int64_t mb, int64_t nb, int lane) {
    typedef uint32_t u32x4e __attribute__((ext_vector_type(4)));
    constexpr int kRowFloats = WB_N * 16, kPitch = kRowFloats + 4;
    const int g = lane / 16, col = lane % 16;
#pragma unroll
    for (int x = 0; x < WB_M; ++x) {
#pragma unroll
        for (int y = 0; y < WB_N; ++y)
#pragma unroll
            for (int i = 0; i < 4; ++i) slice[(4 * g + i) * kPitch + 16 * y + col] = acc[x][y][i];
        if (bm + x < mb) {
            constexpr int kLanesPerRow = kRowFloats / 8;
#pragma unroll
            for (int q = 0; q < 16 * kLanesPerRow / 64; ++q) {
                const int t = q * 64 + lane, r = t / kLanesPerRow, c8 = 8 * (t % kLanesPerRow);
                const epi_f32x4 v0 = *(__attribute__((address_space(3))) epi_f32x4*)(slice + r * kPitch + c8);
                const epi_f32x4 v1 = *(__attribute__((address_space(3))) epi_f32x4*)(slice + r * kPitch + c8 + 4);
                const u32x4e o{bf16_rne_bits(v0[0]) | (bf16_rne_bits(v0[1]) << 16),
                               bf16_rne_bits(v0[2]) | (bf16_rne_bits(v0[3]) << 16),
                               bf16_rne_bits(v1[0]) | (bf16_rne_bits(v1[1]) << 16),
                               bf16_rne_bits(v1[2]) | (bf16_rne_bits(v1[3]) << 16)};
                if (bn + c8 / 16 < nb)
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4e*>(c + (16 * (bm + x) + r) * n + 16 * bn + c8));
            }
        }
    }
}

}  // namespace swz
