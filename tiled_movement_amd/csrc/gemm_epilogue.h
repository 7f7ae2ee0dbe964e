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

}  // namespace swz
