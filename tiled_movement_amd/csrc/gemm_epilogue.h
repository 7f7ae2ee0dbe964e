// Epilogue of the GEMM kernels: a wave's fp32 accumulators out to C as whole
// row runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swz {

typedef float epi_f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) float lds_f32;

// Lane l holds rows 4*(l/16) .. +3 of column l%16 of each 16 x 16 block (the
// 16x16x32 instruction's result layout).  One row of blocks at a time, the
// wave writes them into its own LDS slice of 16 rows x 16*WB_N floats and
// reads whole rows back, 16 bytes per lane, so every store instruction
// writes whole 64-byte runs of C rows.  The slice is itself swizzled: bit 2
// of the row flips bit 5 of the column (Swizzle<1,5,4> on float offsets
// with 128-float rows), which puts the two 16-lane groups of a half-wave --
// rows r and r + 4, same columns -- on different banks when they write;
// the row reads still cover whole aligned 128-byte blocks.
//   bm, bn : the wave's first block row and block column in C;
//   mb, nb : blocks of C along m and n (rows/columns beyond are not stored).
// A wave's LDS operations complete in order, so the reads see the writes
// and the next row of blocks overwrites the slice only after them.
template <int WB_M, int WB_N>
__device__ __forceinline__ void store_c_blocks(const epi_f32x4 (&acc)[WB_M][WB_N], lds_f32* slice,
                                               float* __restrict__ c, int64_t n, int64_t bm, int64_t bn, int64_t mb,
                                               int64_t nb, int lane) {
    constexpr int kRowFloats = WB_N * 16;
    static_assert(kRowFloats >= 64, "the slice swizzle flips column bit 5");
    const int g = lane / 16, col = lane % 16;
    const int wflip = 32 * (g & 1);  // rows 4g .. 4g+3 share bit 2 = g & 1
#pragma unroll
    for (int x = 0; x < WB_M; ++x) {
#pragma unroll
        for (int y = 0; y < WB_N; ++y)
#pragma unroll
            for (int i = 0; i < 4; ++i) slice[(4 * g + i) * kRowFloats + ((16 * y + col) ^ wflip)] = acc[x][y][i];
        if (bm + x < mb) {
            constexpr int kLanesPerRow = kRowFloats / 4;
#pragma unroll
            for (int q = 0; q < 16 * kLanesPerRow / 64; ++q) {
                const int t = q * 64 + lane, r = t / kLanesPerRow, c4 = 4 * (t % kLanesPerRow);
                const epi_f32x4 v =
                    *(__attribute__((address_space(3))) epi_f32x4*)(slice + r * kRowFloats + (c4 ^ (32 * ((r >> 2) & 1))));
                if (bn + c4 / 16 < nb)
                    __builtin_nontemporal_store(v, reinterpret_cast<epi_f32x4*>(c + (16 * (bm + x) + r) * n + 16 * bn + c4));
            }
        }
    }
}

}  // namespace swz
