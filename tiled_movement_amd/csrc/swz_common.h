// Shared by the HIP kernels and the host-side chooser: the swizzle function,
// the LDS address of a tile element, and, for each read kind, which tile
// element every lane touches at every step.  Keeping the lane maps in one
// place means the chooser predicts conflicts for exactly the accesses the
// kernels issue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swz.h"

namespace swz {

// Swizzle<B,M,S> of a 32-bit element offset: the B-bit field at bit M+S is
// XORed into the B-bit field at bit M ("CuTe Swizzle 学习手册", swizzle
// formula).  B == 0 is the identity.  Callers guarantee M+S+B <= 32.
__host__ __device__ __forceinline__ uint32_t swizzle(uint32_t x, uint32_t B, uint32_t M, uint32_t S) {
    if (B == 0) return x;
    const uint32_t mask = (B >= 32u) ? 0xffffffffu : ((1u << B) - 1u);
    return x ^ (((x >> (M + S)) & mask) << M);
}

// How a tile sits in LDS: element (r, c) lives at element offset
// swizzle(r * ld + c).  ld = tile_cols (+ pad for the padded layout); the
// swizzle is the identity (B = 0) for PAD and PLAIN.
struct LdsLayout {
    uint32_t ld;  // LDS row pitch in elements
    uint32_t B, M, S;
};

__host__ __device__ __forceinline__ uint32_t lds_elem(const LdsLayout& L, uint32_t r, uint32_t c) {
    return swizzle(r * L.ld + c, L.B, L.M, L.S);
}

// ---------------------------------------------------------------------------
// Tile shapes and thread counts of each read kind.
// ---------------------------------------------------------------------------
template <int KIND> struct Kind;

// 4-byte elements, 32x32 tile.  Staging: each thread writes single elements,
// a wave covering two full 128-byte rows.  Read: each thread reads single
// elements down a column, a wave covering two columns.
template <> struct Kind<SWZ_READ_SCALAR_COL> {
    static constexpr int ESZ = 4, TR = 32, TC = 32, NT = 256;
    static constexpr int VEC = 4;                        // LDS store width (bytes)
    static constexpr int WSTEPS = TR * TC / NT;          // element stores per thread
    static constexpr int RSTEPS = TR * TC / NT;          // element loads per thread
    static constexpr int RWIDTH = 4;                     // LDS load width (bytes)
    __host__ __device__ static void wcoord(int t, int i, int& r, int& c) { r = t / 32 + i * (NT / 32); c = t % 32; }
    __host__ __device__ static void rcoord(int t, int i, int& r, int& c) { r = t % 32; c = t / 32 + i * (NT / 32); }
};

// 2-byte elements, 64x64 tile (128-byte rows).  Staging: 16-byte vectors,
// 8 lanes per row.  Read: thread q owns row block k = q%8 (rows 8k..8k+7)
// and column group g = q/8 (columns 4g..4g+3); step i reads the 8 bytes of
// row 8k+i in that group.
template <> struct Kind<SWZ_READ_B64_4X4> {
    static constexpr int ESZ = 2, TR = 64, TC = 64, NT = 128;
    static constexpr int VEC = 16;
    static constexpr int WSTEPS = TR * TC * ESZ / VEC / NT;  // 4
    static constexpr int RSTEPS = 8;
    static constexpr int RWIDTH = 8;
    __host__ __device__ static void wcoord(int t, int i, int& r, int& c) { r = t / 8 + i * (NT / 8); c = 8 * (t % 8); }
    __host__ __device__ static void rcoord(int t, int i, int& r, int& c) { r = 8 * (t % 8) + i; c = 4 * (t / 8); }
};

// 2-byte elements, 64x128 tile (256-byte rows).  Staging: 16-byte vectors,
// 16 lanes per row.  Read: thread q owns row block rb = q%8 and 16-byte
// column chunk ch = q/8; step i reads chunk ch of row 8rb+i.
template <> struct Kind<SWZ_READ_B128_8X8> {
    static constexpr int ESZ = 2, TR = 64, TC = 128, NT = 128;
    static constexpr int VEC = 16;
    static constexpr int WSTEPS = TR * TC * ESZ / VEC / NT;  // 8
    static constexpr int RSTEPS = 8;
    static constexpr int RWIDTH = 16;
    __host__ __device__ static void wcoord(int t, int i, int& r, int& c) { r = t / 16 + i * (NT / 16); c = 8 * (t % 16); }
    __host__ __device__ static void rcoord(int t, int i, int& r, int& c) { r = 8 * (t % 8) + i; c = 8 * (t / 8); }
};

// Operand staging: 2-byte elements, 256x64 tile (256 rows of the MN
// dimension, 64 of K; 128-byte rows).  Staging: 16-byte vectors, 8 lanes per
// row.  Read: the 32 fragments of the tile (16 row blocks x 2 k steps); wave
// w reads fragments f = w + 4*i; lane l of fragment f reads row
// 16*(f%16) + l%16, k = 32*(f/16) + 8*(l/16) .. +7.
template <> struct Kind<SWZ_READ_MFMA_16X16X32> {
    static constexpr int ESZ = 2, TR = 256, TC = 64, NT = 256;
    static constexpr int VEC = 16;
    static constexpr int WSTEPS = TR * TC * ESZ / VEC / NT;  // 8
    static constexpr int RSTEPS = 8;                          // fragments per wave
    static constexpr int RWIDTH = 16;
    __host__ __device__ static int frag_of(int t, int i) { return (t / 64) + 4 * i; }
    __host__ __device__ static void wcoord(int t, int i, int& r, int& c) { r = t / 8 + i * (NT / 8); c = 8 * (t % 8); }
    __host__ __device__ static void rcoord(int t, int i, int& r, int& c) {
        const int f = frag_of(t, i), l = t % 64;
        r = 16 * (f % 16) + l % 16;
        c = 32 * (f / 16) + 8 * (l / 16);
    }
};

}  // namespace swz
