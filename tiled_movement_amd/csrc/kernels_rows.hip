// Transposes of matrices whose rows are narrower than 64 bytes but whose
// width is not a power of two ([rows][3] coordinates, [rows][12], ...).
// The 32 x 32 and 64 x 64 tiles would hold a handful of columns each, and
// the power-of-two whole-row kinds need a width that divides their tiles.
// Here a tile is TR whole rows, one contiguous stretch of the source, copied
// flat into LDS with 16-byte loads; then each lane gathers 4 bytes' worth of
// consecutive rows of one column (1, 2 or 4 elements) and the wave writes
// 64 such words, 256 contiguous bytes of one output row, per store.
//
// LDS: lanes of a read are 4C bytes apart (C words), so the 32 lanes of a
// phase meet 32 / gcd(C, 32) banks: odd widths read without conflicts (the
// flat copy then writes whole 16-byte slots), while an even width C = 2^a m
// alone would serialise 2^a ways.  For those the tile's word w lives at
// w ^ ((w >> S) & (2^B - 1)) (Swizzle<B,0,S> on word offsets, chosen per
// width by rows_choice against the bank model), which spreads the lanes of
// a read over all banks; the copy then writes 4-byte words.
#include "launch.h"

namespace swz {
namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
// Row starts need not be 16-byte (or even 4-byte) aligned: compute queues
// on this GPU run in the unaligned memory access mode, and the compiler
// emits one dwordx4 / dword access for these byte-aligned types.
typedef u32x4v __attribute__((aligned(1))) u32x4_u1;
typedef uint32_t __attribute__((aligned(1))) u32_u1;

constexpr int kRowsThreads = 256;
constexpr int64_t kRowsMaxGrid = int64_t(1) << 22;

// Tile t (of the batch's tiles in order): entry b, rows r0 .. r0 + nr - 1.
// E: element bytes; RL = 4 / E rows per lane-word.
template <int E>
__global__ __launch_bounds__(kRowsThreads) void k_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int64_t rows, int32_t cols, int32_t tile_rows,
                                                       int64_t tiles_per_entry, int64_t tile0, uint32_t sw_b,
                                                       uint32_t sw_s) {
    constexpr int RL = 4 / E;
    __shared__ u32x4v lds_v[kRowsTileBytes / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v);
    const int t = threadIdx.x, lane = t % 64;
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
    const int64_t tile = tile0 + blockIdx.x;
    const int64_t b = tile / tiles_per_entry, r0 = (tile - b * tiles_per_entry) * tile_rows;
    const int nr = static_cast<int>(rows - r0 < tile_rows ? rows - r0 : tile_rows);
    const int64_t row_bytes = static_cast<int64_t>(cols) * E;
    const uint8_t* S = src + (b * rows + r0) * row_bytes;
    const int nbytes = nr * static_cast<int>(row_bytes);

    // LDS byte of tile byte k: its word swizzled, the byte within kept.
    const uint32_t mask = (1u << sw_b) - 1u;
    auto at = [&](uint32_t k) { return ((k >> 2) ^ ((k >> (2 + sw_s)) & mask)) * 4u + (k & 3u); };

    // Flat copy of the tile's bytes: whole 16-byte pieces, then the tail.
    for (int v = t; 16 * v < nbytes; v += kRowsThreads) {
        if (16 * v + 16 <= nbytes) {
            const u32x4v x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_u1*>(S + 16 * v));
            if (sw_b == 0) {
                lds_v[v] = x;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(lds + at(16 * v + 4 * j)) = x[j];
            }
        } else {
            for (int k = 16 * v; k < nbytes; ++k) lds[at(k)] = S[k];
        }
    }
    __syncthreads();

    // Output row c of entry b starts at dst + (b cols + c) rows E; the wave
    // job (c, k) writes its rows 64 RL k .. + 64 RL - 1 of this tile.
    const int steps = (nr + 64 * RL - 1) / (64 * RL);
    const int jobs = cols * steps;
    for (int job = wave; job < jobs; job += kRowsThreads / 64) {
        const int c = job / steps, k = job - c * steps;
        const int rb = 64 * RL * k + RL * lane;  // the lane's first row in the tile
        if (rb >= nr) continue;
        uint8_t* D = dst + ((b * cols + c) * rows + r0 + rb) * E;
        if (rb + RL <= nr) {
            uint32_t w;
            if constexpr (E == 4) {
                w = *reinterpret_cast<const uint32_t*>(lds + at((rb * cols + c) * 4));
            } else if constexpr (E == 2) {
                const uint32_t lo = *reinterpret_cast<const uint16_t*>(lds + at((rb * cols + c) * 2));
                const uint32_t hi = *reinterpret_cast<const uint16_t*>(lds + at(((rb + 1) * cols + c) * 2));
                w = lo | (hi << 16);
            } else {
                w = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) w |= static_cast<uint32_t>(lds[at((rb + i) * cols + c)]) << (8 * i);
            }
            __builtin_nontemporal_store(w, reinterpret_cast<u32_u1*>(D));
        } else {
            for (int i = 0; rb + i < nr; ++i)
                for (int e = 0; e < E; ++e) D[i * E + e] = lds[at(((rb + i) * cols + c) * E + e)];
        }
    }
}

template <int E>
hipError_t launch_rows_e(const ConvertJob& j, hipStream_t stream) {
    const int32_t cols = static_cast<int32_t>(j.cols);
    const int64_t tr = rows_tile_rows(j.cols, E);
    if (tr < 64 * (4 / E)) return hipErrorInvalidValue;  // rows wider than the kind takes
    const int64_t per = (j.rows + tr - 1) / tr, n = j.batch * per;
    for (int64_t t0 = 0; t0 < n; t0 += kRowsMaxGrid) {
        const int64_t cnt = n - t0 < kRowsMaxGrid ? n - t0 : kRowsMaxGrid;
        hipLaunchKernelGGL(k_rows<E>, dim3(static_cast<unsigned>(cnt)), dim3(kRowsThreads), 0, stream,
                           static_cast<const uint8_t*>(j.src), static_cast<uint8_t*>(j.dst), j.rows, cols,
                           static_cast<int32_t>(tr), per, t0, j.layout.B, static_cast<uint32_t>(j.layout.S));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rows(int esz, const ConvertJob& j, hipStream_t stream) {
    if (j.batch == 0 || j.rows == 0 || j.cols == 0) return hipSuccess;
    switch (esz) {
        case 4: return launch_rows_e<4>(j, stream);
        case 2: return launch_rows_e<2>(j, stream);
        case 1: return launch_rows_e<1>(j, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace swz
