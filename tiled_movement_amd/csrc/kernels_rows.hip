// Transposes of matrices of up to 128 columns whose width is not a power of
// two ([rows][3] coordinates, [rows][12], [rows][48], ...).  The 32 x 32 and
// 64 x 64 tiles would leave many of their columns empty, and the
// power-of-two whole-row kinds need a width that divides their tiles.
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

constexpr int64_t kRowsMaxGrid = int64_t(1) << 22;
constexpr int kRowsUnroll = 4;
// Tiles whose run in an output row is at most this many bytes shift their
// runs onto the output's lines (below).  Measured on 64 MiB matrices whose
// output rows are not whole lines: with the shift, fp32 [N][12] (1,280-byte
// runs) 0.66 -> 0.74 of a copy, 2-byte [N][24] (512) 0.57 -> 0.72, bytes
// [N][48] (256) 0.48 -> 0.63; without it, fp32 [N][3] (5,376) 0.83 against
// 0.77 and 2-byte [N][6] (2,560) 0.75 against 0.73.
constexpr int64_t kRowsShiftRun = 2048;

// Tile t (of the batch's tiles in order): entry b, rows r0 .. r0 + nr - 1,
// and with SHIFT up to `halo` rows past them.  E: element bytes; RL = 4 / E
// rows per lane-word; NT threads; LDS the bytes of tile and halo (at most a
// quarter more).
template <int E, bool SHIFT, int NT, int LDS>
__global__ __launch_bounds__(NT) void k_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int64_t rows, int32_t cols, int32_t tile_rows,
                                                       int64_t tiles_per_entry, int64_t tile0, uint32_t sw_b,
                                                       uint32_t sw_s, int32_t halo) {
    constexpr int RL = 4 / E;
    static_assert(LDS % (4 << 10) == 0, "the word swizzle (B <= 10) stays inside the array");
    __shared__ u32x4v lds_v[LDS / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v);
    const int t = threadIdx.x, lane = t % 64;
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
    const int64_t tile = tile0 + blockIdx.x;
    const int64_t b = tile / tiles_per_entry, r0 = (tile - b * tiles_per_entry) * tile_rows;
    const int H = SHIFT ? halo : 0;  // halo rows
    const int rem = static_cast<int>(rows - r0 < tile_rows + H ? rows - r0 : tile_rows + H);
    const int nr = rem < tile_rows ? rem : tile_rows;  // the tile's own rows
    const int64_t row_bytes = static_cast<int64_t>(cols) * E;
    const uint8_t* S = src + (b * rows + r0) * row_bytes;
    const int nbytes = rem * static_cast<int>(row_bytes);  // own rows and halo

    // LDS byte of tile byte k: its word swizzled, the byte within kept.
    const uint32_t mask = (1u << sw_b) - 1u;
    auto at = [&](uint32_t k) { return ((k >> 2) ^ ((k >> (2 + sw_s)) & mask)) * 4u + (k & 3u); };

    // Flat copy of the tile's bytes: the thread's whole 16-byte pieces (at
    // most kRowsPieces) all loaded before any is written, then the tail.
    // Loads past the last piece re-read that piece (in bounds, not written),
    // so none sits behind a branch and all of them are in flight together.
    constexpr int kRowsPieces = LDS / 16 / NT;
    static_assert(kRowsPieces * 16 * NT == LDS, "the array is whole rounds of pieces");
    const int whole = nbytes / 16;
    if (whole > 0) {
        u32x4v x[kRowsPieces];
#pragma unroll
        for (int i = 0; i < kRowsPieces; ++i) {
            const int v = min(t + i * NT, whole - 1);
            x[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_u1*>(S + 16 * v));
        }
#pragma unroll
        for (int i = 0; i < kRowsPieces; ++i) {
            const int v = t + i * NT;
            if (v < whole) {
                if (sw_b == 0) {
                    lds_v[v] = x[i];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(lds + at(16 * v + 4 * j)) = x[i][j];
                }
            }
        }
    }
    if (t == 0)
        for (int k = 16 * whole; k < nbytes; ++k) lds[at(k)] = S[k];
    __syncthreads();

    // Output row c of entry b starts at dst + (b cols + c) rows E.  With
    // SHIFT its rows r0 + sh(c) .. r0 + tile_rows + sh(c) - 1 (of the matrix)
    // are this tile's, sh(c) <= H being the rows up to the first whose output
    // byte starts a kRowsLine-byte line (the same for every tile of the
    // entry: tile_rows E is a multiple of the line; the host sizes H to the
    // largest), so no line of the output is written by two tiles, and the
    // entry's first tile also writes rows 0 .. sh(c) - 1; without, sh(c) = 0.
    // The wave job (c, k) writes 64 lane-words from tile row sh(c) + 64 RL k
    // on.
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst);
    auto shift = [&](int c) -> int {
        if constexpr (SHIFT) {
            const uintptr_t a = d0 + static_cast<uintptr_t>(((b * cols + c) * rows + r0) * E);
            return static_cast<int>(((kRowsLine - a % kRowsLine) % kRowsLine + E - 1) / E);
        } else {
            return 0;
        }
    };
    const int steps = (nr + 64 * RL - 1) / (64 * RL);
    const int jobs = cols * steps;
    // A lane-word: the RL elements of column c in rows rb .. rb + RL - 1, read
    // from tile byte offsets o + i cols E (i < RL).  A job without a whole
    // lane-word reads offset 0 instead (in the tile, unused), so the reads
    // need no branch.
    auto word = [&](uint32_t o) -> uint32_t {
        if constexpr (E == 4) {
            return *reinterpret_cast<const uint32_t*>(lds + at(o));
        } else if constexpr (E == 2) {
            const uint32_t lo = *reinterpret_cast<const uint16_t*>(lds + at(o));
            const uint32_t hi = *reinterpret_cast<const uint16_t*>(lds + at(o + 2 * cols));
            return lo | (hi << 16);
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) w |= static_cast<uint32_t>(lds[at(o + i * cols)]) << (8 * i);
            return w;
        }
    };
    // The wave's jobs kRowsUnroll at a time: every LDS read of the group is
    // issued before the first store.
    constexpr int kWaves = NT / 64;
    for (int job0 = wave; job0 < jobs; job0 += kWaves * kRowsUnroll) {
        uint32_t w[kRowsUnroll];
        int c[kRowsUnroll], rb[kRowsUnroll], hi[kRowsUnroll];
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
            const int job = job0 + kWaves * u;
            c[u] = job / steps;
            const int sh = job < jobs ? shift(c[u]) : 0;
            rb[u] = sh + 64 * RL * (job - c[u] * steps) + RL * lane;
            hi[u] = job < jobs ? (rem < tile_rows + sh ? rem : tile_rows + sh) : 0;
            const bool full = rb[u] + RL <= hi[u];
            w[u] = word(full ? static_cast<uint32_t>((rb[u] * cols + c[u]) * E) : 0u);
        }
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
            if (rb[u] >= hi[u]) continue;
            uint8_t* D = dst + ((b * cols + c[u]) * rows + r0 + rb[u]) * E;
            if (rb[u] + RL <= hi[u]) {
                __builtin_nontemporal_store(w[u], reinterpret_cast<u32_u1*>(D));
            } else {
                for (int i = 0; rb[u] + i < hi[u]; ++i)
                    for (int e = 0; e < E; ++e) D[i * E + e] = lds[at(((rb[u] + i) * cols + c[u]) * E + e)];
            }
        }
    }
    // The entry's first rows before each output row's first line.
    if (SHIFT && r0 == 0) {
        for (int q = t; q < cols * H; q += NT) {
            const int c = q / H, i = q - c * H;
            if (i >= shift(c) || i >= rem) continue;
            uint8_t* D = dst + ((b * cols + c) * rows + i) * E;
            for (int e = 0; e < E; ++e) D[e] = lds[at((i * cols + c) * E + e)];
        }
    }
}

// Rows of halo a launch needs: none unless the tile's run in an output row
// is at most kRowsShiftRun bytes; then the largest sh(c) over the entries
// and columns (the line phase of output row j = b cols + c repeats with a
// period of at most kRowsLine rows).
template <int E>
int32_t rows_halo(const ConvertJob& j, int64_t tr) {
    if (tr * E > kRowsShiftRun) return 0;
    const uintptr_t d = reinterpret_cast<uintptr_t>(j.dst);
    const int64_t n = j.batch * j.cols < kRowsLine ? j.batch * j.cols : kRowsLine;
    int32_t h = 0;
    for (int64_t r = 0; r < n; ++r) {
        const uintptr_t a = d + static_cast<uintptr_t>(r * j.rows * E);
        const int32_t sh = static_cast<int32_t>(((kRowsLine - a % kRowsLine) % kRowsLine + E - 1) / E);
        h = sh > h ? sh : h;
    }
    return h;
}

template <int E, int NT, int LDS>
hipError_t launch_rows_e(const ConvertJob& j, hipStream_t stream) {
    const int32_t cols = static_cast<int32_t>(j.cols);
    const int64_t tr = rows_tile_rows(j.cols, E);
    if (tr < 64 * (4 / E) || rows_lds_bytes(j.cols) != LDS || rows_threads(j.cols) != NT)
        return hipErrorInvalidValue;  // rows wider than the kind takes
    const int32_t halo = rows_halo<E>(j, tr);
    const int64_t per = (j.rows + tr - 1) / tr, n = j.batch * per;
    for (int64_t t0 = 0; t0 < n; t0 += kRowsMaxGrid) {
        const int64_t cnt = n - t0 < kRowsMaxGrid ? n - t0 : kRowsMaxGrid;
        const dim3 grid(static_cast<unsigned>(cnt)), block(NT);
        const auto* s = static_cast<const uint8_t*>(j.src);
        auto* d = static_cast<uint8_t*>(j.dst);
        const auto sb = static_cast<uint32_t>(j.layout.B), ss = static_cast<uint32_t>(j.layout.S);
        if (halo > 0)
            hipLaunchKernelGGL((k_rows<E, true, NT, LDS>), grid, block, 0, stream, s, d, j.rows, cols,
                               static_cast<int32_t>(tr), per, t0, sb, ss, halo);
        else
            hipLaunchKernelGGL((k_rows<E, false, NT, LDS>), grid, block, 0, stream, s, d, j.rows, cols,
                               static_cast<int32_t>(tr), per, t0, sb, ss, 0);
    }
    return hipGetLastError();
}

template <int E>
hipError_t launch_rows_w(const ConvertJob& j, hipStream_t stream) {
    return j.cols <= 64 ? launch_rows_e<E, 256, 20480>(j, stream) : launch_rows_e<E, 512, 40960>(j, stream);
}

}  // namespace

hipError_t launch_rows(int esz, const ConvertJob& j, hipStream_t stream) {
    if (j.batch == 0 || j.rows == 0 || j.cols == 0) return hipSuccess;
    switch (esz) {
        case 4: return launch_rows_w<4>(j, stream);
        case 2: return launch_rows_w<2>(j, stream);
        case 1: return launch_rows_w<1>(j, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace swz
