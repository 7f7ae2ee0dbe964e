// Tile staging kernels for gfx950: coalesced 16-byte row loads from HBM into
// an LDS tile laid out by Swizzle<B,M,S> (or padded / plain rows) -- through
// registers, or by direct HBM -> LDS loads that apply the swizzle on the HBM
// side -- a read back along columns (4-byte column reads, 8- and 16-byte
// row pieces with in-register transposes, or gfx950's 16- and 8-bit LDS
// transpose reads) or in the operand-fragment pattern, and coalesced 16-byte
// row stores.
//
// The method is the one of "CuTe Swizzle 学习手册" (typical scenario: column
// access of a row-major tile; swizzle formula) and "CUDA 013 - Swizzle 的
// 工作原理" (sections 如何避免 Bank Conflict, Swizzle 技术, 更通用的映射规则):
// remap the flat offset of each tile element so that the rows written by a
// wave and the columns read by a wave both spread over all LDS banks.
//
// HBM side (measured on MI355X): with row-major tile order every tile in
// flight writes the same column offset of rows 2^k bytes apart, so the
// writes pile onto a few memory channels.  Tiles are therefore visited in
// diagonal order (consecutive tiles differ in both tile row and tile
// column), and global loads and stores are non-temporal: every byte is read
// once and written once.
#include <type_traits>

#include "launch.h"

#ifndef SWZ_TILE_ORDER  // transposes: 1 = diagonal tile order, 0 = row-major
#define SWZ_TILE_ORDER 1
#endif
#ifndef SWZ_STAGE_ORDER  // operand staging: row-major keeps reads and writes contiguous
#define SWZ_STAGE_ORDER 0
#endif
#ifndef SWZ_GRID3D  // 1: 3-D grids (tile row, tile column, batch) where they fit
#define SWZ_GRID3D 1
#endif
#ifndef SWZ_NONTEMPORAL  // 1: non-temporal global loads and stores
#define SWZ_NONTEMPORAL 1
#endif

namespace swz {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tiles per launch; larger jobs are launched in chunks, one tile per
// workgroup (no loop in the kernel, so nothing is kept live across tiles).
constexpr int64_t kMaxGrid = int64_t(1) << 22;

// Cache-policy operand of the direct load for a non-temporal access.
constexpr int kDirectNT = 2;

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if (SWZ_NONTEMPORAL) return __builtin_nontemporal_load(q);
    return *q;
}

__device__ __forceinline__ void gstore16(uint8_t* p, u32x4 v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    if (SWZ_NONTEMPORAL)
        __builtin_nontemporal_store(v, q);
    else
        *q = v;
}

// Tile (batch b, tile row tr, tile column tc) of linear tile index t.
// Diagonal orders: t -> tr = t % tiles_r, tc = (t / tiles_r + f(tr)) %
// tiles_c with f(tr) = (tr * O.num) >> O.sh: slope 1 (the default), 1/2, 3,
// or 0 (tile columns in turn).  One-to-one for any grid shape (for each tr,
// q -> (q + f(tr)) mod tiles_c is a permutation).  Row-major: tc fastest.
struct TileOrder {
    uint32_t num, sh;
};

template <bool DIAGONAL>
__device__ __forceinline__ void decode_tile(int64_t t, int64_t tiles_r, int64_t tiles_c, TileOrder O, int64_t& b,
                                            int64_t& tr, int64_t& tc) {
    const int64_t per = tiles_r * tiles_c;
    b = t / per;
    const int64_t w = t - b * per;
    if (DIAGONAL) {
        tr = w % tiles_r;
        tc = (w / tiles_r + ((tr * O.num) >> O.sh) % tiles_c) % tiles_c;
    } else {
        tr = w / tiles_c;
        tc = w % tiles_c;
    }
}

// Element j of row a in the low half, element j of row b in the high half.
template <typename V>
__device__ __forceinline__ uint32_t pair_col(const V& a, const V& b, int j) {
    const uint32_t wa = a[j >> 1], wb = b[j >> 1];
    return (j & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// 16 bytes = 16/ESZ consecutive elements of one row, zero outside the matrix.
template <int ESZ>
__device__ __forceinline__ u32x4 load16_guarded(const uint8_t* S, int64_t row, int64_t col, int64_t rows,
                                                int64_t cols) {
    constexpr int N = 16 / ESZ;
    uint32_t e[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const bool in = row < rows && col + k < cols;
        if (ESZ == 4)
            e[k] = in ? reinterpret_cast<const uint32_t*>(S)[row * cols + col + k] : 0u;
        else if (ESZ == 2)
            e[k] = in ? reinterpret_cast<const uint16_t*>(S)[row * cols + col + k] : 0u;
        else
            e[k] = in ? S[row * cols + col + k] : 0u;
    }
    if constexpr (ESZ == 4) {
        return u32x4{e[0], e[1], e[2], e[3]};
    } else if constexpr (ESZ == 2) {
        return u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    } else {
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            o[w] = e[4 * w] | (e[4 * w + 1] << 8) | (e[4 * w + 2] << 16) | (e[4 * w + 3] << 24);
        return o;
    }
}

// 16 bytes = 16/ESZ consecutive elements of one output row; only those
// inside the matrix are written.
template <int ESZ>
__device__ __forceinline__ void store16_guarded(uint8_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                                const u32x4& o) {
    if (row >= nrows) return;
    if (ESZ == 1) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (col + k < ncols) D[row * ncols + col + k] = static_cast<uint8_t>(o[k >> 2] >> (8 * (k & 3)));
    } else if (ESZ == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (col + k < ncols) reinterpret_cast<uint32_t*>(D)[row * ncols + col + k] = o[k];
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (col + k < ncols)
                reinterpret_cast<uint16_t*>(D)[row * ncols + col + k] = static_cast<uint16_t>(o[k >> 1] >> (16 * (k & 1)));
    }
}

// How a tile's 16-byte pieces are guarded at the matrix edge.  kFull: the
// whole tile is inside, no guards.  kVec: the tile sticks out, but every row
// pitch is a multiple of 16 bytes, so each piece is wholly inside or wholly
// outside the matrix: one test per piece, whole-vector accesses.  kElem: row
// pitches that are not multiples of 16 bytes: element by element.
enum Edge { kFull = 0, kVec = 1, kElem = 2 };

template <int EDGE, int ESZ>
__device__ __forceinline__ u32x4 load16_edge(const uint8_t* S, int64_t row, int64_t col, int64_t rows,
                                             int64_t cols) {
    if constexpr (EDGE == kFull) return gload16(S + (row * cols + col) * ESZ);
    if constexpr (EDGE == kVec) return row < rows && col < cols ? gload16(S + (row * cols + col) * ESZ) : u32x4{0u, 0u, 0u, 0u};
    return load16_guarded<ESZ>(S, row, col, rows, cols);
}

template <int EDGE, int ESZ>
__device__ __forceinline__ void store16_edge(uint8_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                             u32x4 v) {
    if constexpr (EDGE == kFull) {
        gstore16(D + (row * ncols + col) * ESZ, v);
    } else if constexpr (EDGE == kVec) {
        if (row < nrows && col < ncols) gstore16(D + (row * ncols + col) * ESZ, v);
    } else {
        store16_guarded<ESZ>(D, row, col, nrows, ncols, v);
    }
}

// Workgroups per CU.  The transposed HBM pattern of the 16-bit and 8-bit
// tiles runs faster with fewer tiles in flight (measured with an LDS-free
// probe of the same pattern: 64 x 64 16-bit tiles at 8 to 16 workgroups per
// CU 5.41-5.48 TB/s, at 4-5 per CU 5.69).  Each launch reserves extra LDS so
// that a CU holds at most this many workgroups of the kind (0: no limit).
// Values from a sweep of the kernels themselves (2 to 8 per CU): 4 for the
// 64-row 16-bit kinds (+3 to +8%), 5 for the byte kind (+4%); the fp32 tile
// loses bandwidth when limited and staging's 32 KiB tile already sits at 5.
#ifndef SWZ_OCC_SCALAR
#define SWZ_OCC_SCALAR 0
#endif
#ifndef SWZ_OCC_B64
#define SWZ_OCC_B64 4
#endif
#ifndef SWZ_OCC_B128
#define SWZ_OCC_B128 4
#endif
#ifndef SWZ_OCC_STAGE
#define SWZ_OCC_STAGE 0
#endif
#ifndef SWZ_OCC_TR16
#define SWZ_OCC_TR16 4
#endif
#ifndef SWZ_OCC_TR8
#define SWZ_OCC_TR8 5
#endif
#ifndef SWZ_OCC_NARROW
#define SWZ_OCC_NARROW 0
#endif

// Whole-row tiles: uncapped, except the 16 KiB byte tiles of 32 and 64
// columns, which a sweep (uncapped, 4 and 8 per CU) put 4% faster at 4;
// every other narrow kind lost up to 20% when capped.
#ifndef SWZ_OCC_BNARROW_WIDE
#define SWZ_OCC_BNARROW_WIDE 4
#endif

template <int KIND>
constexpr int occupancy_limit() {
    return KIND == SWZ_READ_SCALAR_COL ? SWZ_OCC_SCALAR
           : KIND == SWZ_READ_B64_4X4  ? SWZ_OCC_B64
           : KIND == SWZ_READ_B128_8X8 ? SWZ_OCC_B128
           : KIND == SWZ_READ_MFMA_16X16X32 ? SWZ_OCC_STAGE
           : KIND == SWZ_READ_B64_TR16 ? SWZ_OCC_TR16
           : KIND == SWZ_READ_B64_TR8  ? SWZ_OCC_TR8
           : (KIND == SWZ_READ_BNARROW32 || KIND == SWZ_READ_BNARROW64) ? SWZ_OCC_BNARROW_WIDE
                                       : SWZ_OCC_NARROW;
}

constexpr int kLdsPerCu = 160 * 1024;

// Dynamic LDS to add to a launch whose kernel uses `static_bytes` so that at
// most occupancy_limit<KIND>() workgroups fit on a CU.
template <int KIND>
constexpr unsigned occupancy_pad(int static_bytes) {
    const int limit = occupancy_limit<KIND>();
    if (limit <= 0) return 0;
    // floor(kLdsPerCu / per_wg) == limit for per_wg = kLdsPerCu / limit, and
    // rounding the pad up can only lower the count further.
    const int per_wg = kLdsPerCu / limit;
    return static_cast<unsigned>(per_wg > static_bytes ? (per_wg - static_bytes + 511) / 512 * 512 : 0);
}

// How a kernel fills the LDS tile: through registers into swizzled (or
// plain) rows, through registers into padded rows, or by direct loads into
// swizzled (or plain) rows.
enum Fill { kRegs = 0, kPadded = 1, kDirect = 2 };

template <int KIND, int FILL>
struct LdsTile {
    using K = Kind<KIND>;
    // The padded layout adds one element (element-wide LDS stores) or one
    // LDS store's width per row.
    static constexpr int PAD = K::VEC == K::ESZ ? 1 : K::VEC / K::ESZ;
    static constexpr int BYTES = K::TR * (K::TC + (FILL == kPadded ? PAD : 0)) * K::ESZ;
};

// Element offset in LDS of step i of this lane: the lane's first offset
// `base` combined with the step's lane-independent move (see steps_decompose).
// PADDED: rows of L.ld = TC + PAD elements, offsets add.  Otherwise rows of
// TC elements under Swizzle<B,M,S> (B = 0: plain rows), offsets combine by
// XOR.  Either way the move is one value shared by the wave; the row pitch
// is a run-time value in both, so the three layouts issue the same LDS
// instructions (no pairing into two-address forms for one of them) and
// differ only in the addresses.
template <int KIND, bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t step_off(uint32_t base, int i, const LdsLayout& L) {
    using K = Kind<KIND>;
    int dr = 0, dc = 0;
    coord<KIND, WRITE>(0, i, dr, dc);
    if (PADDED) {
        uint32_t d = static_cast<uint32_t>(dr) * L.ld + static_cast<uint32_t>(dc);
        asm volatile("" : "+s"(d));  // keep the move opaque: no two-address pairing
        return base + d;
    }
    return base ^ swizzle(static_cast<uint32_t>(dr * K::TC + dc), L.B, L.M, L.S);
}

template <int KIND, bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t lane_base(int t, const LdsLayout& L) {
    using K = Kind<KIND>;
    int r = 0, c = 0;
    coord<KIND, WRITE>(t, 0, r, c);
    if (PADDED) return static_cast<uint32_t>(r) * L.ld + static_cast<uint32_t>(c);
    return swizzle(static_cast<uint32_t>(r * K::TC + c), L.B, L.M, L.S);
}

// Direct fill of one tile (see Direct in swz_common.h): each load writes
// VB bytes per lane to consecutive LDS slots starting at a wave-uniform
// address, and the lane fetches the tile element the swizzled layout keeps in
// its slot.  rows x cols is the source matrix (r0, c0 the tile's corner);
// with FULL false, slots whose element lies outside the matrix are filled
// from the tile's corner element instead, which is always inside and never
// stored.  Rows must be 16-byte aligned for 2-byte elements, so a 16-byte
// slot is wholly inside or wholly outside.  Waits for its own loads; the
// caller's barrier then publishes the tile.
template <int KIND, bool FULL>
__device__ __forceinline__ void direct_fill(const uint8_t* __restrict__ S, int64_t rows, int64_t cols, int64_t r0,
                                            int64_t c0, uint8_t* lds, const LdsLayout& L, int t) {
    using K = Kind<KIND>;
    using D = Direct<KIND>;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const uint32_t base = swizzle(static_cast<uint32_t>(D::EPL * t), L.B, L.M, L.S);
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
#pragma unroll
    for (int j = 0; j < D::LOADS; ++j) {
        const uint32_t e = base ^ swizzle(static_cast<uint32_t>(D::EPL * K::NT * j), L.B, L.M, L.S);
        const int64_t r = r0 + static_cast<int64_t>(e / K::TC), c = c0 + static_cast<int64_t>(e % K::TC);
        const uint8_t* g = (FULL || (r < rows && c < cols)) ? S + (r * cols + c) * K::ESZ : S + (r0 * cols + c0) * K::ESZ;
        lds_u8* slot = (lds_u8*)lds + D::VB * (64 * wave + K::NT * j);
        __builtin_amdgcn_global_load_lds(g, slot, D::VB, 0, SWZ_NONTEMPORAL ? kDirectNT : 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Transpose / layout conversion of one tile.
// ---------------------------------------------------------------------------

// Global loads of one tile into registers, guarded at the matrix edge as EDGE
// says (Edge above).
template <int KIND, int EDGE>
__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ S, int64_t rows, int64_t cols, int64_t r0,
                                          int64_t c0, int t, u32x4* v) {
    using K = Kind<KIND>;
    constexpr int PER = 16 / K::ESZ;  // elements per global load
#pragma unroll
    for (int j = 0; j < K::GLOADS; ++j) {
        int r = 0, c = 0;
        K::wcoord(t, j * (K::WSTEPS / K::GLOADS), r, c);
        c -= c % PER;  // the vector's first column
        if (is_narrow(KIND))  // whole-row tiles: a vector may span rows, guard the flat index
            v[j] = load16_edge<EDGE, K::ESZ>(S, 0, (r0 + r) * cols + c0 + c, 1, rows * cols);
        else
            v[j] = load16_edge<EDGE, K::ESZ>(S, r0 + r, c0 + c, rows, cols);
    }
}

template <int KIND, bool PADDED>
__device__ __forceinline__ void lds_store(uint8_t* lds, uint32_t wbase, const LdsLayout& L, const u32x4* v) {
    using K = Kind<KIND>;
    if constexpr (K::VEC == 4 && K::ESZ < 4) {
        // Narrow rows of 2- or 1-byte elements: 4-byte runs (M >= 1 resp. 2
        // keeps them together); step 4j + e writes word e ^ s of the vector,
        // s = bits 3-4 of the lane for the wide rows (SWAP, lane map in
        // swz_common.h), picked with two 2-way selects.  Those steps combine
        // by XOR only, so padded rows compute each step's row and column.
        const int t = threadIdx.x;
        const bool sw1 = K::SWAP && ((t >> 3) & 1), sw2 = K::SWAP && ((t >> 4) & 1);
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t off;
                if constexpr (PADDED) {
                    int r = 0, c = 0;
                    K::wcoord(t, 4 * j + e, r, c);
                    off = static_cast<uint32_t>(r) * L.ld + static_cast<uint32_t>(c);
                } else {
                    off = step_off<KIND, true, false>(wbase, 4 * j + e, L);
                }
                const uint32_t lo = sw1 ? v[j][e ^ 1] : v[j][e], hi = sw1 ? v[j][e ^ 3] : v[j][e ^ 2];
                *reinterpret_cast<uint32_t*>(lds + K::ESZ * off) = sw2 ? hi : lo;
            }
        }
    } else if constexpr (K::VEC == 4) {
        // 4-byte elements, one per write
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                reinterpret_cast<uint32_t*>(lds)[step_off<KIND, true, PADDED>(wbase, 4 * j + e, L)] = v[j][e];
        }
    } else if constexpr (K::ESZ == 1) {
        // Two 8-byte writes per 16-byte vector (the swizzle keeps 8-byte
        // runs); step 2j + h writes half h ^ (row % 2) (lane map in
        // swz_common.h).  The steps combine by XOR only, so padded rows
        // compute each step's row and column.
        const int t = threadIdx.x;
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t off;
                if constexpr (PADDED) {
                    int r = 0, c = 0;
                    K::wcoord(t, 2 * j + h, r, c);
                    off = static_cast<uint32_t>(r) * L.ld + static_cast<uint32_t>(c);
                } else {
                    off = step_off<KIND, true, false>(wbase, 2 * j + h, L);
                }
                int r0 = 0, c0 = 0;
                K::wcoord(t, 2 * j, r0, c0);
                const int half = (c0 / 8) % 2 ^ h;  // which half of the vector this step writes
                *reinterpret_cast<u32x2*>(lds + off) = half ? u32x2{v[j][2], v[j][3]} : u32x2{v[j][0], v[j][1]};
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j)
            *reinterpret_cast<u32x4*>(lds + 2 * step_off<KIND, true, PADDED>(wbase, j, L)) = v[j];
    }
}

// Read this thread's pieces of the tile back from LDS, transposed, and store
// them to the output, guarded at the matrix edge as EDGE says.
template <int KIND, bool PADDED, int EDGE>
__device__ __forceinline__ void lds_read_store(const uint8_t* lds, uint32_t rbase, const LdsLayout& L,
                                               uint8_t* __restrict__ D, int64_t rows, int64_t cols, int64_t r0,
                                               int64_t c0, int t) {
    using K = Kind<KIND>;
    if constexpr (K::ESZ == 4 && (KIND == SWZ_READ_SCALAR_COL || is_narrow(KIND))) {
        // Task j: four rows of one source column -> 16 bytes of an output row.
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = reinterpret_cast<const uint32_t*>(lds)[step_off<KIND, false, PADDED>(rbase, 4 * j + e, L)];
            int r = 0, c = 0;
            K::rcoord(t, 4 * j, r, c);
            const int64_t orow = c0 + c, ocol = r0 + r;
            // Assembled from four loads, the vector is otherwise rebuilt at
            // the store in a way that drops the store's non-temporal hint.
            asm volatile("" : "+v"(o));
            store16_edge<EDGE, 4>(D, orow, ocol, cols, rows, o);
        }
    } else if constexpr (narrow_by_element<KIND>()) {
        // Narrow rows of 2-byte elements read an element at a time: PER rows
        // of one column packed into 16 bytes of one output row.
        constexpr int PER = K::PER;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t x = *reinterpret_cast<const uint16_t*>(lds + 2 * step_off<KIND, false, PADDED>(rbase, e, L));
            w[e / 2] |= x << (16 * (e % 2));
        }
        u32x4 o{w[0], w[1], w[2], w[3]};
        int r = 0, c = 0;
        K::rcoord(t, 0, r, c);
        asm volatile("" : "+v"(o));
        store16_edge<EDGE, 2>(D, c0 + c, r0 + r, cols, rows, o);
    } else if constexpr (is_narrow(KIND)) {
        // Narrow rows of 2- or 1-byte elements: the lane's block of PER rows
        // and CB columns arrives as RSTEPS whole words (EPW columns of one
        // row each, or RPW whole rows of C columns); piece j gathers column
        // CB*g + j of the PER rows, element q from word q / RPW at position
        // (q % RPW) * C + j, into 16 bytes of one output row.
        constexpr int E = K::ESZ, EPW = K::EPW, CB = K::CB, RPW = K::RPW, C = K::TC;
        constexpr uint32_t kMask = E == 2 ? 0xffffu : 0xffu;
        uint32_t w[K::RSTEPS];
#pragma unroll
        for (int i = 0; i < K::RSTEPS; ++i)
            w[i] = *reinterpret_cast<const uint32_t*>(lds + E * step_off<KIND, false, PADDED>(rbase, i, L));
        int r = 0, c = 0;
        K::rcoord(t, 0, r, c);
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            u32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t x = 0u;
#pragma unroll
                for (int p = 0; p < EPW; ++p) {
                    const int q = d * EPW + p;  // row within the block
                    const int pos = (q % RPW) * C + j;
                    x |= ((w[q / RPW] >> (8 * E * pos)) & kMask) << (8 * E * p);
                }
                o[d] = x;
            }
            asm volatile("" : "+v"(o));
            store16_edge<EDGE, E>(D, c0 + c + j, r0 + r, cols, rows, o);
        }
    } else if constexpr (KIND == SWZ_READ_B64_TR8) {
        // Task j: in each of two steps h the 8-bit transpose read gives this
        // lane rows 64h + 16g + 8(q/8) .. +7 of one column (the lane map in
        // swz_common.h).  Lanes q and q+8 of a 16-lane group hold the two
        // 8-row halves of the same 16 rows; they swap one piece (a DPP
        // rotate by 8 within the row of 16 lanes) so that lane q ends up
        // with rows 16g .. 16g + 15 and lane q+8 with rows 64 + 16g .. +15:
        // one 16-byte output piece each, eight lanes per 128-byte output row.
        typedef int v2i32 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
        const int l = t % 64, g = l / 16, q = l % 16;
        const bool upper = q >= 8;
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            const int ch = t / 64 + (K::NT / 64) * j;
            u32x2 h[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint32_t off = step_off<KIND, false, PADDED>(rbase, 2 * j + s, L);
                h[s] = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)((__attribute__((address_space(3))) uint8_t*)lds + off)));
            }
            // lane q < 8 sends its step-1 piece and keeps step 0; lane q >= 8
            // sends step 0 and keeps step 1
            const u32x2 send = upper ? h[0] : h[1];
            u32x2 got;
            got[0] = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send[0]), 0x128, 0xf, 0xf, false));
            got[1] = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(send[1]), 0x128, 0xf, 0xf, false));
            const u32x4 o = upper ? u32x4{got[0], got[1], h[1][0], h[1][1]} : u32x4{h[0][0], h[0][1], got[0], got[1]};
            const int64_t orow = c0 + 8 * ch + q % 8;
            const int64_t ocol = r0 + (upper ? 64 : 0) + 16 * g;
            store16_edge<EDGE, 1>(D, orow, ocol, cols, rows, o);
        }
    } else if constexpr (KIND == SWZ_READ_B64_TR16) {
        // Task j: two transpose reads give this lane 8 consecutive rows of
        // one column (the lane map in swz_common.h); odd 16-lane groups read
        // their upper four rows first, so their halves are swapped back.
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const int l = t % 64, g = l / 16, q = l % 16;
        const bool odd = g & 1;
        int lr0 = 0, lc0 = 0;
        K::rcoord(t, 0, lr0, lc0);
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            u32x2 h[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                uint32_t off;
                if constexpr (PADDED) {
                    int dr = 0, dc = 0;
                    K::rcoord(0, 2 * j + s, dr, dc);
                    off = static_cast<uint32_t>(lr0 ^ dr) * L.ld + static_cast<uint32_t>(lc0 ^ dc);
                } else {
                    off = step_off<KIND, false, false>(rbase, 2 * j + s, L);
                }
                const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((__attribute__((address_space(3))) uint8_t*)lds + 2 * off));
                h[s] = __builtin_bit_cast(u32x2, v);
            }
            const u32x2 lo = odd ? h[1] : h[0], hi = odd ? h[0] : h[1];
            const u32x4 o{lo[0], lo[1], hi[0], hi[1]};
            const int ch = t / 64 + (K::NT / 64) * j;
            const int64_t orow = c0 + 8 * ch + 4 * ((q / 4) % 2) + q % 4;
            const int64_t ocol = r0 + 16 * g + 8 * (q / 8);
            store16_edge<EDGE, 2>(D, orow, ocol, cols, rows, o);
        }
    } else {
        // Task j: 8 rows of a column block; transpose 16-bit elements in
        // registers and write one 16-byte piece of each output row.
        using R = typename std::conditional<K::RWIDTH == 8, u32x2, u32x4>::type;
        constexpr int kCols = K::RWIDTH / 2;
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            R x[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                x[s] = *reinterpret_cast<const R*>(lds + 2 * step_off<KIND, false, PADDED>(rbase, 8 * j + s, L));
            int rb = 0, cb = 0;
            K::rcoord(t, 8 * j, rb, cb);
#pragma unroll
            for (int q = 0; q < kCols; ++q) {
                const u32x4 o{pair_col(x[0], x[1], q), pair_col(x[2], x[3], q), pair_col(x[4], x[5], q),
                              pair_col(x[6], x[7], q)};
                const int64_t orow = c0 + cb + q, ocol = r0 + rb;
                store16_edge<EDGE, 2>(D, orow, ocol, cols, rows, o);
            }
        }
    }
}

template <int KIND, int FILL, int EDGE>
__device__ __forceinline__ void convert_tile(const uint8_t* __restrict__ S, uint8_t* __restrict__ D, int64_t rows,
                                             int64_t cols, int64_t r0, int64_t c0, uint8_t* lds, uint32_t wbase,
                                             uint32_t rbase, const LdsLayout& L, int t) {
    using K = Kind<KIND>;
    constexpr bool PADDED = FILL == kPadded;
    if constexpr (FILL == kDirect) {
        static_assert(EDGE != kElem, "the direct fill needs 16-byte aligned rows");
        direct_fill<KIND, EDGE == kFull>(S, rows, cols, r0, c0, lds, L, t);
    } else {
        u32x4 v[K::GLOADS];
        load_tile<KIND, EDGE>(S, rows, cols, r0, c0, t, v);
        lds_store<KIND, PADDED>(lds, wbase, L, v);
    }
    __syncthreads();
    lds_read_store<KIND, PADDED, EDGE>(lds, rbase, L, D, rows, cols, r0, c0, t);
}

// Which tile this workgroup moves.  GRID3D: blockIdx = (tile row, tile
// column step, batch entry), the diagonal order needing one 32-bit modulo;
// otherwise a 1-D chunk of the linear tile order (grids beyond the
// hardware's y / z limits).
template <bool DIAGONAL, bool GRID3D>
__device__ __forceinline__ void my_tile(int64_t tiles_r, int64_t tiles_c, int64_t tile0, TileOrder O, int64_t& b,
                                        int64_t& tr, int64_t& tc) {
    if (GRID3D) {
        b = blockIdx.z;
        if (DIAGONAL) {
            const uint32_t n = static_cast<uint32_t>(tiles_c);
            tr = blockIdx.x;
            tc = static_cast<int64_t>((blockIdx.y + ((blockIdx.x * O.num) >> O.sh) % n) % n);
        } else {
            tc = blockIdx.x;
            tr = blockIdx.y;
        }
    } else {
        decode_tile<DIAGONAL>(tile0 + blockIdx.x, tiles_r, tiles_c, O, b, tr, tc);
    }
}

template <int KIND, int FILL, bool ALIGNED, bool GRID3D>
__global__ __launch_bounds__(Kind<KIND>::NT) void k_convert(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int64_t rows, int64_t cols, int64_t tiles_r,
                                                            int64_t tiles_c, int64_t tile0, LdsLayout L,
                                                            TileOrder O) {
    using K = Kind<KIND>;
    constexpr bool PADDED = FILL == kPadded;
    static_assert(FILL != kDirect || ALIGNED, "the direct fill needs 16-byte aligned rows");
    __shared__ u32x4 lds_v[(LdsTile<KIND, FILL>::BYTES + 15) / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v);
    const int t = threadIdx.x;
    const int64_t plane = rows * cols * K::ESZ;  // bytes of one batch entry
    const uint32_t wbase = FILL == kDirect ? 0u : lane_base<KIND, true, PADDED>(t, L);
    const uint32_t rbase = lane_base<KIND, false, PADDED>(t, L);

    int64_t b, tr, tc;
    my_tile<SWZ_TILE_ORDER != 0, GRID3D>(tiles_r, tiles_c, tile0, O, b, tr, tc);
    const int64_t r0 = tr * K::TR, c0 = tc * K::TC;
    const uint8_t* S = src + b * plane;
    uint8_t* D = dst + b * plane;
    if constexpr (ALIGNED) {
        if (r0 + K::TR <= rows && c0 + K::TC <= cols)
            convert_tile<KIND, FILL, kFull>(S, D, rows, cols, r0, c0, lds, wbase, rbase, L, t);
        else
            convert_tile<KIND, FILL, kVec>(S, D, rows, cols, r0, c0, lds, wbase, rbase, L, t);
    } else {
        convert_tile<KIND, FILL, kElem>(S, D, rows, cols, r0, c0, lds, wbase, rbase, L, t);
    }
}

// ---------------------------------------------------------------------------
// Operand staging: 256x64 K-tiles of a K-contiguous 16-bit operand, read
// back as 16x16x32 operand fragments and written out in lane order.
// ---------------------------------------------------------------------------
template <int FILL, bool FULL>
__device__ __forceinline__ void stage_tile(const uint8_t* __restrict__ src, uint8_t* __restrict__ frag, int64_t mn,
                                           int64_t k, int64_t r0, int64_t k0, uint8_t* lds, uint32_t wbase,
                                           uint32_t rbase, const LdsLayout& L, int t) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    constexpr bool PADDED = FILL == kPadded;
    using K = Kind<KD>;
    if constexpr (FILL == kDirect) {
        direct_fill<KD, FULL>(src, mn, k, r0, k0, lds, L, t);
    } else {
        u32x4 v[K::GLOADS];
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
            int r = 0, c = 0;
            K::wcoord(t, j, r, c);
            // mn and k are multiples of 16 and 32, so a 16-byte chunk is either
            // wholly inside the operand or wholly outside.
            v[j] = (FULL || (r0 + r < mn && k0 + c < k)) ? gload16(src + ((r0 + r) * k + k0 + c) * 2)
                                                         : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j)
            *reinterpret_cast<u32x4*>(lds + 2 * step_off<KD, true, PADDED>(wbase, j, L)) = v[j];
    }
    __syncthreads();
    const int64_t ksteps = k / 32;
    const int lane = t % 64;
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        const int f = K::frag_of(t, i);
        const int blk = f % 16, ks = f / 16;
        const u32x4 x = *reinterpret_cast<const u32x4*>(lds + 2 * step_off<KD, false, PADDED>(rbase, i, L));
        if (FULL || (r0 + 16 * blk < mn && k0 + 32 * ks < k)) {
            const int64_t fi = (r0 / 16 + blk) * ksteps + (k0 / 32 + ks);
            gstore16(frag + (fi * 64 + lane) * 16, x);
        }
    }
}

template <int FILL, bool GRID3D>
__global__ __launch_bounds__(Kind<SWZ_READ_MFMA_16X16X32>::NT) void k_stage(const uint8_t* __restrict__ src,
                                                                            uint8_t* __restrict__ frag, int64_t mn,
                                                                            int64_t k, int64_t tiles_m,
                                                                            int64_t tiles_k, int64_t tile0,
                                                                            LdsLayout L) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    constexpr bool PADDED = FILL == kPadded;
    using K = Kind<KD>;
    __shared__ u32x4 lds_v[LdsTile<KD, FILL>::BYTES / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v);
    const int t = threadIdx.x;
    const uint32_t wbase = FILL == kDirect ? 0u : lane_base<KD, true, PADDED>(t, L);
    const uint32_t rbase = lane_base<KD, false, PADDED>(t, L);

    int64_t b, tm, tk;
    my_tile<SWZ_STAGE_ORDER != 0, GRID3D>(tiles_m, tiles_k, tile0, TileOrder{1u, 0u}, b, tm, tk);
    const int64_t r0 = tm * K::TR, k0 = tk * K::TC;
    if (r0 + K::TR <= mn && k0 + K::TC <= k)
        stage_tile<FILL, true>(src, frag, mn, k, r0, k0, lds, wbase, rbase, L, t);
    else
        stage_tile<FILL, false>(src, frag, mn, k, r0, k0, lds, wbase, rbase, L, t);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Grid limits of a 3-D launch: work-items along x below 2^31, y and z up to
// 65535 workgroups.
bool fits_3d(int64_t x, int64_t y, int64_t z, int threads) {
    return SWZ_GRID3D && x * threads < (int64_t(1) << 31) && y <= 65535 && z <= 65535;
}

template <int KIND, int FILL, bool ALIGNED>
void launch_variant(const ConvertJob& j, int64_t tiles_r, int64_t tiles_c, int64_t n_tiles, hipStream_t stream) {
    using K = Kind<KIND>;
    const auto* s = static_cast<const uint8_t*>(j.src);
    auto* d = static_cast<uint8_t*>(j.dst);
    const bool diag = SWZ_TILE_ORDER != 0;
    const int64_t gx = diag ? tiles_r : tiles_c, gy = diag ? tiles_c : tiles_r;
    // slope of the diagonal order per SWZ_ORDER_* value: 1, 1/2, 0, 3
    static constexpr TileOrder kOrders[4] = {{1u, 0u}, {1u, 1u}, {0u, 0u}, {3u, 0u}};
    const TileOrder O = kOrders[j.order >= 0 && j.order < 4 ? j.order : 0];
    if (fits_3d(gx, gy, j.batch, K::NT)) {
        hipLaunchKernelGGL((k_convert<KIND, FILL, ALIGNED, true>),
                           dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy), static_cast<unsigned>(j.batch)),
                           dim3(K::NT), occupancy_pad<KIND>(LdsTile<KIND, FILL>::BYTES), stream, s, d, j.rows, j.cols,
                           tiles_r, tiles_c, int64_t(0), j.layout, O);
        return;
    }
    for (int64_t t0 = 0; t0 < n_tiles; t0 += kMaxGrid) {
        const int64_t n = n_tiles - t0 < kMaxGrid ? n_tiles - t0 : kMaxGrid;
        hipLaunchKernelGGL((k_convert<KIND, FILL, ALIGNED, false>), dim3(static_cast<unsigned>(n)), dim3(K::NT),
                           occupancy_pad<KIND>(LdsTile<KIND, FILL>::BYTES),
                           stream, s, d, j.rows, j.cols, tiles_r, tiles_c, t0, j.layout, O);
    }
}

template <int KIND>
hipError_t launch_kind(const ConvertJob& j, hipStream_t stream) {
    using K = Kind<KIND>;
    const int64_t tiles_r = ceil_div(j.rows, K::TR), tiles_c = ceil_div(j.cols, K::TC);
    const int64_t n_tiles = j.batch * tiles_r * tiles_c;
    if (n_tiles == 0) return hipSuccess;
    const bool padded = j.layout.ld != static_cast<uint32_t>(K::TC);
    if (padded && j.layout.ld != static_cast<uint32_t>(K::TC + LdsTile<KIND, kPadded>::PAD)) return hipErrorInvalidValue;
    if (j.direct) {
        if (padded || !j.aligned) return hipErrorInvalidValue;
        launch_variant<KIND, kDirect, true>(j, tiles_r, tiles_c, n_tiles, stream);
    } else if (padded) {
        // no padded rows narrower than one 4-byte LDS write
        if constexpr (is_narrow(KIND) && K::TC * K::ESZ < 4) {
            return hipErrorInvalidValue;
        } else {
            if (j.aligned)
                launch_variant<KIND, kPadded, true>(j, tiles_r, tiles_c, n_tiles, stream);
            else
                launch_variant<KIND, kPadded, false>(j, tiles_r, tiles_c, n_tiles, stream);
        }
    } else {
        if (j.aligned)
            launch_variant<KIND, kRegs, true>(j, tiles_r, tiles_c, n_tiles, stream);
        else
            launch_variant<KIND, kRegs, false>(j, tiles_r, tiles_c, n_tiles, stream);
    }
    return hipGetLastError();
}

template <int FILL>
void launch_stage_fill(const StageJob& j, int64_t tiles_m, int64_t tiles_k, hipStream_t stream) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    using K = Kind<KD>;
    const auto* s = static_cast<const uint8_t*>(j.src);
    auto* f = static_cast<uint8_t*>(j.frag);
    const bool diag = SWZ_STAGE_ORDER != 0;
    const int64_t gx = diag ? tiles_m : tiles_k, gy = diag ? tiles_k : tiles_m;
    if (fits_3d(gx, gy, 1, K::NT)) {
        hipLaunchKernelGGL((k_stage<FILL, true>), dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy), 1),
                           dim3(K::NT), occupancy_pad<KD>(LdsTile<KD, FILL>::BYTES), stream, s, f, j.mn, j.k, tiles_m, tiles_k, int64_t(0), j.layout);
        return;
    }
    const int64_t n_tiles = tiles_m * tiles_k;
    for (int64_t t0 = 0; t0 < n_tiles; t0 += kMaxGrid) {
        const dim3 grid(static_cast<unsigned>(n_tiles - t0 < kMaxGrid ? n_tiles - t0 : kMaxGrid));
        hipLaunchKernelGGL((k_stage<FILL, false>), grid, dim3(K::NT), occupancy_pad<KD>(LdsTile<KD, FILL>::BYTES), stream,
                           s, f, j.mn, j.k, tiles_m, tiles_k,
                           t0, j.layout);
    }
}

}  // namespace

hipError_t launch_convert(int kind, const ConvertJob& j, hipStream_t stream) {
    switch (kind) {
        case SWZ_READ_SCALAR_COL: return launch_kind<SWZ_READ_SCALAR_COL>(j, stream);
        case SWZ_READ_B64_4X4: return launch_kind<SWZ_READ_B64_4X4>(j, stream);
        case SWZ_READ_B128_8X8: return launch_kind<SWZ_READ_B128_8X8>(j, stream);
        case SWZ_READ_B64_TR16: return launch_kind<SWZ_READ_B64_TR16>(j, stream);
        case SWZ_READ_B64_TR8: return launch_kind<SWZ_READ_B64_TR8>(j, stream);
        case SWZ_READ_NARROW1: return launch_kind<SWZ_READ_NARROW1>(j, stream);
        case SWZ_READ_NARROW2: return launch_kind<SWZ_READ_NARROW2>(j, stream);
        case SWZ_READ_NARROW4: return launch_kind<SWZ_READ_NARROW4>(j, stream);
        case SWZ_READ_NARROW8: return launch_kind<SWZ_READ_NARROW8>(j, stream);
        case SWZ_READ_NARROW16: return launch_kind<SWZ_READ_NARROW16>(j, stream);
        case SWZ_READ_HNARROW1: return launch_kind<SWZ_READ_HNARROW1>(j, stream);
        case SWZ_READ_HNARROW2: return launch_kind<SWZ_READ_HNARROW2>(j, stream);
        case SWZ_READ_HNARROW4: return launch_kind<SWZ_READ_HNARROW4>(j, stream);
        case SWZ_READ_HNARROW8: return launch_kind<SWZ_READ_HNARROW8>(j, stream);
        case SWZ_READ_HNARROW16: return launch_kind<SWZ_READ_HNARROW16>(j, stream);
        case SWZ_READ_HNARROW32: return launch_kind<SWZ_READ_HNARROW32>(j, stream);
        case SWZ_READ_BNARROW1: return launch_kind<SWZ_READ_BNARROW1>(j, stream);
        case SWZ_READ_BNARROW2: return launch_kind<SWZ_READ_BNARROW2>(j, stream);
        case SWZ_READ_BNARROW4: return launch_kind<SWZ_READ_BNARROW4>(j, stream);
        case SWZ_READ_BNARROW8: return launch_kind<SWZ_READ_BNARROW8>(j, stream);
        case SWZ_READ_BNARROW16: return launch_kind<SWZ_READ_BNARROW16>(j, stream);
        case SWZ_READ_BNARROW32: return launch_kind<SWZ_READ_BNARROW32>(j, stream);
        case SWZ_READ_BNARROW64: return launch_kind<SWZ_READ_BNARROW64>(j, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stage(const StageJob& j, hipStream_t stream) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    using K = Kind<KD>;
    const int64_t tiles_m = ceil_div(j.mn, K::TR), tiles_k = ceil_div(j.k, K::TC);
    if (tiles_m * tiles_k == 0) return hipSuccess;
    const bool padded = j.layout.ld != static_cast<uint32_t>(K::TC);
    if (padded && j.layout.ld != static_cast<uint32_t>(K::TC + LdsTile<KD, kPadded>::PAD)) return hipErrorInvalidValue;
    if (j.direct) {
        if (padded) return hipErrorInvalidValue;
        launch_stage_fill<kDirect>(j, tiles_m, tiles_k, stream);
    } else if (padded) {
        launch_stage_fill<kPadded>(j, tiles_m, tiles_k, stream);
    } else {
        launch_stage_fill<kRegs>(j, tiles_m, tiles_k, stream);
    }
    return hipGetLastError();
}

}  // namespace swz
