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
// once and written once.  The whole-tile launch of the 64 x 64 16-bit tiles
// and of staging moves two or four tiles per workgroup, so that the HBM
// runs are longer (interior_stack).
#include <tuple>
#include <type_traits>

#include "launch.h"

namespace swz {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Workgroups per 1-D launch; larger jobs are launched in chunks.  A
// workgroup moves its tile (or the interior's stacked tiles) in one round,
// with no loop in the kernel, so nothing is kept live across tiles.
constexpr int64_t kMaxGrid = int64_t(1) << 22;

// Cache-policy operand of the direct load for a non-temporal access.
constexpr int kDirectNT = 2;

// Every byte is read once and written once: non-temporal 16-byte accesses.
__device__ __forceinline__ u32x4 gload16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void gstore16(uint8_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// The same through the caches (CACHED), for matrices whose row pitches are
// not whole multiples of 64 bytes: two workgroups then share the lines at
// each tile edge, and the pieces written by one meet the other's in L2
// (see kBlocksXcd) instead of reaching memory as partial lines.
template <bool CACHED>
__device__ __forceinline__ u32x4 gload16c(const uint8_t* p) {
    if constexpr (CACHED) return *reinterpret_cast<const u32x4*>(p);
    else return gload16(p);
}
template <bool CACHED>
__device__ __forceinline__ void gstore16c(uint8_t* p, u32x4 v) {
    if constexpr (CACHED) *reinterpret_cast<u32x4*>(p) = v;
    else gstore16(p, v);
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

// 16 bytes of a row whose pitch (or base) is not a multiple of 16 bytes,
// accessed as one 16-byte vector anyway: compute queues on this GPU run in
// the unaligned memory access mode, and the compiler emits a single dwordx4
// for an access that only promises byte alignment.  For 1- and 2-byte
// elements that replaces 16 or 8 accesses by one (bytes 5800 x 5800: 0.13 ->
// 0.38 of a copy; fp16 5801 x 5801: 0.20 -> 0.35).  4-byte elements keep
// their four aligned dword accesses with non-temporal accesses (fp32 4001 x
// 4001: 0.44 against 0.37 with vectors), but take the vector too on the
// cached XCD-grouped grid, where it is the faster (0.45 -> 0.64).
typedef u32x4 __attribute__((aligned(1))) u32x4_unaligned;

// 16 bytes = 16/ESZ consecutive elements of one row, zero outside the matrix.
template <int ESZ, bool CACHED = false>
__device__ __forceinline__ u32x4 load16_guarded(const uint8_t* S, int64_t row, int64_t col, int64_t rows,
                                                int64_t cols) {
    constexpr int N = 16 / ESZ;
    if ((ESZ < 4 || CACHED) && row < rows && col + N <= cols) {
        const auto* p = reinterpret_cast<const u32x4_unaligned*>(S + (row * cols + col) * ESZ);
        if constexpr (CACHED) return *p;
        else return __builtin_nontemporal_load(p);
    }
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
template <int ESZ, bool CACHED = false>
__device__ __forceinline__ void store16_guarded(uint8_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                                const u32x4& o) {
    if (row >= nrows) return;
    if ((ESZ < 4 || CACHED) && col + 16 / ESZ <= ncols) {
        auto* p = reinterpret_cast<u32x4_unaligned*>(D + (row * ncols + col) * ESZ);
        if constexpr (CACHED) *p = o;
        else __builtin_nontemporal_store(o, p);
        return;
    }
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

template <int EDGE, int ESZ, bool CACHED = false>
__device__ __forceinline__ u32x4 load16_edge(const uint8_t* S, int64_t row, int64_t col, int64_t rows,
                                             int64_t cols) {
    if constexpr (EDGE == kFull) return gload16c<CACHED>(S + (row * cols + col) * ESZ);
    if constexpr (EDGE == kVec)
        return row < rows && col < cols ? gload16c<CACHED>(S + (row * cols + col) * ESZ) : u32x4{0u, 0u, 0u, 0u};
    return load16_guarded<ESZ, CACHED>(S, row, col, rows, cols);
}

template <int EDGE, int ESZ, bool CACHED = false>
__device__ __forceinline__ void store16_edge(uint8_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                             u32x4 v) {
    if constexpr (EDGE == kFull) {
        gstore16c<CACHED>(D + (row * ncols + col) * ESZ, v);
    } else if constexpr (EDGE == kVec) {
        if (row < nrows && col < ncols) gstore16c<CACHED>(D + (row * ncols + col) * ESZ, v);
    } else {
        store16_guarded<ESZ, CACHED>(D, row, col, nrows, ncols, v);
    }
}

// The global side of one tile: its source pieces, in the tile's own
// coordinates (r, c) = source element (r0 + r, c0 + c), and its output
// pieces (orow, ocol) = output element (c0 + orow, r0 + ocol).  A whole tile
// (kFull) keeps two wave-uniform base pointers, the tile's first source and
// output elements, and 32-bit row pitches from the host: a lane's address is
// one 32 x 32 -> 64-bit multiply-add.  Edge tiles (and matrices whose sizes
// need 64 bits) index the matrix with 64-bit products, guarded as EDGE says.
//
// Why the whole-tile path is lean: a workgroup lives for one load and one
// store, and every wave runs the tile's address arithmetic on its CU's one
// scalar unit before its first load.  Measured on MI355X (fp32 4096^2,
// 32x32 tiles): adding 32 / 64 / 128 dependent scalar multiplies ahead of
// the load lengthens the kernel by 1 / 3 / 3.5%, and a general prelude
// (64-bit tile bases and edge tests, the swizzle of every step from run-time
// (B, M, S)) cost the same 3.5%.
template <int EDGE, int ESZ, bool CACHED = false>
struct TileIo {
    const uint8_t* S;  // kFull: the tile's first source element; otherwise the source matrix
    uint8_t* D;        // kFull: the tile's first output element; otherwise the output matrix
    int64_t rows, cols, r0, c0;
    uint32_t sp, dp;  // kFull: source / output row pitch in bytes

    __device__ __forceinline__ const uint8_t* src(int r, int c) const {
        return S + (static_cast<uint64_t>(static_cast<uint32_t>(r)) * sp + static_cast<uint32_t>(c * ESZ));
    }
    __device__ __forceinline__ u32x4 load(int r, int c) const {
        if constexpr (EDGE == kFull) return gload16c<CACHED>(src(r, c));
        else return load16_edge<EDGE, ESZ, CACHED>(S, r0 + r, c0 + c, rows, cols);
    }
    // Whole-row tiles (cols == tile width, c0 = 0): a vector may span rows,
    // so the edge paths guard the flat index.
    __device__ __forceinline__ u32x4 load_flat(int r, int c) const {
        if constexpr (EDGE == kFull) return gload16c<CACHED>(src(r, c));
        else return load16_edge<EDGE, ESZ, CACHED>(S, 0, (r0 + r) * cols + c0 + c, 1, rows * cols);
    }
    __device__ __forceinline__ void store(int orow, int ocol, u32x4 v) const {
        if constexpr (EDGE == kFull)
            gstore16c<CACHED>(D + (static_cast<uint64_t>(static_cast<uint32_t>(orow)) * dp + static_cast<uint32_t>(ocol * ESZ)), v);
        else
            store16_edge<EDGE, ESZ, CACHED>(D, c0 + orow, r0 + ocol, cols, rows, v);
    }
};

// The whole-tile path of a launch, planned on the host: row pitches in bytes
// and the numbers of tile rows and columns whose tiles lie wholly inside the
// matrix; all zero (every tile takes a 64-bit edge path) when a size needs
// more than 32 bits.
struct FastPath {
    uint32_t sp, dp, full_r, full_c;
};

FastPath fast_path(int64_t batch, int64_t rows, int64_t cols, int esz, int tr, int tc) {
    const int64_t lim = int64_t(1) << 31;
    if (batch * rows >= lim || batch * cols >= lim || rows * esz >= 2 * lim || cols * esz >= 2 * lim)
        return FastPath{0u, 0u, 0u, 0u};
    return FastPath{static_cast<uint32_t>(cols * esz), static_cast<uint32_t>(rows * esz), static_cast<uint32_t>(rows / tr),
                    static_cast<uint32_t>(cols / tc)};
}

// Workgroups per CU.  The transposed HBM pattern of the 16-bit and 8-bit
// tiles runs faster with fewer tiles in flight (measured with an LDS-free
// probe of the same pattern: 64 x 64 16-bit tiles at 8 to 16 workgroups per
// CU 5.41-5.48 TB/s, at 4-5 per CU 5.69).  Each launch reserves extra LDS so
// that a CU holds at most this many workgroups of the kind (0: no limit).
// Values from a sweep of the kernels themselves (2 to 8 per CU): 4 for the
// 64-row 16-bit kinds (+3 to +8%), 5 for the byte kind (+4%); the fp32 tile
// loses bandwidth when limited, and staging's interior workgroups (four
// 8 KiB tiles, 1,024 threads) are held to two per CU by their waves.
// The byte tiles of 32 and 64 columns (16 KiB) are capped at 4 per CU (4%
// faster in a sweep of uncapped, 4 and 8); every other whole-row kind lost up
// to 20% when capped.
template <int KIND>
constexpr int occupancy_limit() {
    return KIND == SWZ_READ_B64_4X4 || KIND == SWZ_READ_B128_8X8 || KIND == SWZ_READ_B64_TR16 ? 4
           : KIND == SWZ_READ_B64_TR8                                  ? 5
           : (KIND == SWZ_READ_BNARROW32 || KIND == SWZ_READ_BNARROW64) ? 4
                                                                        : 0;
}

// Whole tiles per workgroup of a transpose's interior launch: stack_of()
// down the source rows times stack_c_of() along them (interior_stack).
template <int KIND>
constexpr int stack_of() {
    return interior_stack(KIND);
}
template <int KIND>
constexpr int stack_c_of() {
    return interior_stack_cols(KIND);
}

// Workgroups per CU of the interior launch (0: no limit): as many tiles in
// flight per CU as the single-tile limit allows (a sweep of 2 to 4 stacked
// 16-bit workgroups per CU found 2 and 3 alike, 4 slower).
template <int KIND>
constexpr int interior_occupancy_limit() {
    return occupancy_limit<KIND>() / (stack_of<KIND>() * stack_c_of<KIND>());
}

constexpr int kLdsPerCu = 160 * 1024;

// Dynamic LDS to add to a launch whose kernel uses `static_bytes` so that at
// most `limit` workgroups fit on a CU.
constexpr unsigned occupancy_pad_to(int static_bytes, int limit) {
    if (limit <= 0) return 0;
    // floor(kLdsPerCu / per_wg) == limit for per_wg = kLdsPerCu / limit, and
    // rounding the pad up can only lower the count further.
    const int per_wg = kLdsPerCu / limit;
    return static_cast<unsigned>(per_wg > static_bytes ? (per_wg - static_bytes + 511) / 512 * 512 : 0);
}

template <int KIND>
constexpr unsigned occupancy_pad(int static_bytes) {
    return occupancy_pad_to(static_bytes, occupancy_limit<KIND>());
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

// The LDS layout as the tile kernels take it: the row pitch (padded rows)
// and Swizzle<B,M,S> decoded on the host into x ^ (((x >> src) & mask) <<
// dst), so no wave re-derives masks and shifts from (B, M, S) (mask 0: plain
// rows, the identity).
struct KLayout {
    uint32_t ld, mask, src, dst;
};

__device__ __forceinline__ uint32_t kswizzle(uint32_t x, const KLayout& L) {
    return x ^ (((x >> L.src) & L.mask) << L.dst);
}

KLayout decode_layout(const LdsLayout& L) {
    const int32_t S = L.S;
    const uint32_t up = S >= 0 ? static_cast<uint32_t>(S) : 0u, dn = S >= 0 ? 0u : static_cast<uint32_t>(-S);
    uint32_t mask = L.B >= 32u ? 0xffffffffu : ((1u << L.B) - 1u);
    if (L.M + up >= 32u || L.M + dn >= 32u) mask = 0u;  // the moved field lies outside 32 bits: identity
    return KLayout{L.ld, mask, (L.M + up) & 31u, (L.M + dn) & 31u};
}

// Element offset in LDS of step i of this lane: the lane's first offset
// `base` combined with the step's wave-uniform move (StepMoves, computed on
// the host).  PADDED: rows of L.ld = TC + PAD elements, offsets add.
// Otherwise rows of TC elements under Swizzle<B,M,S> (B = 0: plain rows),
// offsets combine by XOR.  The three layouts issue the same LDS instructions
// and differ only in the addresses.
template <bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t step_off(uint32_t base, int i, const StepMoves& mv) {
    const uint32_t m = WRITE ? mv.w[i] : mv.r[i];
    return PADDED ? base + m : base ^ m;
}

template <int KIND, bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t lane_base(int t, const KLayout& L) {
    using K = Kind<KIND>;
    int r = 0, c = 0;
    coord<KIND, WRITE>(t, 0, r, c);
    if (PADDED) return static_cast<uint32_t>(r) * L.ld + static_cast<uint32_t>(c);
    return kswizzle(static_cast<uint32_t>(r * K::TC + c), L);
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
template <int KIND, int EDGE, bool CACHED>
__device__ __forceinline__ void direct_fill(const TileIo<EDGE, Kind<KIND>::ESZ, CACHED>& io, uint8_t* lds, const KLayout& L,
                                            const StepMoves& mv, int t) {
    using K = Kind<KIND>;
    using D = Direct<KIND>;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    const uint32_t base = kswizzle(static_cast<uint32_t>(D::EPL * t), L);
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
#pragma unroll
    for (int j = 0; j < D::LOADS; ++j) {
        const uint32_t e = base ^ mv.d[j];
        const int lr = static_cast<int>(e / K::TC), lc = static_cast<int>(e % K::TC);
        const uint8_t* g;
        if constexpr (EDGE == kFull) {
            g = io.src(lr, lc);
        } else {
            const int64_t r = io.r0 + lr, c = io.c0 + lc;
            g = r < io.rows && c < io.cols ? io.S + (r * io.cols + c) * K::ESZ : io.S + (io.r0 * io.cols + io.c0) * K::ESZ;
        }
        lds_u8* slot = (lds_u8*)lds + D::VB * (64 * wave + K::NT * j);
        __builtin_amdgcn_global_load_lds(g, slot, D::VB, 0, kDirectNT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Transpose / layout conversion of one tile.
// ---------------------------------------------------------------------------

// Global loads of one tile into registers, guarded at the matrix edge as EDGE
// says (Edge above).
template <int KIND, int EDGE, bool CACHED>
__device__ __forceinline__ void load_tile(const TileIo<EDGE, Kind<KIND>::ESZ, CACHED>& io, int t, u32x4* v) {
    using K = Kind<KIND>;
    constexpr int PER = 16 / K::ESZ;  // elements per global load
#pragma unroll
    for (int j = 0; j < K::GLOADS; ++j) {
        int r = 0, c = 0;
        K::wcoord(t, j * (K::WSTEPS / K::GLOADS), r, c);
        c -= c % PER;  // the vector's first column
        v[j] = is_narrow(KIND) ? io.load_flat(r, c) : io.load(r, c);
    }
}

// t: the thread's index within its tile (a stacked workgroup runs several
// tiles, each on its own NT threads).
template <int KIND, bool PADDED>
__device__ __forceinline__ void lds_store(uint8_t* lds, uint32_t wbase, const KLayout& L, const StepMoves& mv,
                                          const u32x4* v, int t) {
    using K = Kind<KIND>;
    if constexpr (K::VEC == 4 && K::ESZ < 4) {
        // Narrow rows of 2- or 1-byte elements: 4-byte runs (M >= 1 resp. 2
        // keeps them together); step 4j + e writes word e ^ s of the vector,
        // s = bits 3-4 of the lane for the wide rows (SWAP, lane map in
        // swz_common.h), picked with two 2-way selects.  Those steps combine
        // by XOR only, so padded rows compute each step's row and column.
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
                    off = step_off<true, false>(wbase, 4 * j + e, mv);
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
                reinterpret_cast<uint32_t*>(lds)[step_off<true, PADDED>(wbase, 4 * j + e, mv)] = v[j][e];
        }
    } else if constexpr (K::ESZ == 1) {
        // Two 8-byte writes per 16-byte vector (the swizzle keeps 8-byte
        // runs); step 2j + h writes half h ^ (row % 2) (lane map in
        // swz_common.h).  The steps combine by XOR only, so padded rows
        // compute each step's row and column.
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
                    off = step_off<true, false>(wbase, 2 * j + h, mv);
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
            *reinterpret_cast<u32x4*>(lds + 2 * step_off<true, PADDED>(wbase, j, mv)) = v[j];
    }
}

// Read this thread's pieces of the tile back from LDS, transposed, and store
// them to the output, guarded at the matrix edge as EDGE says.
template <int KIND, bool PADDED, int EDGE, bool CACHED>
__device__ __forceinline__ void lds_read_store(const uint8_t* lds, uint32_t rbase, const KLayout& L,
                                               const StepMoves& mv, const TileIo<EDGE, Kind<KIND>::ESZ, CACHED>& io,
                                               int t) {
    using K = Kind<KIND>;
    if constexpr (K::ESZ == 4 && (KIND == SWZ_READ_SCALAR_COL || is_narrow(KIND))) {
        // Task j: four rows of one source column -> 16 bytes of an output row.
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = reinterpret_cast<const uint32_t*>(lds)[step_off<false, PADDED>(rbase, 4 * j + e, mv)];
            int r = 0, c = 0;
            K::rcoord(t, 4 * j, r, c);
            // Assembled from four loads, the vector is otherwise rebuilt at
            // the store in a way that drops the store's non-temporal hint.
            asm volatile("" : "+v"(o));
            io.store(c, r, o);
        }
    } else if constexpr (narrow_by_element<KIND>()) {
        // Narrow rows of 2-byte elements read an element at a time: PER rows
        // of one column packed into 16 bytes of one output row.
        constexpr int PER = K::PER;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const uint32_t x = *reinterpret_cast<const uint16_t*>(lds + 2 * step_off<false, PADDED>(rbase, e, mv));
            w[e / 2] |= x << (16 * (e % 2));
        }
        u32x4 o{w[0], w[1], w[2], w[3]};
        int r = 0, c = 0;
        K::rcoord(t, 0, r, c);
        asm volatile("" : "+v"(o));
        io.store(c, r, o);
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
            w[i] = *reinterpret_cast<const uint32_t*>(lds + E * step_off<false, PADDED>(rbase, i, mv));
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
            io.store(c + j, r, o);
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
                const uint32_t off = step_off<false, PADDED>(rbase, 2 * j + s, mv);
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
            io.store(8 * ch + q % 8, (upper ? 64 : 0) + 16 * g, o);
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
                    off = step_off<false, false>(rbase, 2 * j + s, mv);
                }
                const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((__attribute__((address_space(3))) uint8_t*)lds + 2 * off));
                h[s] = __builtin_bit_cast(u32x2, v);
            }
            const u32x2 lo = odd ? h[1] : h[0], hi = odd ? h[0] : h[1];
            const u32x4 o{lo[0], lo[1], hi[0], hi[1]};
            const int ch = t / 64 + (K::NT / 64) * j;
            io.store(8 * ch + 4 * ((q / 4) % 2) + q % 4, 16 * g + 8 * (q / 8), o);
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
                x[s] = *reinterpret_cast<const R*>(lds + 2 * step_off<false, PADDED>(rbase, 8 * j + s, mv));
            int rb = 0, cb = 0;
            K::rcoord(t, 8 * j, rb, cb);
#pragma unroll
            for (int q = 0; q < kCols; ++q) {
                const u32x4 o{pair_col(x[0], x[1], q), pair_col(x[2], x[3], q), pair_col(x[4], x[5], q),
                              pair_col(x[6], x[7], q)};
                io.store(cb + q, rb, o);
            }
        }
    }
}

// A workgroup's waves live for one load-store round of their tile, so the
// loads go out first: the lanes' LDS addresses are computed while they
// are in flight.  (An empty asm on a copy of the thread index, ordered after
// the loads, keeps the compiler from hoisting that arithmetic above them;
// issuing the loads ahead of it measured 2% faster on the fp32 tile.)
__device__ __forceinline__ int after_loads(int t) {
    asm volatile("" : "+v"(t));
    __builtin_assume(t >= 0 && t < 1024);  // a thread index: unsigned arithmetic on it
    return t;
}

template <int KIND, int FILL, int EDGE, bool CACHED>
__device__ __forceinline__ void convert_tile(const TileIo<EDGE, Kind<KIND>::ESZ, CACHED>& io, uint8_t* lds, const KLayout& L,
                                             const StepMoves& mv, int t) {
    using K = Kind<KIND>;
    constexpr bool PADDED = FILL == kPadded;
    int ta = t;
    if constexpr (FILL == kDirect) {
        static_assert(EDGE != kElem, "the direct fill needs 16-byte aligned rows");
        direct_fill<KIND, EDGE>(io, lds, L, mv, t);
    } else {
        u32x4 v[K::GLOADS];
        load_tile<KIND, EDGE>(io, t, v);
        ta = after_loads(t);
        lds_store<KIND, PADDED>(lds, lane_base<KIND, true, PADDED>(ta, L), L, mv, v, ta);
    }
    const uint32_t rbase = lane_base<KIND, false, PADDED>(ta, L);
    __syncthreads();
    lds_read_store<KIND, PADDED, EDGE>(lds, rbase, L, mv, io, t);
}

// Which tiles a launch covers and how blockIdx names them.
//   kInterior: a 3-D grid (block row, block column step, batch entry) over
//              whole tiles only, in blocks of stack_of() x stack_c_of()
//              tiles per workgroup, in diagonal order; no edge test at all.
//   kEdge:     a 1-D chunk of the edge tiles (the tile columns and rows of
//              each batch entry past the interior's blocks: whole tiles that
//              did not fill a block, and those that stick out).
//   kBlocks:   every tile of aligned rows in one 3-D launch of blocks of
//              stack_of() x stack_c_of() tiles, as kInterior: a tile of the
//              block that is whole takes the unguarded path, one that sticks
//              out the guarded path, and one past the matrix only the barrier.
//              It replaces kInterior + kEdge where the rows leave edge tiles,
//              so that those cost no launch of their own.
//   kBlocksXcd: kBlocks for output row pitches that are not multiples of
//              64 bytes (partial_line_output).  Tiles then share 64-byte
//              pieces of output lines with their neighbours, which memory
//              serves as partial writes unless both halves meet in one L2
//              first.  Workgroups are dispatched to the eight XCDs (each
//              with its own L2) in turn, so this grid renumbers them:
//              workgroups i, i + 8, i + 16, ..., which share an XCD, take
//              consecutive blocks, and the accesses go through the caches.
//   kAll3D / kAll1D: every tile, 3-D as kInterior or a 1-D chunk of the
//              linear tile order (grids beyond the hardware's y / z limits,
//              sizes past the 32-bit whole-tile path, unaligned pitches).
//   kAll3DXcd: kAll3D renumbered and cached as kBlocksXcd, for unaligned
//              pitches whose output rows are partial_line_output.
enum Grid { kAll3D = 0, kAll1D = 1, kInterior = 2, kEdge = 3, kBlocks = 4, kBlocksXcd = 5, kAll3DXcd = 6 };

// Tile (tr, tc) of a 3-D diagonal-order grid with n tile columns: tc = (y +
// f) mod n, f = (x num) >> sh, y < n.  One conditional subtract, and a
// division only when f reaches n (a uniform branch laid out of line).
__device__ __forceinline__ uint32_t diagonal_column_at(uint32_t x, uint32_t y, uint32_t n, TileOrder O) {
    uint32_t f = (x * O.num) >> O.sh;
    if (__builtin_expect(f >= n, 0)) f %= n;
    const uint32_t c = y + f;
    return c >= n ? c - n : c;
}
__device__ __forceinline__ uint32_t diagonal_column(uint32_t n, TileOrder O) {
    return diagonal_column_at(blockIdx.x, blockIdx.y, n, O);
}

// The XCDs of the chip (each with its own L2), which take the workgroups of
// a launch in turn by their linear number.
constexpr uint32_t kXcds = 8;

// kBlocksXcd's renumbering of this workgroup's (x, y, z): linear number
// L = x + gx (y + gy z) on XCD L mod 8 becomes the (L / 8)-th of that XCD's
// run of consecutive numbers (runs of G / 8, the first G mod 8 one longer),
// decoded back to (x, y, z).  One-to-one for any grid.
__device__ __forceinline__ void xcd_renumber(uint32_t& x, uint32_t& y, uint32_t& z) {
    const uint64_t gx = gridDim.x, gy = gridDim.y, g = gx * gy * gridDim.z;
    const uint64_t l = blockIdx.x + gx * (blockIdx.y + gy * static_cast<uint64_t>(blockIdx.z));
    const uint64_t k = l % kXcds, q = g / kXcds, rem = g % kXcds;
    const uint64_t m = k * q + (k < rem ? k : rem) + l / kXcds;
    x = static_cast<uint32_t>(m % gx);
    y = static_cast<uint32_t>((m / gx) % gy);
    z = static_cast<uint32_t>(m / (gx * gy));
}

// Edge tile e (of one batch entry) outside the first full_r x full_c tiles
// of a matrix of tiles_r x tiles_c tiles: first the tile columns from full_c
// on next to the first full_r tile rows, row by row, then the tile rows from
// full_r on, whole.
__host__ __device__ __forceinline__ int64_t edge_tiles(int64_t full_r, int64_t full_c, int64_t tiles_r,
                                                       int64_t tiles_c) {
    return (tiles_c - full_c) * full_r + (tiles_r - full_r) * tiles_c;
}

__device__ __forceinline__ void edge_tile(int64_t e, int64_t full_r, int64_t full_c, int64_t tiles_c, int64_t& tr,
                                          int64_t& tc) {
    const int64_t w = tiles_c - full_c, right = w * full_r;
    if (e < right) {
        tr = e / w;
        tc = full_c + (e - tr * w);
    } else {
        tr = full_r + (e - right) / tiles_c;
        tc = (e - right) % tiles_c;
    }
}

// Arguments in the order the kernel needs them: the first thirteen dwords
// (pointers, tile columns, tile order, the host's FastPath, 32-bit sizes;
// plain scalars, which is what the build's kernel-argument preload puts in
// SGPRs) are all a whole tile of a 3-D launch reads before its first load.
template <int KIND, int GRID>
constexpr int stack_in() {
    return GRID == kInterior || GRID == kBlocks || GRID == kBlocksXcd ? stack_of<KIND>() * stack_c_of<KIND>() : 1;
}

template <int KIND, int FILL, bool ALIGNED, int GRID>
__global__ __launch_bounds__((Kind<KIND>::NT * stack_in<KIND, GRID>())) void k_convert(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            uint32_t tiles_c32, uint32_t order_num, uint32_t order_sh,
                                                            uint32_t sp, uint32_t dp, uint32_t full_r, uint32_t full_c,
                                                            uint32_t rows32, uint32_t cols32, int64_t rows,
                                                            int64_t cols, int64_t tiles_r, int64_t tile0, KLayout L,
                                                            StepMoves mv) {
    using K = Kind<KIND>;
    constexpr int E = K::ESZ;
    static_assert(FILL != kDirect || ALIGNED, "the direct fill needs 16-byte aligned rows");
    static_assert(ALIGNED || GRID == kAll3D || GRID == kAll3DXcd || GRID == kAll1D,
                  "unaligned pitches take the element-wise path");
    constexpr int STACK = stack_in<KIND, GRID>();
    constexpr int TILE_V = (LdsTile<KIND, FILL>::BYTES + 15) / 16;
    __shared__ u32x4 lds_v[STACK * TILE_V];
    // the interior's stacked tiles: each NT threads (whole waves) move one
    static_assert(STACK == 1 || (K::NT % 64 == 0 && (K::NT & (K::NT - 1)) == 0), "whole waves per tile");
    const int g = STACK == 1 ? 0 : static_cast<int>(threadIdx.x) / K::NT;
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v + g * TILE_V);
    const int t = STACK == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) & (K::NT - 1);
    const TileOrder O{order_num, order_sh};
    constexpr bool CACHED = GRID == kBlocksXcd || GRID == kAll3DXcd;

    // A whole tile: batch entry b's rows follow entry b - 1's in both
    // matrices, so the tile is (b rows + r0, c0) of the source and (b cols +
    // c0, r0) of the output, in 32 bits (the host's FastPath says so).
    auto whole = [&](uint32_t b32, uint32_t tr32, uint32_t tc32) {
        const uint32_t r0 = tr32 * K::TR, c0 = tc32 * K::TC;
        const TileIo<kFull, E, CACHED> io{src + (static_cast<uint64_t>(b32 * rows32 + r0) * sp + c0 * E),
                                  dst + (static_cast<uint64_t>(b32 * cols32 + c0) * dp + r0 * E), 0, 0, 0, 0, sp, dp};
        convert_tile<KIND, FILL, kFull>(io, lds, L, mv, t);
    };
    // Any tile, with 64-bit indexing and the guards of EDGE.
    auto guarded = [&](int64_t b, int64_t tr, int64_t tc) {
        const int64_t plane = rows * cols * E;
        constexpr int EDGE = ALIGNED ? kVec : kElem;
        convert_tile<KIND, FILL, EDGE>(
            TileIo<EDGE, E, CACHED>{src + b * plane, dst + b * plane, rows, cols, tr * K::TR, tc * K::TC, 0u, 0u}, lds, L, mv,
            t);
    };

    if constexpr (GRID == kInterior) {
        // tile g of the workgroup's SR x SC block (tiles_c32: blocks per row)
        constexpr int SR = stack_of<KIND>(), SC = stack_c_of<KIND>();
        whole(blockIdx.z, blockIdx.x * SR + g % SR, diagonal_column(tiles_c32, O) * SC + g / SR);
    } else if constexpr (GRID == kBlocks || GRID == kBlocksXcd) {
        // As kInterior over blocks that may reach past the whole tiles
        // (tiles_c32: blocks per row, rounded up).  The tile test is uniform
        // across each wave (readfirstlane of g), so every wave branches as a
        // whole and runs exactly one barrier: its tile's, or its own where
        // the block reaches past the matrix.
        constexpr int SR = stack_of<KIND>(), SC = stack_c_of<KIND>();
        uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
        if constexpr (GRID == kBlocksXcd) xcd_renumber(bx, by, bz);
        const uint32_t gu = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(g));
        const uint32_t tr = bx * SR + gu % SR, tc = diagonal_column_at(bx, by, tiles_c32, O) * SC + gu / SR;
        if (tr < full_r && tc < full_c)
            whole(bz, tr, tc);
        else if (tr < tiles_r && tc < (cols + K::TC - 1) / K::TC)
            guarded(bz, tr, tc);
        else
            __syncthreads();
    } else if constexpr (GRID == kEdge) {
        const int64_t tiles_c = (cols + K::TC - 1) / K::TC;
        const int64_t per = edge_tiles(full_r, full_c, tiles_r, tiles_c);
        const int64_t idx = tile0 + blockIdx.x;
        const int64_t b = idx / per;
        int64_t tr, tc;
        edge_tile(idx - b * per, full_r, full_c, tiles_c, tr, tc);
        guarded(b, tr, tc);
    } else {
        int64_t b, tr, tc;
        if constexpr (GRID == kAll3D || GRID == kAll3DXcd) {
            uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
            if constexpr (GRID == kAll3DXcd) xcd_renumber(bx, by, bz);
            b = bz;
            tr = bx;
            tc = diagonal_column_at(bx, by, tiles_c32, O);
        } else {
            decode_tile<true>(tile0 + blockIdx.x, tiles_r, tiles_c32, O, b, tr, tc);
        }
        if constexpr (ALIGNED) {
            if (tr < full_r && tc < full_c) {
                whole(static_cast<uint32_t>(b), static_cast<uint32_t>(tr), static_cast<uint32_t>(tc));
                return;
            }
        }
        guarded(b, tr, tc);
    }
}

// ---------------------------------------------------------------------------
// Operand staging: 64x64 K-tiles of a K-contiguous 16-bit operand, read
// back as 16x16x32 operand fragments and written out in lane order.
// ---------------------------------------------------------------------------
// One 64 x 64 tile of a K-contiguous operand (rows r0.., k columns k0..).
// A whole tile (FULL) takes src and frag as the tile's own bases (its first
// element, its first fragment) and addresses its rows and its 4 row blocks
// of fragments with the 32-bit pitches sp (the operand row, 2k bytes) and fp
// (one row block of fragments, 32k bytes); an edge tile indexes the whole
// operand with 64-bit products and guards each 16-byte chunk (mn and k are
// multiples of 16 and 32, so a chunk is wholly inside or outside).
template <int FILL, bool FULL>
__device__ __forceinline__ void stage_tile(const uint8_t* __restrict__ src, uint8_t* __restrict__ frag, int64_t mn,
                                           int64_t k, int64_t r0, int64_t k0, uint32_t sp, uint32_t fp, uint8_t* lds,
                                           const KLayout& L, const StepMoves& mv, int t) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    constexpr bool PADDED = FILL == kPadded;
    constexpr int EDGE = FULL ? kFull : kVec;
    using K = Kind<KD>;
    const TileIo<EDGE, 2> io{src, nullptr, mn, k, r0, k0, sp, 0u};
    int ta = t;
    if constexpr (FILL == kDirect) {
        direct_fill<KD, EDGE>(io, lds, L, mv, t);
    } else {
        u32x4 v[K::GLOADS];
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
            int r = 0, c = 0;
            K::wcoord(t, j, r, c);
            if constexpr (FULL)
                v[j] = gload16(io.src(r, c));
            else
                v[j] = r0 + r < mn && k0 + c < k ? gload16(src + ((r0 + r) * k + k0 + c) * 2) : u32x4{0u, 0u, 0u, 0u};
        }
        ta = after_loads(t);
        const uint32_t wbase = lane_base<KD, true, PADDED>(ta, L);
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j)
            *reinterpret_cast<u32x4*>(lds + 2 * step_off<true, PADDED>(wbase, j, mv)) = v[j];
    }
    const uint32_t rbase = lane_base<KD, false, PADDED>(ta, L);
    __syncthreads();
    const int lane = t % 64;
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        const int f = K::frag_of(t, i);
        const int blk = f % K::RB, ks = f / K::RB;
        const u32x4 x = *reinterpret_cast<const u32x4*>(lds + 2 * step_off<false, PADDED>(rbase, i, mv));
        if constexpr (FULL) {
            gstore16(frag + (static_cast<uint64_t>(static_cast<uint32_t>(blk)) * fp +
                             static_cast<uint32_t>(ks * 1024 + lane * 16)),
                     x);
        } else if (r0 + 16 * blk < mn && k0 + 32 * ks < k) {
            const int64_t fi = (r0 / 16 + blk) * (k / 32) + (k0 / 32 + ks);
            gstore16(frag + (fi * 64 + lane) * 16, x);
        }
    }
}

// Arguments as for k_convert: what a whole tile of a 3-D launch reads first.
// Grids as for k_convert (kInterior: x = k tile, y = row tile, row-major,
// which keeps both the reads and the fragment writes contiguous; kEdge; kAll1D).
// kInterior also stages a second operand of the same k (src2 -> frag2, its
// full_m2 whole row tiles) as grid z = 1, so both operands of a GEMM take
// one launch; rows of y at or past an operand's own count do nothing.
// Whole staging tiles per workgroup of the interior launch, side by side
// along k (interior_stack; four: 1024 threads, 32 KiB of LDS).
constexpr int kStageStack = interior_stack(SWZ_READ_MFMA_16X16X32);

template <int GRID>
constexpr int stage_stack_in() {
    return GRID == kInterior || GRID == kBlocks ? kStageStack : 1;
}

template <int FILL, int GRID>
__global__ __launch_bounds__((Kind<SWZ_READ_MFMA_16X16X32>::NT * stage_stack_in<GRID>())) void k_stage(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ frag, uint32_t sp, uint32_t fp, uint32_t full_m,
    uint32_t full_k, const uint8_t* __restrict__ src2, uint8_t* __restrict__ frag2, uint32_t full_m2, int64_t mn,
    int64_t k, int64_t tiles_m, int64_t tiles_k, int64_t tile0, KLayout L, StepMoves mv, int64_t mn2) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    using K = Kind<KD>;
    constexpr int STACK = stage_stack_in<GRID>();
    constexpr int TILE_V = LdsTile<KD, FILL>::BYTES / 16;
    __shared__ u32x4 lds_v[STACK * TILE_V];
    static_assert(K::NT % 64 == 0 && (K::NT & (K::NT - 1)) == 0, "whole waves per tile");
    const int g = STACK == 1 ? 0 : static_cast<int>(threadIdx.x) / K::NT;
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v + g * TILE_V);
    const int t = STACK == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) & (K::NT - 1);

    // the tile's first element (row TR tm, k 64 tk) and first fragment (row
    // block TR/16 tm, k step 2 tk)
    auto whole = [&](const uint8_t* s, uint8_t* f, uint32_t tm, uint32_t tk) {
        const uint32_t r0 = tm * K::TR, kb0 = tk * K::TC;
        stage_tile<FILL, true>(s + (static_cast<uint64_t>(r0) * sp + 2 * kb0),
                               f + (static_cast<uint64_t>(r0 / 16) * fp + 32 * kb0), mn, k, 0, 0, sp, fp, lds, L, mv,
                               t);
    };
    auto guarded = [&](int64_t tm, int64_t tk) {
        stage_tile<FILL, false>(src, frag, mn, k, tm * K::TR, tk * K::TC, 0u, 0u, lds, L, mv, t);
    };
    if constexpr (GRID == kInterior) {
        const bool second = blockIdx.z != 0;
        if (blockIdx.y >= (second ? full_m2 : full_m)) return;
        whole(second ? src2 : src, second ? frag2 : frag, blockIdx.y, blockIdx.x * STACK + g);
    } else if constexpr (GRID == kBlocks) {
        // As kInterior over every tile of both operands: whole tiles
        // unguarded, partial ones guarded, tiles past the operand only the
        // barrier (the test is uniform across each wave, as in k_convert).
        const bool second = blockIdx.z != 0;
        const uint8_t* s = second ? src2 : src;
        uint8_t* f = second ? frag2 : frag;
        const int64_t m = second ? mn2 : mn;
        const uint32_t tm = blockIdx.y, tk = blockIdx.x * STACK + __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(g));
        if (tm < (second ? full_m2 : full_m) && tk < full_k)
            whole(s, f, tm, tk);
        else if (tm < (m + K::TR - 1) / K::TR && tk < tiles_k)
            stage_tile<FILL, false>(s, f, m, k, tm * int64_t(K::TR), tk * int64_t(K::TC), 0u, 0u, lds, L, mv, t);
        else
            __syncthreads();
    } else if constexpr (GRID == kEdge) {
        int64_t tm, tk;
        edge_tile(tile0 + blockIdx.x, full_m, full_k, tiles_k, tm, tk);
        guarded(tm, tk);
    } else {
        const int64_t idx = tile0 + blockIdx.x, tm = idx / tiles_k, tk = idx - tm * tiles_k;
        if (tm < full_m && tk < full_k)
            whole(src, frag, static_cast<uint32_t>(tm), static_cast<uint32_t>(tk));
        else
            guarded(tm, tk);
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The launch's StepMoves: each step's move (the lane-0 coordinate of the
// step, lane 0 starting at (0, 0)) as an LDS element offset of the layout.
template <int KIND>
StepMoves step_moves(const LdsLayout& L, bool padded) {
    using K = Kind<KIND>;
    static_assert(K::WSTEPS <= kMaxSteps && K::RSTEPS <= kMaxSteps && Direct<KIND>::LOADS <= kMaxSteps,
                  "the step moves fit in StepMoves");
    StepMoves mv{};
    auto move = [&](int dr, int dc) {
        return padded ? static_cast<uint32_t>(dr) * L.ld + static_cast<uint32_t>(dc)
                      : swizzle(static_cast<uint32_t>(dr * K::TC + dc), L.B, L.M, L.S);
    };
    for (int i = 0; i < K::WSTEPS; ++i) {
        int dr = 0, dc = 0;
        coord<KIND, true>(0, i, dr, dc);
        mv.w[i] = move(dr, dc);
    }
    for (int i = 0; i < K::RSTEPS; ++i) {
        int dr = 0, dc = 0;
        coord<KIND, false>(0, i, dr, dc);
        mv.r[i] = move(dr, dc);
    }
    for (int j = 0; j < Direct<KIND>::LOADS; ++j)
        mv.d[j] = swizzle(static_cast<uint32_t>(Direct<KIND>::EPL * K::NT * j), L.B, L.M, L.S);
    return mv;
}

// Grid limits of a 3-D launch: work-items along x below 2^31, y and z up to
// 65535 workgroups.
bool fits_3d(int64_t x, int64_t y, int64_t z, int threads) {
    return x * threads < (int64_t(1) << 31) && y <= 65535 && z <= 65535;
}

// A 1-D launch of n tiles in chunks of at most kMaxGrid workgroups.
template <typename F>
void launch_chunks(int64_t n, F launch) {
    for (int64_t t0 = 0; t0 < n; t0 += kMaxGrid) launch(t0, n - t0 < kMaxGrid ? n - t0 : kMaxGrid);
}

// Whether the output rows of a job are not whole 64-byte pieces: their
// pitch (partial_line_output), or, from the same 2,000 rows, the output
// pointer, which puts every output row off the pieces alike.  Measured with
// both pointers 4 or 16 bytes off (share of a copy, the plain grid against
// the XCD-grouped one): fp32 5760^2 0.44 -> 0.64 and 0.43 -> 0.67, 4096^2
// 0.44 -> 0.53 and 0.45 -> 0.52; 16-bit 8192^2 0.32 -> 0.43 and 0.45 ->
// 0.52; bytes 8192^2 0.39 -> 0.46 and 0.38 -> 0.47, but bytes whose output
// pointer is not 4-byte aligned lost (0.40 -> 0.37), so those keep the
// plain grid.
template <int ESZ>
bool partial_lines(const ConvertJob& j) {
    const uintptr_t d = reinterpret_cast<uintptr_t>(j.dst);
    return partial_line_output(j.rows, ESZ) || (j.rows >= 2000 && d % 64 != 0 && (ESZ > 1 || d % 4 == 0));
}

template <int KIND, int FILL, bool ALIGNED>
void launch_variant(const ConvertJob& j, int64_t tiles_r, int64_t tiles_c, int64_t n_tiles, hipStream_t stream) {
    using K = Kind<KIND>;
    const auto* s = static_cast<const uint8_t*>(j.src);
    auto* d = static_cast<uint8_t*>(j.dst);
    // slope of the diagonal order per SWZ_ORDER_* value: 1, 1/2, 0, 3, 1/8, 1/16, 1/32
    static constexpr TileOrder kOrders[7] = {{1u, 0u}, {1u, 1u}, {0u, 0u}, {3u, 0u}, {1u, 3u}, {1u, 4u}, {1u, 5u}};
    const TileOrder O = kOrders[j.order >= 0 && j.order < 7 ? j.order : 0];
    const StepMoves mv = step_moves<KIND>(j.layout, FILL == kPadded);
    const FastPath fp = fast_path(j.batch, j.rows, j.cols, K::ESZ, K::TR, K::TC);
    // 32-bit sizes for the whole-tile path (only read when FastPath allows it)
    const auto r32 = static_cast<uint32_t>(j.rows), c32 = static_cast<uint32_t>(j.cols);
    const KLayout kl = decode_layout(j.layout);
    const unsigned lds_pad = occupancy_pad<KIND>(LdsTile<KIND, FILL>::BYTES);
    const dim3 block(K::NT);
    auto args = [&](uint32_t cols_of_order, int64_t tile0, uint32_t full_r, uint32_t full_c) {
        return std::make_tuple(s, d, cols_of_order, O.num, O.sh, fp.sp, fp.dp, full_r, full_c, r32, c32, j.rows,
                               j.cols, tiles_r, tile0, kl, mv);
    };
    if constexpr (ALIGNED) {
        // the interior covers the whole tiles in blocks of SR x SC; the
        // whole rows and columns past the last block join the edge strips
        constexpr int SR = stack_of<KIND>(), SC = stack_c_of<KIND>();
        const uint32_t inner_r = fp.full_r / SR * SR, inner_c = fp.full_c / SC * SC;
        const unsigned inner_pad =
            occupancy_pad_to(SR * SC * LdsTile<KIND, FILL>::BYTES, interior_occupancy_limit<KIND>());
        const int64_t blocks_r = ceil_div(tiles_r, SR), blocks_c = ceil_div(tiles_c, SC);
        // output rows off the 64-byte pieces: the XCD-grouped block grid,
        // with or without edge tiles
        bool xcd = false;
        if constexpr (FILL != kDirect && !is_narrow(KIND)) xcd = partial_lines<K::ESZ>(j);
        if ((inner_r != tiles_r || inner_c != tiles_c || xcd) && fp.full_r > 0 && fp.full_c > 0 &&
            fits_3d(blocks_r, blocks_c, j.batch, K::NT * SR * SC)) {
            // edge tiles (or partial output lines): all tiles in one launch of blocks
            const dim3 grid(static_cast<unsigned>(blocks_r), static_cast<unsigned>(blocks_c),
                            static_cast<unsigned>(j.batch));
            const auto a = args(static_cast<uint32_t>(blocks_c), 0, fp.full_r, fp.full_c);
            if constexpr (FILL != kDirect && !is_narrow(KIND)) {
                if (xcd) {
                    std::apply([&](auto... v) {
                        hipLaunchKernelGGL((k_convert<KIND, FILL, true, kBlocksXcd>), grid, dim3(K::NT * SR * SC),
                                           inner_pad, stream, v...);
                    }, a);
                    return;
                }
            }
            std::apply([&](auto... v) {
                hipLaunchKernelGGL((k_convert<KIND, FILL, true, kBlocks>), grid, dim3(K::NT * SR * SC), inner_pad,
                                   stream, v...);
            }, a);
            return;
        }
        if (inner_r > 0 && inner_c > 0 && fits_3d(inner_r / SR, inner_c / SC, j.batch, K::NT * SR * SC)) {
            std::apply([&](auto... a) {
                hipLaunchKernelGGL((k_convert<KIND, FILL, true, kInterior>),
                                   dim3(inner_r / SR, inner_c / SC, static_cast<unsigned>(j.batch)),
                                   dim3(K::NT * SR * SC), inner_pad, stream, a...);
            }, args(inner_c / SC, 0, inner_r, inner_c));
            const int64_t per = edge_tiles(inner_r, inner_c, tiles_r, tiles_c);
            launch_chunks(j.batch * per, [&](int64_t t0, int64_t n) {
                std::apply([&](auto... a) {
                    hipLaunchKernelGGL((k_convert<KIND, FILL, true, kEdge>), dim3(static_cast<unsigned>(n)), block,
                                       lds_pad, stream, a...);
                }, args(static_cast<uint32_t>(tiles_c), t0, inner_r, inner_c));
            });
            return;
        }
    } else {
        if (fits_3d(tiles_r, tiles_c, j.batch, K::NT)) {
            const dim3 grid(static_cast<unsigned>(tiles_r), static_cast<unsigned>(tiles_c),
                            static_cast<unsigned>(j.batch));
            const auto a = args(static_cast<uint32_t>(tiles_c), 0, fp.full_r, fp.full_c);
            if constexpr (!is_narrow(KIND)) {
                if (partial_lines<K::ESZ>(j)) {
                    std::apply([&](auto... v) {
                        hipLaunchKernelGGL((k_convert<KIND, FILL, false, kAll3DXcd>), grid, block, lds_pad, stream,
                                           v...);
                    }, a);
                    return;
                }
            }
            std::apply([&](auto... v) {
                hipLaunchKernelGGL((k_convert<KIND, FILL, false, kAll3D>), grid, block, lds_pad, stream, v...);
            }, a);
            return;
        }
    }
    launch_chunks(n_tiles, [&](int64_t t0, int64_t n) {
        std::apply([&](auto... a) {
            hipLaunchKernelGGL((k_convert<KIND, FILL, ALIGNED, kAll1D>), dim3(static_cast<unsigned>(n)), block, lds_pad,
                               stream, a...);
        }, args(static_cast<uint32_t>(tiles_c), t0, fp.full_r, fp.full_c));
    });
}

template <int KIND>
hipError_t launch_kind(const ConvertJob& j, hipStream_t stream) {
    using K = Kind<KIND>;
    const int64_t tiles_r = ceil_div(j.rows, K::TR), tiles_c = ceil_div(j.cols, K::TC);
    const int64_t n_tiles = j.batch * tiles_r * tiles_c;
    if (n_tiles == 0) return hipSuccess;
    if (tiles_c > int64_t(UINT32_MAX)) return hipErrorInvalidValue;  // the kernel takes it as 32 bits
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
void launch_stage_fill(const StageJob& j, hipStream_t stream) {
    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    using K = Kind<KD>;
    const StepMoves mv = step_moves<KD>(j.layout, FILL == kPadded);
    const KLayout kl = decode_layout(j.layout);
    const unsigned lds_pad = occupancy_pad<KD>(LdsTile<KD, FILL>::BYTES);
    const dim3 block(K::NT);
    const bool pair = j.src2 != nullptr;
    struct Op {
        const uint8_t* s;
        uint8_t* f;
        int64_t mn;
    };
    const Op ops[2] = {{static_cast<const uint8_t*>(j.src), static_cast<uint8_t*>(j.frag), j.mn},
                       {static_cast<const uint8_t*>(j.src2), static_cast<uint8_t*>(j.frag2), pair ? j.mn2 : 0}};
    const int nops = pair ? 2 : 1;
    const int64_t tiles_k = ceil_div(j.k, K::TC);
    // Whole tiles address rows of 2k bytes and row blocks of fragments of
    // 32k bytes with 32-bit pitches: both must fit, else every tile takes
    // the 64-bit edge path.
    const bool fit = j.mn < (int64_t(1) << 31) && ops[1].mn < (int64_t(1) << 31) && j.k * 32 < (int64_t(1) << 32);
    const uint32_t sp = fit ? static_cast<uint32_t>(2 * j.k) : 0u, fpitch = fit ? static_cast<uint32_t>(32 * j.k) : 0u;
    const uint32_t full_k = fit ? static_cast<uint32_t>(j.k / K::TC) : 0u;
    uint32_t full_m[2] = {0u, 0u};
    for (int o = 0; o < nops; ++o) full_m[o] = fit ? static_cast<uint32_t>(ops[o].mn / K::TR) : 0u;
    const uint32_t rows_y = full_m[0] > full_m[1] ? full_m[0] : full_m[1];
    // the interior covers the whole k tiles in groups of kStageStack; the
    // k tiles past the last group join the edge strips
    const uint32_t inner_k = full_k / kStageStack * kStageStack;
    int64_t tiles_y = 0;  // tile rows of the taller operand
    bool edges = inner_k != tiles_k;
    for (int o = 0; o < nops; ++o) {
        const int64_t tm = ceil_div(ops[o].mn, K::TR);
        tiles_y = tm > tiles_y ? tm : tiles_y;
        edges = edges || full_m[o] != tm;
    }
    if (edges && fit && fits_3d(ceil_div(tiles_k, kStageStack), tiles_y, nops, K::NT * kStageStack)) {
        // edge tiles: every tile of every operand in one launch of blocks
        hipLaunchKernelGGL((k_stage<FILL, kBlocks>),
                           dim3(static_cast<unsigned>(ceil_div(tiles_k, kStageStack)), static_cast<unsigned>(tiles_y),
                                nops),
                           dim3(K::NT * kStageStack), 0, stream, ops[0].s, ops[0].f, sp, fpitch, full_m[0], full_k,
                           ops[1].s, ops[1].f, full_m[1], j.mn, j.k, ceil_div(j.mn, K::TR), tiles_k, int64_t(0), kl,
                           mv, ops[1].mn);
        return;
    }
    if (inner_k > 0 && rows_y > 0 && fits_3d(inner_k / kStageStack, rows_y, nops, K::NT * kStageStack)) {
        // the whole tiles of every operand in one launch, then each
        // operand's edge strips
        hipLaunchKernelGGL((k_stage<FILL, kInterior>), dim3(inner_k / kStageStack, rows_y, nops),
                           dim3(K::NT * kStageStack), 0, stream, ops[0].s, ops[0].f, sp, fpitch, full_m[0], inner_k,
                           ops[1].s, ops[1].f, full_m[1], j.mn, j.k, ceil_div(j.mn, K::TR), tiles_k, int64_t(0), kl,
                           mv, ops[1].mn);
        for (int o = 0; o < nops; ++o) {
            const int64_t tiles_m = ceil_div(ops[o].mn, K::TR);
            launch_chunks(edge_tiles(full_m[o], inner_k, tiles_m, tiles_k), [&](int64_t t0, int64_t n) {
                hipLaunchKernelGGL((k_stage<FILL, kEdge>), dim3(static_cast<unsigned>(n)), block, lds_pad, stream,
                                   ops[o].s, ops[o].f, sp, fpitch, full_m[o], inner_k, ops[o].s, ops[o].f, full_m[o],
                                   ops[o].mn, j.k, tiles_m, tiles_k, t0, kl, mv, ops[o].mn);
            });
        }
        return;
    }
    for (int o = 0; o < nops; ++o) {
        const int64_t tiles_m = ceil_div(ops[o].mn, K::TR);
        launch_chunks(tiles_m * tiles_k, [&](int64_t t0, int64_t n) {
            hipLaunchKernelGGL((k_stage<FILL, kAll1D>), dim3(static_cast<unsigned>(n)), block, lds_pad, stream,
                               ops[o].s, ops[o].f, sp, fpitch, full_m[o], full_k, ops[o].s, ops[o].f, full_m[o],
                               ops[o].mn, j.k, tiles_m, tiles_k, t0, kl, mv, ops[o].mn);
        });
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
    const int64_t rows = j.mn + (j.src2 ? j.mn2 : 0);
    if (rows == 0 || ceil_div(j.k, K::TC) == 0) return hipSuccess;
    const bool padded = j.layout.ld != static_cast<uint32_t>(K::TC);
    if (padded && j.layout.ld != static_cast<uint32_t>(K::TC + LdsTile<KD, kPadded>::PAD)) return hipErrorInvalidValue;
    if (j.direct) {
        if (padded) return hipErrorInvalidValue;
        launch_stage_fill<kDirect>(j, stream);
    } else if (padded) {
        launch_stage_fill<kPadded>(j, stream);
    } else {
        launch_stage_fill<kRegs>(j, stream);
    }
    return hipGetLastError();
}

}  // namespace swz
