// Shared by the HIP kernels and the host-side chooser: the swizzle function,
// the LDS address of a tile element, and, for each read kind, which tile
// element every lane touches at every step.  Keeping the lane maps in one
// place means the chooser predicts conflicts for exactly the accesses the
// kernels issue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "swz.h"

namespace swz {

// Swizzle<B,M,S> of a 32-bit element offset: the B-bit field at bit M+S is
// XORed into the B-bit field at bit M ("CuTe Swizzle 学习手册", swizzle
// formula); for S < 0 the field at bit M is XORed into the one at bit
// M + |S| ("NVIDIA CuTe Swizzle", a negative shift moves the mask left).
// B == 0 is the identity.  Written without branches (selects only) and
// without shifts by 32 or more, which C++ leaves undefined.
__host__ __device__ __forceinline__ uint32_t swizzle(uint32_t x, uint32_t B, uint32_t M, int32_t S) {
    const uint32_t mask = B >= 32u ? 0xffffffffu : ((1u << B) - 1u);
    const uint32_t up = S >= 0 ? static_cast<uint32_t>(S) : 0u;    // source above the target
    const uint32_t dn = S >= 0 ? 0u : static_cast<uint32_t>(-S);   // source below the target
    const uint32_t src = (M + up) >= 32u ? 0u : ((x >> (M + up)) & mask);
    return x ^ ((M + dn) >= 32u ? 0u : (src << (M + dn)));
}

// How a tile sits in LDS: element (r, c) lives at element offset
// swizzle(r * ld + c).  ld = tile_cols (+ pad for the padded layout); the
// swizzle is the identity (B = 0) for PAD and PLAIN.
struct LdsLayout {
    uint32_t ld;  // LDS row pitch in elements
    uint32_t B, M;
    int32_t S;
};

__host__ __device__ __forceinline__ uint32_t lds_elem(const LdsLayout& L, uint32_t r, uint32_t c) {
    return swizzle(r * L.ld + c, L.B, L.M, L.S);
}

// ---------------------------------------------------------------------------
// Tile shapes, thread counts and lane maps of each read kind.
//
// Every kernel stages a tile with 16-byte global loads (VEC bytes of LDS per
// store, SUB stores per global load) and reads it back with RWIDTH-byte LDS
// loads, RPER of them per output piece.  wcoord(t, i, r, c): the tile element
// thread t's i-th LDS store starts at; rcoord(t, i, r, c): the same for its
// i-th LDS load.  Step counts are per thread per tile.
// ---------------------------------------------------------------------------
template <int KIND> struct Kind;

// 4-byte elements, 32x32 tile (128-byte rows).  Staging: thread vector
// v = t + NT*j (j < 256/NT) holds row v/8, columns 4(v%8)..+3 and stores them
// as four 4-byte LDS writes (step i = 4j + e writes column 4(v%8)+e).  Read:
// task u = t + NT*j owns source column u/8 and rows 4(u%8)..+3, read as four
// 4-byte column reads (step i = 4j + e reads row 4(u%8)+e), and writes them
// as one 16-byte piece of output row u/8.
template <> struct Kind<SWZ_READ_SCALAR_COL> {
    static constexpr int ESZ = 4, TR = 32, TC = 32, NT = 256;
    static constexpr int VEC = 4;                     // LDS store width (bytes)
    static constexpr int RWIDTH = 4;                  // LDS load width (bytes)
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;  // 16-byte global loads per thread
    static constexpr int WSTEPS = GLOADS * 4;
    static constexpr int TASKS = TR * TC / 4 / NT;    // 16-byte output pieces per thread
    static constexpr int RSTEPS = TASKS * 4;
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * (i / 4);
        r = v / 8;
        c = 4 * (v % 8) + i % 4;
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int u = t + NT * (i / 4);
        r = 4 * (u % 8) + i % 4;
        c = u / 8;
    }
};

// 2-byte elements, 64x64 tile (128-byte rows).  Staging: vector v = t + NT*j
// is row v/8, 16-byte chunk v%8 (one 16-byte LDS write).  Read: task
// u = t + NT*j owns row block k = u%8 (rows 8k..8k+7) and column group
// g = u/8 (columns 4g..4g+3); step 8j + s reads the 8 bytes of row 8k+s.
template <> struct Kind<SWZ_READ_B64_4X4> {
    static constexpr int ESZ = 2, TR = 64, TC = 64, NT = 128;
    static constexpr int VEC = 16;
    static constexpr int RWIDTH = 8;
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = GLOADS;
    static constexpr int TASKS = 128 / NT;
    static constexpr int RSTEPS = TASKS * 8;
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * i;
        r = v / 8;
        c = 8 * (v % 8);
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int u = t + NT * (i / 8);
        r = 8 * (u % 8) + i % 8;
        c = 4 * (u / 8);
    }
};

// 2-byte elements, 64x128 tile (256-byte rows).  Staging: vector v = t + NT*j
// is row v/16, chunk v%16.  Read: task u owns row block rb = u%8 and 16-byte
// chunk ch = u/8; step 8j + s reads chunk ch of row 8rb+s.
template <> struct Kind<SWZ_READ_B128_8X8> {
    static constexpr int ESZ = 2, TR = 64, TC = 128, NT = 128;
    static constexpr int VEC = 16;
    static constexpr int RWIDTH = 16;
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = GLOADS;
    static constexpr int TASKS = 128 / NT;
    static constexpr int RSTEPS = TASKS * 8;
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * i;
        r = v / 16;
        c = 8 * (v % 16);
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int u = t + NT * (i / 8);
        r = 8 * (u % 8) + i % 8;
        c = 8 * (u / 8);
    }
};

// Operand staging: 2-byte elements, 64x64 tile (64 rows of the MN
// dimension, 64 of K; 128-byte rows), 256 threads: two 16-byte loads per
// thread.  (256 x 64 tiles with four loads per thread, and 128- or 32-row
// tiles, staged both 8192 x 4096 operands 2-8% slower, stacked four along k
// as these are.)  Staging: vector v = t + NT*j is row v/8, chunk v%8.  Read:
// the 8 fragments of the tile (RB = 4 row blocks x 2 k steps); wave w reads
// fragments f = w + (NT/64)*i; lane l of fragment f reads row
// 16*(f%RB) + l%16, k = 32*(f/RB) + 8*(l/16) .. +7.
template <> struct Kind<SWZ_READ_MFMA_16X16X32> {
    static constexpr int ESZ = 2, TR = 64, TC = 64, NT = 256;
    static constexpr int VEC = 16;
    static constexpr int RWIDTH = 16;
    static constexpr int RB = TR / 16;  // row blocks of 16 rows
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = GLOADS;
    static constexpr int RSTEPS = RB * (TC / 32) / (NT / 64);  // fragments per wave
    __host__ __device__ static constexpr int frag_of(int t, int i) { return (t / 64) + (NT / 64) * i; }
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * i;
        r = v / 8;
        c = 8 * (v % 8);
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int f = frag_of(t, i), l = t % 64;
        r = 16 * (f % RB) + l % 16;
        c = 32 * (f / RB) + 8 * (l / 16);
    }
};

// 2-byte elements, 64x64 tile read back with the gfx950 transpose read
// (ds_read_b64_tr_b16).  Its lane semantics, measured on the hardware: in
// each group of 16 lanes, lane q receives element q%4 of the 8-byte pieces
// that lanes q/4, q/4 + 4, q/4 + 8 and q/4 + 12 of its group addressed.  So
// if loader lane s = a + 4j (a = s%4) addresses row R_a + j of the 4-column
// block at column C_a, receiver q = 4a + e gets rows R_a .. R_a + 3 of
// column C_a + e in order: a 4x4 transpose inside the read.
// Staging as for the 4x4 read.  Read: wave w's task k covers 16-byte chunk
// ch = w + (NT/64)*k (8 columns) of all 64 rows; group g of the wave takes
// rows 16g .. 16g + 15.  Loader q of group g reads row
// 16g + 8*((q%4)/2) + 4*h + q/4, columns 8ch + 4*(q%2), in two steps
// h = s ^ (g%2), s = 0, 1: odd groups read their upper four rows first.
// Receiver q then holds rows 16g + 8*(q/8) + 0..7 of column
// 8ch + 4*((q/4)%2) + q%4 after both steps -- one 16-byte output piece --
// and a wave's store covers 8 output rows of 64 source rows each (whole
// 128-byte rows).  The swapped order puts the two groups of one LDS phase
// on different row bit 2, which the swizzle can turn into different banks.
template <> struct Kind<SWZ_READ_B64_TR16> {
    static constexpr int ESZ = 2, TR = 64, TC = 64, NT = 256;
    static constexpr int VEC = 16;
    static constexpr int RWIDTH = 8;
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = GLOADS;
    static constexpr int TASKS = (TC / 8) / (NT / 64);  // 16-byte chunks per wave
    static constexpr int RSTEPS = 2 * TASKS;
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * i;
        r = v / 8;
        c = 8 * (v % 8);
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int w = t / 64, l = t % 64, g = l / 16, q = l % 16;
        const int k = i / 2, h = (i % 2) ^ (g % 2);
        r = 16 * g + 8 * ((q % 4) / 2) + 4 * h + q / 4;
        c = 8 * (w + (NT / 64) * k) + 4 * (q % 2);
    }
};

// 1-byte elements, 128x128 tile (128-byte rows) read back with the gfx950
// 8-bit transpose read (ds_read_b64_tr_b8).  Its lane semantics, measured
// on the hardware: in each group of 16 lanes, lane q receives byte q%8 of
// the 8-byte pieces that lanes q/8, q/8 + 2, ..., q/8 + 14 of its group
// addressed.  So if loader lane s = a + 2j (a = s%2) addresses row R_a + j
// of the 8-byte column block C_a, receiver q = 8a + e gets rows
// R_a .. R_a + 7 of column C_a + e: an 8x8 byte transpose inside the read.
// Staging: 16-byte global loads stored as two 8-byte LDS writes (the
// swizzle keeps 8-byte runs whole, M >= 3): vector v = t + NT*j is row v/8,
// bytes 16(v%8) .. +15, and write step 2j + h writes its half h ^ (row % 2)
// -- odd rows write their upper halves first, so the two 128-byte rows one
// 16-lane write phase covers use complementary 8-byte chunks.  Read: wave
// w's task k covers the 8-byte column block ch = w + (NT/64)*k of all 128
// rows in two steps h; loader q of group g reads row
// 64h + 16g + 8(q%2) + q/2 of that block, so receiver q holds rows
// 64h + 16g + 8(q/8) .. +7 of column 8ch + q%8: one 8-byte output piece per
// step.  Within one LDS phase (two groups) the rows read differ in their
// five low bits, which a 4-bit swizzle field over 8-byte chunks (source: row
// bits 1-4) spreads over all 64 banks.
template <> struct Kind<SWZ_READ_B64_TR8> {
    static constexpr int ESZ = 1, TR = 128, TC = 128, NT = 256;
    static constexpr int VEC = 8;
    static constexpr int RWIDTH = 8;
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = 2 * GLOADS;
    static constexpr int TASKS = (TC / 8) / (NT / 64);  // 8-byte column blocks per wave
    static constexpr int RSTEPS = 2 * TASKS;
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int v = t + NT * (i / 2);
        r = v / 8;
        c = 16 * (v % 8) + 8 * ((i % 2) ^ (r % 2));
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        const int w = t / 64, l = t % 64, g = l / 16, q = l % 16;
        const int k = i / 2, h = i % 2;
        r = 64 * h + 16 * g + 8 * (q % 2) + q / 2;
        c = 8 * (w + (NT / 64) * k);
    }
};

// Narrow rows of C columns, whole rows per tile: one contiguous stretch of
// the source.  A row is narrower than a bank row, so the tile is treated as
// the flat offsets r*C + c and the swizzle's source field comes from the row
// bits above the ones that make up one line of banks: it spans several rows
// ("CUDA 013 - Swizzle 的工作原理", usage example 4, int num[32][8] taken
// four rows at a time).  PER = 16 / E elements fill 16 bytes, EPW = 4 / E
// fill one 4-byte LDS word.  Each lane owns a block of PER rows and CB
// columns and turns it into CB 16-byte pieces of output rows.  With WORDS
// the block is CB = min(C, EPW) columns read back as whole 4-byte words (a
// word holds EPW columns of one row, or RPW = EPW / C whole rows when
// C < EPW); otherwise it is one column read an element at a time (CB = 1,
// RPW = 1, E-byte loads).  Words take a quarter of the loads for 1-byte
// elements and are faster there; for 2-byte elements element loads measured
// faster at 2 to 16 columns (8 loads per piece), words at 1 and 32.  NT
// lanes (256 by default), so a tile is 16 * NT * CB bytes:
// TR = 16 * NT * CB / (E * C) rows.  Staging: vector
// v = t + NT*j (j < CB) is flat elements PER*v .. PER*v + PER - 1, stored
// as four 4-byte LDS writes; step i = 4j + w writes word w, or, for E < 4
// and C >= 16, word w ^ ((t >> 3) & 3) (SWAP).  The four quarters of a
// 32-lane write phase (vectors 8 apart, whose words share banks) then write
// different banks whatever the swizzle's source bits above the phase; wide
// rows need that, because their reads put the lanes' row blocks 4C >= 64
// words apart, so the swizzle's source field must start above the bits a
// write phase spans.  Read:
// lane t owns columns CB*g .. CB*g + CB - 1 with g = t / (TR/PER) and rows
// PER*b .. PER*b + PER - 1 with b = t % (TR/PER); step i reads the word (or
// element) at row PER*b + RPW*i, column CB*g.  Each output row is a run of
// TR elements.
// E = 4: 1 to 16 columns (4096-byte tiles, one word per row and lane, the
// scalar-column reads); E = 2: 1 to 32; E = 1: 1 to 64.
template <int C, int E>
struct NarrowKind {
    static_assert(E == 4 || E == 2 || E == 1, "4-, 2- or 1-byte elements");
    static_assert(C >= 1 && (C & (C - 1)) == 0 && C * E <= 64, "narrow rows: a power of two up to 64 bytes");
    static constexpr int PER = 16 / E;                   // elements per 16 bytes
    static constexpr int EPW = 4 / E;                    // elements per 4-byte word
    static constexpr bool WORDS = E != 2 || C == 1 || C >= 32;
    static constexpr int CB = !WORDS ? 1 : C < EPW ? C : EPW;   // columns per lane block
    static constexpr int RPW = WORDS && C < EPW ? EPW / C : 1;  // rows per load
    // Lanes per tile.  Byte rows: a sweep of 64, 128 and 256 lanes on 64 MiB
    // matrices put the best at 64 up to 4 columns (+2-4%), 128 at 8 (+8%)
    // and 256 from 16 columns on.
    static constexpr int NT = E != 1   ? 256
                              : C <= 4 ? 64
                              : C == 8 ? 128
                                       : 256;
    static constexpr int ESZ = E, TR = NT * 16 * CB / E / C, TC = C;
    static constexpr int VEC = 4;
    static constexpr int RWIDTH = WORDS ? 4 : E;
    static constexpr int GLOADS = TR * TC * ESZ / 16 / NT;
    static constexpr int WSTEPS = GLOADS * 4;
    static constexpr int TASKS = 1;
    static constexpr int RSTEPS = PER / RPW;
    static constexpr bool SWAP = WORDS && E < 4 && C >= 16;
    __host__ __device__ static constexpr int wword(int t, int i) { return SWAP ? (i % 4) ^ ((t >> 3) & 3) : i % 4; }
    __host__ __device__ static constexpr void wcoord(int t, int i, int& r, int& c) {
        const int e = PER * (t + NT * (i / 4)) + wword(t, i) * EPW;
        r = e / C;
        c = e % C;
    }
    __host__ __device__ static constexpr void rcoord(int t, int i, int& r, int& c) {
        r = PER * (t % (TR / PER)) + RPW * i;
        c = CB * (t / (TR / PER));
    }
};
template <> struct Kind<SWZ_READ_NARROW1> : NarrowKind<1, 4> {};
template <> struct Kind<SWZ_READ_NARROW2> : NarrowKind<2, 4> {};
template <> struct Kind<SWZ_READ_NARROW4> : NarrowKind<4, 4> {};
template <> struct Kind<SWZ_READ_NARROW8> : NarrowKind<8, 4> {};
template <> struct Kind<SWZ_READ_NARROW16> : NarrowKind<16, 4> {};
template <> struct Kind<SWZ_READ_HNARROW1> : NarrowKind<1, 2> {};
template <> struct Kind<SWZ_READ_HNARROW2> : NarrowKind<2, 2> {};
template <> struct Kind<SWZ_READ_HNARROW4> : NarrowKind<4, 2> {};
template <> struct Kind<SWZ_READ_HNARROW8> : NarrowKind<8, 2> {};
template <> struct Kind<SWZ_READ_HNARROW16> : NarrowKind<16, 2> {};
template <> struct Kind<SWZ_READ_HNARROW32> : NarrowKind<32, 2> {};
template <> struct Kind<SWZ_READ_BNARROW1> : NarrowKind<1, 1> {};
template <> struct Kind<SWZ_READ_BNARROW2> : NarrowKind<2, 1> {};
template <> struct Kind<SWZ_READ_BNARROW4> : NarrowKind<4, 1> {};
template <> struct Kind<SWZ_READ_BNARROW8> : NarrowKind<8, 1> {};
template <> struct Kind<SWZ_READ_BNARROW16> : NarrowKind<16, 1> {};
template <> struct Kind<SWZ_READ_BNARROW32> : NarrowKind<32, 1> {};
template <> struct Kind<SWZ_READ_BNARROW64> : NarrowKind<64, 1> {};

__host__ __device__ constexpr bool is_narrow(int kind) {
    return kind >= SWZ_READ_NARROW1 && kind <= SWZ_READ_BNARROW64;
}

// A narrow-row kind whose read-back goes an element at a time (not WORDS).
template <int KIND>
__host__ __device__ constexpr bool narrow_by_element() {
    if constexpr (is_narrow(KIND))
        return !Kind<KIND>::WORDS;
    else
        return false;
}

// Host dispatch on a run-time read kind: calls f(std::integral_constant<int,
// KIND>{}) and returns true, or returns false for an unknown kind.
template <typename F>
bool with_kind(int kind, F&& f) {
    switch (kind) {
#define SWZ_WITH_KIND_CASE(KD)                  \
    case KD:                                    \
        f(std::integral_constant<int, KD>{});   \
        return true;
        SWZ_WITH_KIND_CASE(SWZ_READ_SCALAR_COL)
        SWZ_WITH_KIND_CASE(SWZ_READ_B64_4X4)
        SWZ_WITH_KIND_CASE(SWZ_READ_B128_8X8)
        SWZ_WITH_KIND_CASE(SWZ_READ_MFMA_16X16X32)
        SWZ_WITH_KIND_CASE(SWZ_READ_B64_TR16)
        SWZ_WITH_KIND_CASE(SWZ_READ_B64_TR8)
        SWZ_WITH_KIND_CASE(SWZ_READ_NARROW1)
        SWZ_WITH_KIND_CASE(SWZ_READ_NARROW2)
        SWZ_WITH_KIND_CASE(SWZ_READ_NARROW4)
        SWZ_WITH_KIND_CASE(SWZ_READ_NARROW8)
        SWZ_WITH_KIND_CASE(SWZ_READ_NARROW16)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW1)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW2)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW4)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW8)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW16)
        SWZ_WITH_KIND_CASE(SWZ_READ_HNARROW32)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW1)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW2)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW4)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW8)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW16)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW32)
        SWZ_WITH_KIND_CASE(SWZ_READ_BNARROW64)
#undef SWZ_WITH_KIND_CASE
        default:
            return false;
    }
}
constexpr int kNumKinds = SWZ_READ_BNARROW64 + 1;

// ---------------------------------------------------------------------------
// Offsets of a lane's later steps from its first one.
//
// In every lane map above, step i's row and column are the first step's
// XORed with amounts that do not depend on the lane, so (rows of TC
// elements, TC a power of two) the flat offset is the first one XOR a
// wave-wide value d.  The swizzle is linear over GF(2)
// (x -> x ^ ((x >> (M+S)) & mask) << M), so swizzle(base ^ d) =
// swizzle(base) ^ swizzle(d): each access is the lane's one swizzled base XOR
// a value shared by the whole wave.  Except in the 16-bit transpose read and
// the 8-bit kind's staging writes, the moved bits never overlap the first
// step's, so the same amounts also add, which is what padded rows use (those
// two compute each step's row and column instead).  The checks below prove these properties
// for every lane and step at compile time.
// ---------------------------------------------------------------------------
template <int KIND, bool WRITE>
__host__ __device__ constexpr void coord(int t, int i, int& r, int& c) {
    if (WRITE)
        Kind<KIND>::wcoord(t, i, r, c);
    else
        Kind<KIND>::rcoord(t, i, r, c);
}

// ADDITIVE: also r = r0 + dr and c = c0 + dc (what the padded layout's
// offsets need); the transpose read's steps only combine by XOR, and its
// padded variant computes each step's row and column instead.
template <int KIND, bool WRITE>
constexpr bool steps_decompose(bool additive = true) {
    using K = Kind<KIND>;
    const int steps = WRITE ? K::WSTEPS : K::RSTEPS;
    for (int t = 0; t < K::NT; ++t) {
        int r0 = 0, c0 = 0, z0 = 0, z1 = 0;
        coord<KIND, WRITE>(t, 0, r0, c0);
        coord<KIND, WRITE>(0, 0, z0, z1);
        if (t == 0 && (z0 != 0 || z1 != 0)) return false;  // lane 0 starts at (0, 0)
        for (int i = 0; i < steps; ++i) {
            int r = 0, c = 0, dr = 0, dc = 0;
            coord<KIND, WRITE>(t, i, r, c);
            coord<KIND, WRITE>(0, i, dr, dc);
            if (r != (r0 ^ dr) || c != (c0 ^ dc)) return false;
            if (additive && (r - r0 != dr || c - c0 != dc)) return false;
            if (r >= K::TR || c >= K::TC || r < 0 || c < 0) return false;
        }
    }
    return true;
}

// Thread counts must split each tile's loads and read-back tasks evenly.
template <int KIND>
constexpr bool even_split() {
    using K = Kind<KIND>;
    return K::NT % 64 == 0 && K::GLOADS >= 1 && K::GLOADS * K::NT * 16 == K::TR * K::TC * K::ESZ &&
           K::RSTEPS >= 1;
}
static_assert(even_split<SWZ_READ_SCALAR_COL>() && Kind<SWZ_READ_SCALAR_COL>::TASKS * Kind<SWZ_READ_SCALAR_COL>::NT * 4 == 32 * 32,
              "scalar-column thread count");
static_assert(even_split<SWZ_READ_B64_4X4>() && Kind<SWZ_READ_B64_4X4>::TASKS * Kind<SWZ_READ_B64_4X4>::NT == 128,
              "4x4 thread count");
static_assert(even_split<SWZ_READ_B128_8X8>() && Kind<SWZ_READ_B128_8X8>::TASKS * Kind<SWZ_READ_B128_8X8>::NT == 128,
              "8x8 thread count");
static_assert(even_split<SWZ_READ_MFMA_16X16X32>() &&
                  Kind<SWZ_READ_MFMA_16X16X32>::RSTEPS * (Kind<SWZ_READ_MFMA_16X16X32>::NT / 64) ==
                      Kind<SWZ_READ_MFMA_16X16X32>::RB * 2,
              "fragment thread count");

static_assert(steps_decompose<SWZ_READ_SCALAR_COL, true>() && steps_decompose<SWZ_READ_SCALAR_COL, false>(),
              "scalar-column lane map");
static_assert(steps_decompose<SWZ_READ_B64_4X4, true>() && steps_decompose<SWZ_READ_B64_4X4, false>(),
              "4x4 lane map");
static_assert(steps_decompose<SWZ_READ_B128_8X8, true>() && steps_decompose<SWZ_READ_B128_8X8, false>(),
              "8x8 lane map");
static_assert(steps_decompose<SWZ_READ_MFMA_16X16X32, true>() && steps_decompose<SWZ_READ_MFMA_16X16X32, false>(),
              "fragment lane map");
static_assert(even_split<SWZ_READ_B64_TR16>() && Kind<SWZ_READ_B64_TR16>::TASKS * (Kind<SWZ_READ_B64_TR16>::NT / 64) == 8,
              "transpose-read thread count");
static_assert(steps_decompose<SWZ_READ_B64_TR16, true>() && steps_decompose<SWZ_READ_B64_TR16, false>(false),
              "transpose-read lane map");
static_assert(Kind<SWZ_READ_B64_TR8>::GLOADS * Kind<SWZ_READ_B64_TR8>::NT * 16 == 128 * 128 &&
                  Kind<SWZ_READ_B64_TR8>::TASKS * (Kind<SWZ_READ_B64_TR8>::NT / 64) == 16 &&
                  Kind<SWZ_READ_B64_TR8>::NT % 64 == 0,
              "8-bit transpose-read thread count");
static_assert(steps_decompose<SWZ_READ_B64_TR8, true>(false) && steps_decompose<SWZ_READ_B64_TR8, false>(),
              "8-bit transpose-read lane map");
template <int KIND>
constexpr bool narrow_ok() {
    using K = Kind<KIND>;
    // with SWAP the writes exchange word pairs by lane, so their steps only
    // combine by XOR (padded rows compute each step's row and column)
    return even_split<KIND>() && K::NT * K::PER * K::CB == K::TR * K::TC && K::TR % K::PER == 0 &&
           K::GLOADS == K::CB && steps_decompose<KIND, true>(!K::SWAP) && steps_decompose<KIND, false>();
}
// one assertion per kind: each evaluation has its own constexpr step budget
static_assert(narrow_ok<SWZ_READ_NARROW1>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_NARROW2>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_NARROW4>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_NARROW8>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_NARROW16>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW1>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW2>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW4>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW8>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW16>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_HNARROW32>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW1>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW2>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW4>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW8>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW16>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW32>(), "narrow-row lane map and thread count");
static_assert(narrow_ok<SWZ_READ_BNARROW64>(), "narrow-row lane map and thread count");

// ---------------------------------------------------------------------------
// Direct fill (SWZ_LAYOUT_SWIZZLE_DIRECT): the tile goes from HBM straight
// into LDS.  Load j of thread t writes VB bytes at LDS byte VB * (t + NT*j),
// so each wave's load fills one contiguous stretch of LDS, lane after lane.
// The slot at element offset p = EPL * (t + NT*j) must hold the tile element
// the swizzled layout keeps there, swizzle^-1(p) = swizzle(p) (S >= B makes
// the swizzle an involution: the XOR source bits are left as they are).
// 16-byte loads for 2-byte elements (M >= 3 keeps the 8 elements of a slot
// consecutive in one tile row); 4-byte loads otherwise: one element each
// for 4-byte elements, whose swizzle moves single elements, and 4-byte runs
// (which M >= 1 resp. M >= 2 keeps together) for the narrow-row kinds of
// smaller elements and the 8-bit kind.  As with the lane maps,
// swizzle(EPL*(t + NT*j)) = swizzle(EPL*t) ^ swizzle(EPL*NT*j): the bits of
// the two terms are disjoint, so each lane keeps one base and every load
// adds a wave-uniform XOR.
// ---------------------------------------------------------------------------
template <int KIND>
struct Direct {
    using K = Kind<KIND>;
    // bytes per lane per load: 16 for the 2-byte tile kinds (M >= 3 keeps 8
    // elements together); 4 otherwise (one 4-byte element; the 4-byte runs
    // of the narrow-row kinds; four 1-byte ones of the 8-bit kind, whose
    // swizzle keeps only 8-byte runs together and no 8-byte direct load
    // exists)
    static constexpr int VB = K::ESZ == 2 && K::VEC == 16 ? 16 : 4;
    static constexpr int EPL = VB / K::ESZ;          // elements per lane per load
    static constexpr int LOADS = K::TR * K::TC / EPL / K::NT;
};

// The wave-uniform part of every LDS access of a tile kernel, in element
// units, computed on the host once per launch (step_moves): step i of a lane
// is at base ^ w[i] / r[i] for swizzled and plain rows (the moved bits never
// overlap the lane's own, and the swizzle is linear over GF(2)) and at
// base + w[i] / r[i] for padded rows; direct load j fills the slots of lane
// base ^ d[j].  Kernels get them as an argument, so no wave re-derives
// swizzle(move) from run-time (B, M, S).
constexpr int kMaxSteps = 16;
struct StepMoves {
    uint32_t w[kMaxSteps];  // LDS stores
    uint32_t r[kMaxSteps];  // LDS loads
    uint32_t d[kMaxSteps];  // direct HBM -> LDS loads
};

// Whole tiles per workgroup of the whole-tile (interior) launch, stacked
// where that lengthens the HBM runs or keeps more requests in flight:
// interior_stack tiles down the source rows times interior_stack_cols tiles
// along them.  The 64 x 64 16-bit transposes take two tiles down the rows, so
// each output row gets one 256-byte run of the pair; the fp32 32 x 32
// transpose takes 2 x 2 tiles (1,024 threads: 256-byte runs on both sides);
// staging takes four 64 x 64 K-tiles side by side along k (its k runs along
// the rows of the operand), so each operand row gives a 512-byte run and
// each row block of fragments an 8 KiB one.  Measured on fp16 8192 x 8192:
// +4% (4x4 reads) and +3% (transpose reads); fp32 4096 x 4096: +1.5-2% with
// 2 x 2, -5% with two down the rows, -7% with two along them; staging both
// 8192 x 4096 operands (then in 256 x 64 tiles): +3% with two, +4% with
// four.  The byte tile lost 2% (rows) to 10% (2 x 2), the whole-row tiles
// of narrow matrices 2% (fp32, fp16) and 8% (bytes), and the 8x8-read 16-bit
// tile gained under 1% down the rows and lost 2% in 2 x 2, so they keep one
// tile per workgroup.  Edge tiles always take a workgroup each.
constexpr int interior_stack(int kind) {
    return kind == SWZ_READ_B64_4X4 || kind == SWZ_READ_B64_TR16 || kind == SWZ_READ_SCALAR_COL ? 2
           : kind == SWZ_READ_MFMA_16X16X32                                                       ? 4
                                                                                                   : 1;
}

constexpr int interior_stack_cols(int kind) {
    return kind == SWZ_READ_SCALAR_COL ? 2 : 1;
}

// Whether a transpose of `rows` source rows of esz-byte elements writes its
// output rows at a pitch that is not a whole number of 64-byte pieces, at a
// size where the XCD-grouped block grid pays (tile kernels with 16-byte
// aligned rows).  Output rows 32 bytes off such a piece left each piece
// half-written by two workgroups and ran at 0.45-0.60 of a copy; grouping
// the neighbours on one XCD's L2 brought 0.63-0.75 (fp32, 16-bit and byte
// matrices of 2,000 to 9,000 rows).  With fewer rows the grouping lost up to
// 13%, and a source pitch off the 64-byte pieces alone did not gain.
constexpr bool partial_line_output(int64_t rows, int esz) {
    return (rows * esz) % 64 != 0 && rows >= 2000;
}

template <int KIND>
constexpr bool direct_split() {
    using D = Direct<KIND>;
    using K = Kind<KIND>;
    return D::LOADS >= 1 && D::LOADS * D::EPL * K::NT == K::TR * K::TC && (K::NT & (K::NT - 1)) == 0 &&
           (K::TC & (K::TC - 1)) == 0;
}
static_assert(direct_split<SWZ_READ_SCALAR_COL>() && direct_split<SWZ_READ_B64_4X4>() &&
                  direct_split<SWZ_READ_B128_8X8>() && direct_split<SWZ_READ_MFMA_16X16X32>() &&
                  direct_split<SWZ_READ_B64_TR16>() && direct_split<SWZ_READ_B64_TR8>() &&
                  direct_split<SWZ_READ_NARROW1>() && direct_split<SWZ_READ_NARROW2>() &&
                  direct_split<SWZ_READ_NARROW4>() && direct_split<SWZ_READ_NARROW8>() &&
                  direct_split<SWZ_READ_NARROW16>() && direct_split<SWZ_READ_HNARROW1>() &&
                  direct_split<SWZ_READ_HNARROW32>() && direct_split<SWZ_READ_BNARROW1>() &&
                  direct_split<SWZ_READ_BNARROW64>(),
              "direct fill split");

}  // namespace swz
