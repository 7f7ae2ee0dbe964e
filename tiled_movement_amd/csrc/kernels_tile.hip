// Tile staging kernels for gfx950: coalesced 16-byte row loads from HBM into
// an LDS tile laid out by Swizzle<B,M,S> (or padded / plain rows), a read back
// along columns or in the operand-fragment pattern, and coalesced 16-byte
// row stores.
//
// The method is the one of "CuTe Swizzle 学习手册" (typical scenario: column
// access of a row-major tile; swizzle formula) and "CUDA 013 - Swizzle 的
// 工作原理" (sections 如何避免 Bank Conflict, Swizzle 技术, 更通用的映射规则):
// remap the flat offset of each tile element so that the rows written by a
// wave and the columns read by a wave both spread over all LDS banks.
//
// Each workgroup loops over tiles (grid sized to the resident capacity of
// the GPU).  The next tile's global loads are issued as soon as the current
// tile sits in LDS, so they are in flight while the current tile is read
// back and stored.
#include <type_traits>

#include "launch.h"

namespace swz {
namespace {

__device__ __forceinline__ void decode_tile(int64_t t, int64_t tiles_r, int64_t tiles_c, int64_t& b, int64_t& tr,
                                            int64_t& tc) {
    tc = t % tiles_c;
    const int64_t q = t / tiles_c;
    tr = q % tiles_r;
    b = q / tiles_r;
}

// Word `w` of an 8- or 16-byte register group.
__device__ __forceinline__ uint32_t word(const uint2& x, int w) { return w == 0 ? x.x : x.y; }
__device__ __forceinline__ uint32_t word(const uint4& x, int w) {
    return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
}

// Element j of row a in the low half, element j of row b in the high half.
template <typename V>
__device__ __forceinline__ uint32_t pair_col(const V& a, const V& b, int j) {
    const uint32_t wa = word(a, j >> 1), wb = word(b, j >> 1);
    return (j & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// 16 bytes = 16/ESZ consecutive elements of one row, zero outside the matrix.
template <int ESZ>
__device__ __forceinline__ uint4 load16_guarded(const uint8_t* S, int64_t row, int64_t col, int64_t rows,
                                                int64_t cols) {
    constexpr int N = 16 / ESZ;
    uint32_t e[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const bool in = row < rows && col + k < cols;
        if (ESZ == 4)
            e[k] = in ? reinterpret_cast<const uint32_t*>(S)[row * cols + col + k] : 0u;
        else
            e[k] = in ? reinterpret_cast<const uint16_t*>(S)[row * cols + col + k] : 0u;
    }
    if (ESZ == 4) return make_uint4(e[0], e[1], e[2], e[3]);
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
}

template <int ESZ>
__device__ __forceinline__ void store16_guarded(uint8_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                                const uint4& o) {
    if (row >= nrows) return;
    const uint32_t w[4] = {o.x, o.y, o.z, o.w};
    if (ESZ == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (col + k < ncols) reinterpret_cast<uint32_t*>(D)[row * ncols + col + k] = w[k];
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (col + k < ncols)
                reinterpret_cast<uint16_t*>(D)[row * ncols + col + k] = static_cast<uint16_t>(w[k >> 1] >> (16 * (k & 1)));
    }
}

// Global loads of one tile into registers.  VEC: unguarded 16-byte loads
// (whole tile inside the matrix, 16-byte aligned rows); else per element.
template <int KIND, bool VEC>
__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ S, int64_t rows, int64_t cols, int64_t r0,
                                          int64_t c0, int t, uint4* v) {
    using K = Kind<KIND>;
    constexpr int PER = 16 / K::ESZ;  // elements per global load
#pragma unroll
    for (int j = 0; j < K::GLOADS; ++j) {
        int r, c;
        K::wcoord(t, j * (K::WSTEPS / K::GLOADS), r, c);
        c -= c % PER;  // the vector's first column
        if (VEC)
            v[j] = *reinterpret_cast<const uint4*>(S + ((r0 + r) * cols + c0 + c) * K::ESZ);
        else
            v[j] = load16_guarded<K::ESZ>(S, r0 + r, c0 + c, rows, cols);
    }
}

// ---------------------------------------------------------------------------
// Transpose / layout conversion.  One kernel template for the three read
// kinds; D holds the transposed tile of every batch entry.
// ---------------------------------------------------------------------------
template <int KIND>
struct LdsTile {
    using K = Kind<KIND>;
    // Room for the padded layout: one extra element (4-byte) or vector.
    static constexpr int PAD = K::ESZ == 4 ? 1 : 8;
    static constexpr int BYTES = K::TR * (K::TC + PAD) * K::ESZ;
};

// Element offset in LDS of step i of this lane: the lane's first offset
// `base` combined with the step's lane-independent move (see steps_decompose).
// PADDED: rows of TC + PAD elements, offsets add (compile-time constants).
// Otherwise rows of TC elements under Swizzle<B,M,S> (B = 0: plain rows),
// offsets combine by XOR with a value uniform across the wave.
template <int KIND, bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t step_off(uint32_t base, int i, const LdsLayout& L) {
    using K = Kind<KIND>;
    int dr = 0, dc = 0;
    coord<KIND, WRITE>(0, i, dr, dc);
    if (PADDED) return base + static_cast<uint32_t>(dr * (K::TC + LdsTile<KIND>::PAD) + dc);
    return base ^ swizzle(static_cast<uint32_t>(dr * K::TC + dc), L.B, L.M, L.S);
}

template <int KIND, bool WRITE, bool PADDED>
__device__ __forceinline__ uint32_t lane_base(int t, const LdsLayout& L) {
    using K = Kind<KIND>;
    int r = 0, c = 0;
    coord<KIND, WRITE>(t, 0, r, c);
    if (PADDED) return static_cast<uint32_t>(r * (K::TC + LdsTile<KIND>::PAD) + c);
    return swizzle(static_cast<uint32_t>(r * K::TC + c), L.B, L.M, L.S);
}

// Write the staged registers into LDS.
template <int KIND, bool PADDED>
__device__ __forceinline__ void lds_store(uint8_t* lds, uint32_t wbase, const LdsLayout& L, const uint4* v) {
    using K = Kind<KIND>;
    if constexpr (K::ESZ == 4) {
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) {
            const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                reinterpret_cast<uint32_t*>(lds)[step_off<KIND, true, PADDED>(wbase, 4 * j + e, L)] = w[e];
        }
    } else {
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j)
            *reinterpret_cast<uint4*>(lds + 2 * step_off<KIND, true, PADDED>(wbase, j, L)) = v[j];
    }
}

// Read this thread's pieces of the tile back from LDS, transposed, and store
// them to the output.  FULL: unguarded 16-byte stores.
template <int KIND, bool PADDED, bool FULL>
__device__ __forceinline__ void lds_read_store(const uint8_t* lds, uint32_t rbase, const LdsLayout& L,
                                               uint8_t* __restrict__ D, int64_t rows, int64_t cols, int64_t r0,
                                               int64_t c0, int t) {
    using K = Kind<KIND>;
    if constexpr (KIND == SWZ_READ_SCALAR_COL) {
        // Task j: four rows of one source column -> 16 bytes of an output row.
#pragma unroll
        for (int j = 0; j < K::TASKS; ++j) {
            uint32_t x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = reinterpret_cast<const uint32_t*>(lds)[step_off<KIND, false, PADDED>(rbase, 4 * j + e, L)];
            int r = 0, c = 0;
            K::rcoord(t, 4 * j, r, c);
            const uint4 o = make_uint4(x[0], x[1], x[2], x[3]);
            const int64_t orow = c0 + c, ocol = r0 + r;
            if (FULL)
                *reinterpret_cast<uint4*>(D + (orow * rows + ocol) * 4) = o;
            else
                store16_guarded<4>(D, orow, ocol, cols, rows, o);
        }
    } else {
        // Task j: 8 rows of a column block; transpose 16-bit elements in
        // registers and write one 16-byte piece of each output row.
        using R = typename std::conditional<K::RWIDTH == 8, uint2, uint4>::type;
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
                const uint4 o = make_uint4(pair_col(x[0], x[1], q), pair_col(x[2], x[3], q),
                                           pair_col(x[4], x[5], q), pair_col(x[6], x[7], q));
                const int64_t orow = c0 + cb + q, ocol = r0 + rb;
                if (FULL)
                    *reinterpret_cast<uint4*>(D + (orow * rows + ocol) * 2) = o;
                else
                    store16_guarded<2>(D, orow, ocol, cols, rows, o);
            }
        }
    }
}

template <int KIND, bool PADDED, bool ALIGNED>
__global__ __launch_bounds__(Kind<KIND>::NT) void k_convert(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            int64_t rows, int64_t cols, int64_t tiles_r,
                                                            int64_t tiles_c, int64_t n_tiles, LdsLayout L) {
    using K = Kind<KIND>;
    __shared__ uint4 lds_v[LdsTile<KIND>::BYTES / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds_v);
    const int t = threadIdx.x;
    const int64_t plane = rows * cols * K::ESZ;  // bytes of one batch entry
    const uint32_t wbase = lane_base<KIND, true, PADDED>(t, L);
    const uint32_t rbase = lane_base<KIND, false, PADDED>(t, L);

    auto full_tile = [&](int64_t r0, int64_t c0) { return ALIGNED && r0 + K::TR <= rows && c0 + K::TC <= cols; };

    int64_t tile = blockIdx.x;
    if (tile >= n_tiles) return;
    uint4 v[K::GLOADS];
    int64_t b, tr, tc;
    decode_tile(tile, tiles_r, tiles_c, b, tr, tc);
    int64_t r0 = tr * K::TR, c0 = tc * K::TC;
    if (full_tile(r0, c0))
        load_tile<KIND, true>(src + b * plane, rows, cols, r0, c0, t, v);
    else
        load_tile<KIND, false>(src + b * plane, rows, cols, r0, c0, t, v);

    for (;;) {
        lds_store<KIND, PADDED>(lds, wbase, L, v);
        __syncthreads();

        // Prefetch the next tile while this one is read back and stored.
        const int64_t next = tile + gridDim.x;
        int64_t nb = 0, ntr = 0, ntc = 0;
        if (next < n_tiles) {
            decode_tile(next, tiles_r, tiles_c, nb, ntr, ntc);
            if (full_tile(ntr * K::TR, ntc * K::TC))
                load_tile<KIND, true>(src + nb * plane, rows, cols, ntr * K::TR, ntc * K::TC, t, v);
            else
                load_tile<KIND, false>(src + nb * plane, rows, cols, ntr * K::TR, ntc * K::TC, t, v);
        }

        if (full_tile(r0, c0))
            lds_read_store<KIND, PADDED, true>(lds, rbase, L, dst + b * plane, rows, cols, r0, c0, t);
        else
            lds_read_store<KIND, PADDED, false>(lds, rbase, L, dst + b * plane, rows, cols, r0, c0, t);
        __syncthreads();

        if (next >= n_tiles) break;
        tile = next;
        b = nb;
        r0 = ntr * K::TR;
        c0 = ntc * K::TC;
    }
}

// ---------------------------------------------------------------------------
// Operand staging: 256x64 K-tiles of a K-contiguous 16-bit operand, read
// back as 16x16x32 operand fragments and written out in lane order.
// ---------------------------------------------------------------------------
template <bool FULL>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ src, int64_t mn, int64_t k, int64_t r0,
                                           int64_t k0, int t, uint4* v) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
#pragma unroll
    for (int j = 0; j < K::GLOADS; ++j) {
        int r, c;
        K::wcoord(t, j, r, c);
        // mn and k are multiples of 16 and 32, so a 16-byte chunk is either
        // wholly inside the operand or wholly outside.
        v[j] = (FULL || (r0 + r < mn && k0 + c < k)) ? *reinterpret_cast<const uint4*>(src + (r0 + r) * k + k0 + c)
                                                     : make_uint4(0u, 0u, 0u, 0u);
    }
}

template <bool PADDED>
__global__ __launch_bounds__(Kind<SWZ_READ_MFMA_16X16X32>::NT) void k_stage(const uint16_t* __restrict__ src,
                                                                            uint4* __restrict__ frag, int64_t mn,
                                                                            int64_t k, int64_t tiles_k,
                                                                            int64_t n_tiles, LdsLayout L) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
    __shared__ uint4 lds_v[LdsTile<SWZ_READ_MFMA_16X16X32>::BYTES / 16];
    uint16_t* lds = reinterpret_cast<uint16_t*>(lds_v);
    const int t = threadIdx.x, lane = t % 64;

    constexpr int KD = SWZ_READ_MFMA_16X16X32;
    const uint32_t wbase = lane_base<KD, true, PADDED>(t, L);
    const uint32_t rbase = lane_base<KD, false, PADDED>(t, L);
    const int64_t ksteps = k / 32;
    auto full_tile = [&](int64_t r0, int64_t k0) { return r0 + K::TR <= mn && k0 + K::TC <= k; };

    int64_t tile = blockIdx.x;
    if (tile >= n_tiles) return;
    int64_t r0 = (tile / tiles_k) * K::TR, k0 = (tile % tiles_k) * K::TC;
    uint4 v[K::GLOADS];
    if (full_tile(r0, k0))
        stage_load<true>(src, mn, k, r0, k0, t, v);
    else
        stage_load<false>(src, mn, k, r0, k0, t, v);

    for (;;) {
#pragma unroll
        for (int j = 0; j < K::GLOADS; ++j) *reinterpret_cast<uint4*>(lds + step_off<KD, true, PADDED>(wbase, j, L)) = v[j];
        __syncthreads();

        const int64_t next = tile + gridDim.x;
        const int64_t nr0 = (next / tiles_k) * K::TR, nk0 = (next % tiles_k) * K::TC;
        if (next < n_tiles) {
            if (full_tile(nr0, nk0))
                stage_load<true>(src, mn, k, nr0, nk0, t, v);
            else
                stage_load<false>(src, mn, k, nr0, nk0, t, v);
        }

        const bool full = full_tile(r0, k0);
#pragma unroll
        for (int i = 0; i < K::RSTEPS; ++i) {
            const int f = K::frag_of(t, i);
            const int blk = f % 16, ks = f / 16;
            const uint4 x = *reinterpret_cast<const uint4*>(lds + step_off<KD, false, PADDED>(rbase, i, L));
            if (full || (r0 + 16 * blk < mn && k0 + 32 * ks < k)) {
                const int64_t fi = (r0 / 16 + blk) * ksteps + (k0 / 32 + ks);
                frag[fi * 64 + lane] = x;
            }
        }
        __syncthreads();
        if (next >= n_tiles) break;
        tile = next;
        r0 = nr0;
        k0 = nk0;
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename F>
int64_t grid_for(F kernel, int threads, int64_t n_tiles) {
    return resident_grid(reinterpret_cast<const void*>(kernel), threads, n_tiles);
}

template <int KIND, bool PADDED, bool ALIGNED>
void launch_variant(const ConvertJob& j, int64_t tiles_r, int64_t tiles_c, int64_t n_tiles, hipStream_t stream) {
    using K = Kind<KIND>;
    const int64_t grid = grid_for(k_convert<KIND, PADDED, ALIGNED>, K::NT, n_tiles);
    hipLaunchKernelGGL((k_convert<KIND, PADDED, ALIGNED>), dim3(static_cast<unsigned>(grid)), dim3(K::NT), 0, stream,
                       static_cast<const uint8_t*>(j.src), static_cast<uint8_t*>(j.dst), j.rows, j.cols, tiles_r,
                       tiles_c, n_tiles, j.layout);
}

template <int KIND>
hipError_t launch_kind(const ConvertJob& j, hipStream_t stream) {
    using K = Kind<KIND>;
    const int64_t tiles_r = ceil_div(j.rows, K::TR), tiles_c = ceil_div(j.cols, K::TC);
    const int64_t n_tiles = j.batch * tiles_r * tiles_c;
    if (n_tiles == 0) return hipSuccess;
    const bool padded = j.layout.ld != static_cast<uint32_t>(K::TC);
    if (padded && j.layout.ld != static_cast<uint32_t>(K::TC + LdsTile<KIND>::PAD)) return hipErrorInvalidValue;
    if (padded) {
        if (j.aligned)
            launch_variant<KIND, true, true>(j, tiles_r, tiles_c, n_tiles, stream);
        else
            launch_variant<KIND, true, false>(j, tiles_r, tiles_c, n_tiles, stream);
    } else {
        if (j.aligned)
            launch_variant<KIND, false, true>(j, tiles_r, tiles_c, n_tiles, stream);
        else
            launch_variant<KIND, false, false>(j, tiles_r, tiles_c, n_tiles, stream);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_convert(int kind, const ConvertJob& j, hipStream_t stream) {
    switch (kind) {
        case SWZ_READ_SCALAR_COL: return launch_kind<SWZ_READ_SCALAR_COL>(j, stream);
        case SWZ_READ_B64_4X4: return launch_kind<SWZ_READ_B64_4X4>(j, stream);
        case SWZ_READ_B128_8X8: return launch_kind<SWZ_READ_B128_8X8>(j, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stage(const StageJob& j, hipStream_t stream) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
    const int64_t tiles_m = ceil_div(j.mn, K::TR), tiles_k = ceil_div(j.k, K::TC);
    const int64_t n_tiles = tiles_m * tiles_k;
    if (n_tiles == 0) return hipSuccess;
    const bool padded = j.layout.ld != static_cast<uint32_t>(K::TC);
    if (padded && j.layout.ld != static_cast<uint32_t>(K::TC + LdsTile<SWZ_READ_MFMA_16X16X32>::PAD))
        return hipErrorInvalidValue;
    const auto* s = static_cast<const uint16_t*>(j.src);
    auto* f = static_cast<uint4*>(j.frag);
    if (padded) {
        const int64_t grid = grid_for(k_stage<true>, K::NT, n_tiles);
        hipLaunchKernelGGL(k_stage<true>, dim3(static_cast<unsigned>(grid)), dim3(K::NT), 0, stream, s, f, j.mn, j.k,
                           tiles_k, n_tiles, j.layout);
    } else {
        const int64_t grid = grid_for(k_stage<false>, K::NT, n_tiles);
        hipLaunchKernelGGL(k_stage<false>, dim3(static_cast<unsigned>(grid)), dim3(K::NT), 0, stream, s, f, j.mn, j.k,
                           tiles_k, n_tiles, j.layout);
    }
    return hipGetLastError();
}

}  // namespace swz
