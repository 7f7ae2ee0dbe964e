// Tile staging kernels for gfx950: coalesced row loads from HBM into an LDS
// tile laid out by Swizzle<B,M,S> (or padded / plain rows), a read back
// along columns or in the operand-fragment pattern, and coalesced row stores.
//
// The method is the one of "CuTe Swizzle 学习手册" (typical scenario: column
// access of a row-major tile; swizzle formula) and "CUDA 013 - Swizzle 的
// 工作原理" (sections 如何避免 Bank Conflict, Swizzle 技术, 更通用的映射规则):
// remap the flat offset of each tile element so that the rows written by a
// wave and the columns read by a wave both spread over all LDS banks.
#include <type_traits>

#include "launch.h"

namespace swz {
namespace {

constexpr int64_t kMaxGrid = int64_t(1) << 20;

__device__ __forceinline__ void decode_tile(int64_t t, int64_t tiles_r, int64_t tiles_c, int64_t& b, int64_t& tr,
                                            int64_t& tc) {
    tc = t % tiles_c;
    const int64_t q = t / tiles_c;
    tr = q % tiles_r;
    b = q / tiles_r;
}

// ---------------------------------------------------------------------------
// 4-byte elements, 32x32 tile, scalar column reads.
// ---------------------------------------------------------------------------

// One tile: FULL tiles take straight-line unguarded loads and stores so all
// loads of a thread are in flight together; edge tiles check every element.
template <bool FULL>
__device__ __forceinline__ void scalar_col_tile(const uint32_t* __restrict__ S, uint32_t* __restrict__ D, int64_t rows,
                                                int64_t cols, int64_t r0, int64_t c0, uint32_t* lds,
                                                const uint32_t* woff, const uint32_t* roff, int t) {
    using K = Kind<SWZ_READ_SCALAR_COL>;
    uint32_t v[K::WSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        v[i] = (FULL || (r0 + r < rows && c0 + c < cols)) ? S[(r0 + r) * cols + c0 + c] : 0u;
    }
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) lds[woff[i]] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        int r, c;
        K::rcoord(t, i, r, c);
        const uint32_t x = lds[roff[i]];
        if (FULL || (r0 + r < rows && c0 + c < cols)) D[(c0 + c) * rows + r0 + r] = x;
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void k_scalar_col(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                    int64_t rows, int64_t cols, int64_t tiles_r, int64_t tiles_c,
                                                    int64_t n_tiles, LdsLayout L) {
    using K = Kind<SWZ_READ_SCALAR_COL>;
    __shared__ uint32_t lds[K::TR * (K::TC + 1)];
    const int t = threadIdx.x;

    // LDS offsets depend only on the lane, not on the tile.
    uint32_t woff[K::WSTEPS], roff[K::RSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        woff[i] = lds_elem(L, r, c);
    }
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        int r, c;
        K::rcoord(t, i, r, c);
        roff[i] = lds_elem(L, r, c);
    }

    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        int64_t b, tr, tc;
        decode_tile(tile, tiles_r, tiles_c, b, tr, tc);
        const int64_t r0 = tr * K::TR, c0 = tc * K::TC;
        const uint32_t* S = src + b * rows * cols;
        uint32_t* D = dst + b * rows * cols;
        if ((r0 + K::TR <= rows) && (c0 + K::TC <= cols))
            scalar_col_tile<true>(S, D, rows, cols, r0, c0, lds, woff, roff, t);
        else
            scalar_col_tile<false>(S, D, rows, cols, r0, c0, lds, woff, roff, t);
    }
}

// ---------------------------------------------------------------------------
// 2-byte elements: 16-byte staging stores, 8- or 16-byte column-block reads
// and an in-register transpose of 16-bit elements.
// ---------------------------------------------------------------------------

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

__device__ __forceinline__ uint4 load8_guarded(const uint16_t* S, int64_t row, int64_t col, int64_t rows,
                                               int64_t cols) {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (row < rows && col + e < cols) ? S[row * cols + col + e] : 0u;
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

__device__ __forceinline__ void store8_guarded(uint16_t* D, int64_t row, int64_t col, int64_t nrows, int64_t ncols,
                                               const uint4& o) {
    if (row >= nrows) return;
    const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (col + e < ncols) D[row * ncols + col + e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
}

// One tile.  VEC: 16-byte global loads and stores (tile wholly inside the
// matrix and all pitches 16-byte multiples); otherwise every element is
// checked against the matrix bounds.
template <int KIND, bool VEC>
__device__ __forceinline__ void vec16_tile(const uint16_t* __restrict__ S, uint16_t* __restrict__ D, int64_t rows,
                                           int64_t cols, int64_t r0, int64_t c0, uint16_t* lds, const uint32_t* woff,
                                           const uint32_t* roff, int t, int rb, int cb) {
    using K = Kind<KIND>;
    uint4 v[K::WSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        if (VEC)
            v[i] = *reinterpret_cast<const uint4*>(S + (r0 + r) * cols + c0 + c);
        else
            v[i] = load8_guarded(S, r0 + r, c0 + c, rows, cols);
    }
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) *reinterpret_cast<uint4*>(lds + woff[i]) = v[i];
    __syncthreads();

    // Read 8 rows of this thread's column block, transpose in registers and
    // write one 16-byte piece of each output row (= source column).
    using R = typename std::conditional<K::RWIDTH == 8, uint2, uint4>::type;
    constexpr int kCols = K::RWIDTH / 2;
    R x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const R*>(lds + roff[i]);
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
        const uint4 o = make_uint4(pair_col(x[0], x[1], j), pair_col(x[2], x[3], j), pair_col(x[4], x[5], j),
                                   pair_col(x[6], x[7], j));
        const int64_t orow = c0 + cb + j, ocol = r0 + rb;
        if (VEC)
            *reinterpret_cast<uint4*>(D + orow * rows + ocol) = o;
        else
            store8_guarded(D, orow, ocol, cols, rows, o);
    }
    __syncthreads();
}

template <int KIND, bool ALIGNED>
__global__ __launch_bounds__(128) void k_vec16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                               int64_t rows, int64_t cols, int64_t tiles_r, int64_t tiles_c,
                                               int64_t n_tiles, LdsLayout L) {
    using K = Kind<KIND>;
    static_assert(K::ESZ == 2 && K::VEC == 16 && K::NT == 128, "16-bit vector staging");
    constexpr int kLdsElems = K::TR * (K::TC + 8);
    __shared__ uint4 lds_v[kLdsElems * 2 / 16];
    uint16_t* lds = reinterpret_cast<uint16_t*>(lds_v);
    const int t = threadIdx.x;

    uint32_t woff[K::WSTEPS], roff[K::RSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        woff[i] = lds_elem(L, r, c);
    }
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        int r, c;
        K::rcoord(t, i, r, c);
        roff[i] = lds_elem(L, r, c);
    }
    int rb, cb;  // first row / column of this thread's read block
    K::rcoord(t, 0, rb, cb);

    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        int64_t b, tr, tc;
        decode_tile(tile, tiles_r, tiles_c, b, tr, tc);
        const int64_t r0 = tr * K::TR, c0 = tc * K::TC;
        const uint16_t* S = src + b * rows * cols;
        uint16_t* D = dst + b * rows * cols;
        if (ALIGNED && (r0 + K::TR <= rows) && (c0 + K::TC <= cols))
            vec16_tile<KIND, true>(S, D, rows, cols, r0, c0, lds, woff, roff, t, rb, cb);
        else
            vec16_tile<KIND, false>(S, D, rows, cols, r0, c0, lds, woff, roff, t, rb, cb);
    }
}

// ---------------------------------------------------------------------------
// Operand staging: 256x64 K-tiles of a K-contiguous 16-bit operand, read
// back as 16x16x32 operand fragments and written out in lane order.
// ---------------------------------------------------------------------------
template <bool FULL>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ src, uint4* __restrict__ frag, int64_t mn,
                                           int64_t k, int64_t r0, int64_t k0, uint16_t* lds, const uint32_t* woff,
                                           const uint32_t* roff, int t) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
    const int lane = t % 64;
    uint4 v[K::WSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        // mn and k are multiples of 16 and 32, so a 16-byte chunk is either
        // wholly inside the operand or wholly outside.
        v[i] = (FULL || (r0 + r < mn && k0 + c < k)) ? *reinterpret_cast<const uint4*>(src + (r0 + r) * k + k0 + c)
                                                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) *reinterpret_cast<uint4*>(lds + woff[i]) = v[i];
    __syncthreads();
    const int64_t ksteps = k / 32;
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        const int f = K::frag_of(t, i);
        const int blk = f % 16, ks = f / 16;
        const uint4 x = *reinterpret_cast<const uint4*>(lds + roff[i]);
        if (FULL || (r0 + 16 * blk < mn && k0 + 32 * ks < k)) {
            const int64_t fi = (r0 / 16 + blk) * ksteps + (k0 / 32 + ks);
            frag[fi * 64 + lane] = x;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void k_stage(const uint16_t* __restrict__ src, uint4* __restrict__ frag, int64_t mn,
                                               int64_t k, int64_t tiles_k, int64_t n_tiles, LdsLayout L) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
    __shared__ uint4 lds_v[K::TR * (K::TC + 8) * 2 / 16];
    uint16_t* lds = reinterpret_cast<uint16_t*>(lds_v);
    const int t = threadIdx.x;

    uint32_t woff[K::WSTEPS], roff[K::RSTEPS];
#pragma unroll
    for (int i = 0; i < K::WSTEPS; ++i) {
        int r, c;
        K::wcoord(t, i, r, c);
        woff[i] = lds_elem(L, r, c);
    }
#pragma unroll
    for (int i = 0; i < K::RSTEPS; ++i) {
        int r, c;
        K::rcoord(t, i, r, c);
        roff[i] = lds_elem(L, r, c);
    }

    for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        const int64_t tm = tile / tiles_k, tk = tile % tiles_k;
        const int64_t r0 = tm * K::TR, k0 = tk * K::TC;
        if (r0 + K::TR <= mn && k0 + K::TC <= k)
            stage_tile<true>(src, frag, mn, k, r0, k0, lds, woff, roff, t);
        else
            stage_tile<false>(src, frag, mn, k, r0, k0, lds, woff, roff, t);
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_convert(int kind, const ConvertJob& j, hipStream_t stream) {
    int tr = 0, tc = 0;
    switch (kind) {
        case SWZ_READ_SCALAR_COL: tr = Kind<SWZ_READ_SCALAR_COL>::TR; tc = Kind<SWZ_READ_SCALAR_COL>::TC; break;
        case SWZ_READ_B64_4X4: tr = Kind<SWZ_READ_B64_4X4>::TR; tc = Kind<SWZ_READ_B64_4X4>::TC; break;
        case SWZ_READ_B128_8X8: tr = Kind<SWZ_READ_B128_8X8>::TR; tc = Kind<SWZ_READ_B128_8X8>::TC; break;
        default: return hipErrorInvalidValue;
    }
    const int64_t tiles_r = ceil_div(j.rows, tr), tiles_c = ceil_div(j.cols, tc);
    const int64_t n_tiles = j.batch * tiles_r * tiles_c;
    if (n_tiles == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(n_tiles < kMaxGrid ? n_tiles : kMaxGrid);
    switch (kind) {
        case SWZ_READ_SCALAR_COL:
            hipLaunchKernelGGL(k_scalar_col, dim3(grid), dim3(Kind<SWZ_READ_SCALAR_COL>::NT), 0, stream,
                               static_cast<const uint32_t*>(j.src), static_cast<uint32_t*>(j.dst), j.rows, j.cols,
                               tiles_r, tiles_c, n_tiles, j.layout);
            break;
        case SWZ_READ_B64_4X4:
            if (j.aligned)
                hipLaunchKernelGGL((k_vec16<SWZ_READ_B64_4X4, true>), dim3(grid), dim3(128), 0, stream,
                                   static_cast<const uint16_t*>(j.src), static_cast<uint16_t*>(j.dst), j.rows,
                                   j.cols, tiles_r, tiles_c, n_tiles, j.layout);
            else
                hipLaunchKernelGGL((k_vec16<SWZ_READ_B64_4X4, false>), dim3(grid), dim3(128), 0, stream,
                                   static_cast<const uint16_t*>(j.src), static_cast<uint16_t*>(j.dst), j.rows,
                                   j.cols, tiles_r, tiles_c, n_tiles, j.layout);
            break;
        case SWZ_READ_B128_8X8:
            if (j.aligned)
                hipLaunchKernelGGL((k_vec16<SWZ_READ_B128_8X8, true>), dim3(grid), dim3(128), 0, stream,
                                   static_cast<const uint16_t*>(j.src), static_cast<uint16_t*>(j.dst), j.rows,
                                   j.cols, tiles_r, tiles_c, n_tiles, j.layout);
            else
                hipLaunchKernelGGL((k_vec16<SWZ_READ_B128_8X8, false>), dim3(grid), dim3(128), 0, stream,
                                   static_cast<const uint16_t*>(j.src), static_cast<uint16_t*>(j.dst), j.rows,
                                   j.cols, tiles_r, tiles_c, n_tiles, j.layout);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_stage(const StageJob& j, hipStream_t stream) {
    using K = Kind<SWZ_READ_MFMA_16X16X32>;
    const int64_t tiles_m = ceil_div(j.mn, K::TR), tiles_k = ceil_div(j.k, K::TC);
    const int64_t n_tiles = tiles_m * tiles_k;
    if (n_tiles == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(n_tiles < kMaxGrid ? n_tiles : kMaxGrid);
    hipLaunchKernelGGL(k_stage, dim3(grid), dim3(K::NT), 0, stream, static_cast<const uint16_t*>(j.src),
                       static_cast<uint4*>(j.frag), j.mn, j.k, tiles_k, n_tiles, j.layout);
    return hipGetLastError();
}

}  // namespace swz
