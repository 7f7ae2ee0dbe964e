// C = A * B^T (fp32) from bf16 operands in their natural layouts -- A [m][k]
// row-major, B^T [n][k] row-major (B column-major) -- staged through
// swizzled LDS tiles inside the GEMM: the use the pages build the swizzle
// for ("NVIDIA CuTe Swizzle", cp.async into a swizzled tile, then ldmatrix
// feeding the MMA; "CuTe Swizzle 学习手册", usage steps 2, 3 and 5).
//
// Each k stage brings a 256 x 64 tile of A and one of B^T into LDS with
// direct HBM -> LDS loads (the cp.async role): a load writes lane l's 16
// bytes to LDS slot base + l, so the lane fetches the tile element the
// swizzled layout keeps in that slot, swizzle(p) (the swizzle is its own
// inverse for |S| >= B).  The operand reads then take each 16x16x32
// fragment straight from the tile -- lane l reads row l%16, k 8*(l/16) .. +7
// of a 16-row block with one 16-byte read -- which is the read pattern the
// chooser makes conflict-free (Swizzle<4,3,4> for this tile, the same as the
// staging call's).  With plain rows (B = 0) the same reads serialise on
// the banks; unlike the HBM-bound transposes, this kernel feeds the matrix
// unit from LDS, so the conflicts cost time.
//
// Workgroup tile 256 x 256 of C, eight waves in 4 x 2, each wave 64 x 128
// (4 x 8 blocks); two stage buffers of 64 KiB; the same epilogue as the
// fragment GEMM (accumulators out through padded per-wave LDS slices as
// whole 64-byte row runs).  From sweeps on MI355X at 8192 x 8192 x 4096:
// with every workgroup reading the same (cache-resident) operands the
// kernel ran only 3% faster, so the time goes to the schedule around the
// stage barrier, not to operand latency: after each barrier all eight waves
// asked LDS for fragments at once and the two waves of a SIMD waited
// together.  Running half of the waves half a stage behind (the ping-pong
// schedule below) took it from 1.15-1.23 to 1.22-1.28 PFLOP/s.  Four waves
// of 128 x 128 (one per SIMD) ran 1.10; raising the wave priority around the
// products, letting only the lagging waves issue the loads, giving each XCD a
// contiguous run of tiles and scheduling hints (the compiler's MFMA / LDS
// interleave strategy, or explicit groups of four products per fragment
// read) did not help; neither did 32-wide k stages (1.12, also with four
// stage buffers and loads three stages ahead) or four-wave 128 x 256
// workgroups, two per CU (1.07).
#include "gemm_epilogue.h"
#include "launch.h"

namespace swz {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Waves along m / n; each wave owns kWbM x kWbN blocks of 16 x 16.
constexpr int kWavesM = 4, kWavesN = 2, kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWbM = 4, kWbN = 8;
constexpr int kTileRows = 256;                        // rows of A / of B^T per workgroup tile
constexpr int kTileK = 64;                            // k per stage (two 32-wide steps)
constexpr int kTileBytes = kTileRows * kTileK * 2;    // one operand tile: 32 KiB
constexpr int kBufBytes = 2 * kTileBytes;             // A and B^T of one stage
constexpr int kChunks = kTileBytes / 16;              // 16-byte slots per operand tile
constexpr int64_t kMaxGridY = 65535;
static_assert(kWavesM * kWbM * 16 == kTileRows && kWavesN * kWbN * 16 == kTileRows, "wave tiles cover the tile");
static_assert(2 * kBufBytes <= 160 * 1024, "two stages fit in LDS");

__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct fill of one 256 x 64 operand tile (rows r0 .., k columns k0 ..) of
// X [rows][k] into LDS at dst.  Slot p (16 bytes, element offset 8p) receives
// tile element swizzle(8p); slots whose element lies outside the matrix are
// filled from X's first element (their rows are never stored; their k
// columns are never multiplied).  swizzle(8(t + 512q)) = swizzle(8t) ^
// swizzle(4096q): one per-lane base, one wave-uniform XOR per load.
template <int NT>  // NT threads share the fill; t < NT, wave = t / 64
__device__ __forceinline__ void fill_tile(const uint8_t* __restrict__ X, int64_t rows, int64_t k, int64_t r0,
                                          int64_t k0, lds_u8* dst, const LdsLayout& L, int t, int wave) {
    static_assert(kChunks % NT == 0, "the fill splits evenly");
    const uint32_t base = swizzle(static_cast<uint32_t>(8 * t), L.B, L.M, L.S);
#pragma unroll
    for (int q = 0; q < kChunks / NT; ++q) {
        const uint32_t e = base ^ swizzle(static_cast<uint32_t>(8 * NT * q), L.B, L.M, L.S);
        const int64_t r = r0 + e / kTileK, c = k0 + e % kTileK;
        const uint8_t* g = (r < rows && c < k) ? X + (r * k + c) * 2 : X;
        __builtin_amdgcn_global_load_lds(g, dst + 16 * (64 * wave + NT * q), 16, 0, 0);
    }
}

// This wave's operand fragments of 32-wide k step ks from the staged tiles:
// A blocks wm*kWbM + x, B^T blocks wn*kWbN + y.  Block i and step ks move
// the lane's element by (16i rows, 32ks columns), bits disjoint from the
// lane's own, so each read address is fbase ^ swizzle(move).
__device__ __forceinline__ bf16x8 read_b1(const lds_u8* t, int ks, int w, int blk, uint32_t fbase, const LdsLayout& L) {
    const uint32_t e = fbase ^ swizzle(static_cast<uint32_t>((16 * (w * kWbN + blk)) * kTileK + 32 * ks), L.B, L.M, L.S);
    return *(const __attribute__((address_space(3))) bf16x8*)(t + 2 * e);
}

__device__ __forceinline__ void read_a(const lds_u8* ta, int ks, int wm, uint32_t fbase, const LdsLayout& L, bf16x8* av) {
#pragma unroll
    for (int x = 0; x < kWbM; ++x) {
        const uint32_t e = fbase ^ swizzle(static_cast<uint32_t>((16 * (wm * kWbM + x)) * kTileK + 32 * ks), L.B, L.M, L.S);
        av[x] = *(const __attribute__((address_space(3))) bf16x8*)(ta + 2 * e);
    }
}

__device__ __forceinline__ void read_b(const lds_u8* tb, int ks, int wn, uint32_t fbase, const LdsLayout& L, bf16x8* bv) {
#pragma unroll
    for (int y = 0; y < kWbN; ++y) bv[y] = read_b1(tb, ks, wn, y, fbase, L);
}

__device__ __forceinline__ void mma_step(f32x4 (&acc)[kWbM][kWbN], const bf16x8* av, const bf16x8* bv) {
#pragma unroll
    for (int x = 0; x < kWbM; ++x)
#pragma unroll
        for (int y = 0; y < kWbN; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[x], bv[y], acc[x][y], 0, 0, 0);
}

template <bool BF16C>  // C in bf16 (rounded to nearest even) instead of fp32
__global__ __launch_bounds__(kThreads) void k_gemm_tiles(const uint8_t* __restrict__ a, const uint8_t* __restrict__ bt,
                                                         void* __restrict__ c, int64_t m, int64_t n, int64_t k,
                                                         int64_t tile_row0, LdsLayout L) {
    __shared__ bf16x8 lds_v[2 * kBufBytes / 16];
    lds_u8* lds = (lds_u8*)(reinterpret_cast<uint8_t*>(lds_v));
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
    const int lane = t % 64;
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int64_t mb = m / 16, nb = n / 16, kb = k / 32;
    const int64_t ty = blockIdx.y, tx = blockIdx.x;
    const int64_t r0a = (tile_row0 + ty) * kTileRows, r0b = tx * kTileRows;
    const int64_t bm0 = r0a / 16, bn0 = r0b / 16;
    const int64_t stages = (k + kTileK - 1) / kTileK;

    // Lane l's fragment element: row l%16 of a 16-row block, k 8*(l/16) of a
    // 32-wide step.
    const uint32_t fbase = swizzle(static_cast<uint32_t>((lane % 16) * kTileK + 8 * (lane / 16)), L.B, L.M, L.S);

    f32x4 acc[kWbM][kWbN];
#pragma unroll
    for (int x = 0; x < kWbM; ++x)
#pragma unroll
        for (int y = 0; y < kWbN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (stages > 0) {
        fill_tile<kThreads>(a, m, k, r0a, 0, lds, L, t, wave);
        fill_tile<kThreads>(bt, n, k, r0b, 0, lds + kTileBytes, L, t, wave);
    }
    // Stage s: wait until it has landed (this wave's loads; the barrier
    // covers the others) and every wave is done with stage s - 1, whose
    // buffer the next loads reuse; then start stage s + 1's loads.
    auto begin_stage = [&](int64_t s) {
        // (LDS reads of the buffer the next loads overwrite have all
        // returned: their results are used before this point, or, for
        // fragments held over a barrier, waited for here.)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        stage_barrier();
        if (s + 1 < stages) {
            lds_u8* nxt = lds + ((s + 1) & 1) * kBufBytes;
            fill_tile<kThreads>(a, m, k, r0a, (s + 1) * kTileK, nxt, L, t, wave);
            fill_tile<kThreads>(bt, n, k, r0b, (s + 1) * kTileK, nxt + kTileBytes, L, t, wave);
        }
    };
    const int64_t full = kb / 2;  // stages with both 32-wide k steps
    // Waves 0-3 and 4-7 share the SIMDs pairwise.  The first half starts
    // each stage with its fragment reads; the second half starts it with the
    // products of the previous stage's second k step, whose fragments it
    // read before the barrier, so one wave of each SIMD feeds the matrix
    // unit while the other waits for LDS.  The k steps still accumulate in
    // increasing order.
    const bool lag = wave >= kWaves / 2;
    if (!lag) {
        for (int64_t s = 0; s < full; ++s) {
            begin_stage(s);
            const lds_u8* ta = lds + (s & 1) * kBufBytes;
            const lds_u8* tb = ta + kTileBytes;
            bf16x8 a0[kWbM], bq[kWbN], a1[kWbM];
            read_a(ta, 0, wm, fbase, L, a0);
            read_b(tb, 0, wn, fbase, L, bq);
            read_a(ta, 1, wm, fbase, L, a1);
#pragma unroll
            for (int y = 0; y < kWbN; ++y) {
#pragma unroll
                for (int x = 0; x < kWbM; ++x)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[x], bq[y], acc[x][y], 0, 0, 0);
                bq[y] = read_b1(tb, 1, wn, y, fbase, L);
            }
            mma_step(acc, a1, bq);
        }
    } else {
        bf16x8 a1[kWbM], bq[kWbN];
        for (int64_t s = 0; s < full; ++s) {
            begin_stage(s);
            const lds_u8* ta = lds + (s & 1) * kBufBytes;
            const lds_u8* tb = ta + kTileBytes;
            bf16x8 a0[kWbM];
            read_a(ta, 0, wm, fbase, L, a0);
            if (s > 0) {
#pragma unroll
                for (int y = 0; y < kWbN; ++y) {
#pragma unroll
                    for (int x = 0; x < kWbM; ++x)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[x], bq[y], acc[x][y], 0, 0, 0);
                    bq[y] = read_b1(tb, 0, wn, y, fbase, L);
                }
            } else {
                read_b(tb, 0, wn, fbase, L, bq);
            }
            read_a(ta, 1, wm, fbase, L, a1);
#pragma unroll
            for (int y = 0; y < kWbN; ++y) {
#pragma unroll
                for (int x = 0; x < kWbM; ++x)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[x], bq[y], acc[x][y], 0, 0, 0);
                bq[y] = read_b1(tb, 1, wn, y, fbase, L);
            }
            // a1 and bq now hold this stage's second k step, multiplied at
            // the start of the next stage.  Every read of this buffer has
            // returned before the next barrier (begin_stage waits for them).
        }
        if (full > 0) mma_step(acc, a1, bq);
    }
    if (kb % 2) {  // a last stage with one 32-wide k step
        begin_stage(full);
        const lds_u8* ta = lds + (full & 1) * kBufBytes;
        bf16x8 av[kWbM], bv[kWbN];
        read_a(ta, 0, wm, fbase, L, av);
        read_b(ta + kTileBytes, 0, wn, fbase, L, bv);
        mma_step(acc, av, bv);
    }

    // Epilogue: through each wave's own LDS slice of the (now idle) stage
    // buffers, once every wave is done reading the last stage.
    stage_barrier();
    static_assert(kWaves * epilogue_slice_bytes<kWbN>() <= 2 * kBufBytes, "the epilogue slices fit in LDS");
    lds_f32* slice = (lds_f32*)(lds + wave * epilogue_slice_bytes<kWbN>());
    if constexpr (BF16C)
        store_c_blocks_bf16<kWbM, kWbN>(acc, slice, static_cast<uint16_t*>(c), n, bm0 + wm * kWbM, bn0 + wn * kWbN,
                                        mb, nb, lane);
    else
        store_c_blocks<kWbM, kWbN>(acc, slice, static_cast<float*>(c), n, bm0 + wm * kWbM, bn0 + wn * kWbN, mb, nb,
                                   lane);
}

}  // namespace

hipError_t launch_gemm_tiles(const void* a, const void* bt, void* c, int64_t m, int64_t n, int64_t k,
                             const LdsLayout& layout, bool bf16c, hipStream_t stream) {
    const int64_t tiles_m = (m + kTileRows - 1) / kTileRows, tiles_n = (n + kTileRows - 1) / kTileRows;
    if (tiles_m == 0 || tiles_n == 0) return hipSuccess;
    if (tiles_n > 0x7fffffff / kThreads) return hipErrorInvalidValue;
    for (int64_t t0 = 0; t0 < tiles_m; t0 += kMaxGridY) {
        const int64_t ny = tiles_m - t0 < kMaxGridY ? tiles_m - t0 : kMaxGridY;
        const dim3 grid(static_cast<unsigned>(tiles_n), static_cast<unsigned>(ny));
        const auto* pa = static_cast<const uint8_t*>(a);
        const auto* pb = static_cast<const uint8_t*>(bt);
        if (bf16c)
            hipLaunchKernelGGL(k_gemm_tiles<true>, grid, dim3(kThreads), 0, stream, pa, pb, c, m, n, k, t0, layout);
        else
            hipLaunchKernelGGL(k_gemm_tiles<false>, grid, dim3(kThreads), 0, stream, pa, pb, c, m, n, k, t0, layout);
    }
    return hipGetLastError();
}

}  // namespace swz
