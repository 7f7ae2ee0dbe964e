// Consumer of staged operand fragments: C = A * B^T in fp32 from the
// fragments swz_stage_operand writes ([rows/16][k/32][64 lanes][8] bf16, lane
// l holding row l%16 and k 8*(l/16) .. +7 of a 16x32 block), on the 16x16x32
// bf16 matrix instruction.
//
// This is the step the pages put after the swizzled staging: the operand
// read that feeds the matrix unit ("NVIDIA CuTe Swizzle", ldmatrix and
// WGMMA; "CuTe Swizzle 学习手册", usage step 5).  Because the fragments are
// stored in lane order, every fragment is one contiguous KiB: a wave moves it
// from HBM into LDS with one direct load (lane l's 16 bytes to LDS slot l)
// and reads it back with one lane-linear 16-byte read, which touches every
// bank once -- no swizzle is needed on this side, the staging pass already
// did the reordering.
//
// Workgroup tile of (waves along m x WB_M) x (waves along n x WB_N) blocks of
// 16 x 16 (the defaults: 256 x 256 of C, four waves in 2 x 2, each wave
// 128 x 128 = 8 x 8 blocks, 256 fp32 accumulators per lane).  The k loop
// moves STAGE_STEPS 32-wide steps per stage; stages are double-buffered in
// LDS: the loads of stage s+1 are in flight while stage s is multiplied.
#include "launch.h"

namespace swz {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

#ifndef SWZ_GEMM_WAVES_M  // waves along m / n; each wave owns WB_M x WB_N blocks of 16 x 16
#define SWZ_GEMM_WAVES_M 2
#endif
#ifndef SWZ_GEMM_WAVES_N
#define SWZ_GEMM_WAVES_N 2
#endif
#ifndef SWZ_GEMM_WB_M
#define SWZ_GEMM_WB_M 8
#endif
#ifndef SWZ_GEMM_WB_N
#define SWZ_GEMM_WB_N 8
#endif
#ifndef SWZ_GEMM_STAGE_STEPS  // 32-wide k steps per LDS stage
#define SWZ_GEMM_STAGE_STEPS 2
#endif

constexpr int kWavesM = SWZ_GEMM_WAVES_M, kWavesN = SWZ_GEMM_WAVES_N;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kWbM = SWZ_GEMM_WB_M, kWbN = SWZ_GEMM_WB_N;
constexpr int kTileM = kWavesM * kWbM, kTileN = kWavesN * kWbN;  // blocks per workgroup tile
constexpr int kStageSteps = SWZ_GEMM_STAGE_STEPS;
constexpr int kFragBytes = 64 * 16;                              // one fragment: 64 lanes x 16 bytes
constexpr int kStageFragsA = kTileM * kStageSteps, kStageFragsB = kTileN * kStageSteps;
constexpr int kBufBytes = (kStageFragsA + kStageFragsB) * kFragBytes;  // A and B of one stage
static_assert((kStageFragsA + kStageFragsB) % kWaves == 0, "stage loads split over the waves");
static_assert(2 * kBufBytes <= 160 * 1024, "two stages fit in LDS");
constexpr int64_t kMaxGridY = 65535;

// Issue this wave's share of stage s's direct loads into LDS buffer buf.
// Fragment f < kStageFragsA is A block f % kTileM of k step f / kTileM; the
// rest are B fragments likewise.  Blocks past the matrix edge load the
// tile's first block instead (their results are never stored); k steps past
// the end are never multiplied.
__device__ __forceinline__ void load_stage(const uint8_t* __restrict__ fa, const uint8_t* __restrict__ fb,
                                           int64_t bm0, int64_t bn0, int64_t mb, int64_t nb, int64_t kb, int64_t s,
                                           lds_u8* buf, int wave, int lane) {
    constexpr int kPerWave = (kStageFragsA + kStageFragsB) / kWaves;
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
        const int f = wave * kPerWave + q;
        const bool is_a = f < kStageFragsA;
        const int g = is_a ? f : f - kStageFragsA;
        const int tile = is_a ? kTileM : kTileN;
        const int blk = g % tile, ks = g / tile;
        int64_t kk = s * kStageSteps + ks;
        kk = kk < kb ? kk : kb - 1;
        const int64_t b0 = is_a ? bm0 : bn0, lim = is_a ? mb : nb;
        const int64_t row = b0 + blk < lim ? b0 + blk : b0;
        const uint8_t* src = (is_a ? fa : fb) + (row * kb + kk) * kFragBytes + lane * 16;
        __builtin_amdgcn_global_load_lds(src, buf + f * kFragBytes, 16, 0, 0);
    }
}

__global__ __launch_bounds__(kGemmThreads) void k_gemm_frag(const uint8_t* __restrict__ fa,
                                                             const uint8_t* __restrict__ fb, float* __restrict__ c,
                                                             int64_t m, int64_t n, int64_t k, int64_t tile_row0) {
    __shared__ bf16x8 lds_v[2 * kBufBytes / 16];
    lds_u8* lds = (lds_u8*)(reinterpret_cast<uint8_t*>(lds_v));
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int lane = threadIdx.x % 64;
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int64_t mb = m / 16, nb = n / 16, kb = k / 32;
    const int64_t bm0 = (tile_row0 + blockIdx.y) * kTileM, bn0 = static_cast<int64_t>(blockIdx.x) * kTileN;
    const int64_t stages = (kb + kStageSteps - 1) / kStageSteps;

    f32x4 acc[kWbM][kWbN];
#pragma unroll
    for (int x = 0; x < kWbM; ++x)
#pragma unroll
        for (int y = 0; y < kWbN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (stages > 0) load_stage(fa, fb, bm0, bn0, mb, nb, kb, 0, lds, wave, lane);  // k = 0: C = 0
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int64_t s = 0; s < stages; ++s) {
        lds_u8* cur = lds + (s & 1) * kBufBytes;
        if (s + 1 < stages) load_stage(fa, fb, bm0, bn0, mb, nb, kb, s + 1, lds + ((s + 1) & 1) * kBufBytes, wave, lane);
#pragma unroll
        for (int ks = 0; ks < kStageSteps; ++ks) {
            if (s * kStageSteps + ks >= kb) break;  // uniform: a k tail of one step
            bf16x8 a[kWbM], b[kWbN];
#pragma unroll
            for (int x = 0; x < kWbM; ++x)
                a[x] = *(__attribute__((address_space(3))) bf16x8*)(cur + (ks * kTileM + wm * kWbM + x) * kFragBytes + lane * 16);
#pragma unroll
            for (int y = 0; y < kWbN; ++y)
                b[y] = *(__attribute__((address_space(3))) bf16x8*)(cur + (kStageFragsA + ks * kTileN + wn * kWbN + y) * kFragBytes + lane * 16);
#pragma unroll
            for (int x = 0; x < kWbM; ++x)
#pragma unroll
                for (int y = 0; y < kWbN; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // Lane l holds rows 4*(l/16) .. +3 of column l%16 of each 16 x 16 block.
    const int r4 = 4 * (lane / 16), col = lane % 16;
#pragma unroll
    for (int x = 0; x < kWbM; ++x) {
        const int64_t bi = bm0 + wm * kWbM + x;
        if (bi >= mb) continue;
#pragma unroll
        for (int y = 0; y < kWbN; ++y) {
            const int64_t bj = bn0 + wn * kWbN + y;
            if (bj >= nb) continue;
            float* out = c + (16 * bi + r4) * n + 16 * bj + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(acc[x][y][i], out + i * n);
        }
    }
}

}  // namespace

hipError_t launch_gemm_frag(const void* fa, const void* fb, float* c, int64_t m, int64_t n, int64_t k,
                            hipStream_t stream) {
    const int64_t tiles_m = (m / 16 + kTileM - 1) / kTileM;
    const int64_t tiles_n = (n / 16 + kTileN - 1) / kTileN;
    if (tiles_m == 0 || tiles_n == 0) return hipSuccess;
    if (tiles_n > 0x7fffffff / kGemmThreads) return hipErrorInvalidValue;
    for (int64_t t0 = 0; t0 < tiles_m; t0 += kMaxGridY) {
        const int64_t ny = tiles_m - t0 < kMaxGridY ? tiles_m - t0 : kMaxGridY;
        hipLaunchKernelGGL(k_gemm_frag, dim3(static_cast<unsigned>(tiles_n), static_cast<unsigned>(ny)),
                           dim3(kGemmThreads), 0, stream, static_cast<const uint8_t*>(fa),
                           static_cast<const uint8_t*>(fb), c, m, n, k, t0);
    }
    return hipGetLastError();
}

}  // namespace swz
