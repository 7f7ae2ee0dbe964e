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
// 16 x 16.  The defaults, from a sweep on MI355X at 8192 x 8192 x 4096: a
// 256 x 256 tile of C, eight waves in 4 x 2, each wave 64 x 128 = 4 x 8
// blocks (128 fp32 accumulators per lane, two waves per SIMD); one 32-wide k
// step per stage, two stage buffers (64 KiB of LDS): the loads of stage s+1
// are in flight while stage s is multiplied.  Larger wave tiles spill
// registers (8 x 8 blocks with two k steps per stage ran at half the rate),
// and deeper pipelines (three or four buffers) did not help.  Running half
// of the waves one stage's products behind the other half (the ping-pong
// schedule below, as in the fused GEMM) gained 2-3%.
#include "gemm_epilogue.h"
#include "launch.h"

namespace swz {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Waves along m / n; each wave owns kWbM x kWbN blocks of 16 x 16; one 32-wide
// k step per stage, two stage buffers.
constexpr int kWavesM = 4, kWavesN = 2;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kWbM = 4, kWbN = 8;
constexpr int kTileM = kWavesM * kWbM, kTileN = kWavesN * kWbN;  // blocks per workgroup tile
constexpr int kFragBytes = 64 * 16;                              // one fragment: 64 lanes x 16 bytes
constexpr int kBufBytes = (kTileM + kTileN) * kFragBytes;        // A and B of one stage
static_assert((kTileM + kTileN) % kWaves == 0, "stage loads split over the waves");
constexpr int kPerWave = (kTileM + kTileN) / kWaves;  // direct loads per wave per stage
// The two stage buffers, reused by the epilogue's slices once the last stage
// is done (the slices may need a little more).
constexpr int kSliceBytes = kWaves * epilogue_slice_bytes<kWbN>();
constexpr int kLdsBytes = 2 * kBufBytes > kSliceBytes ? 2 * kBufBytes : kSliceBytes;
static_assert(kLdsBytes <= 160 * 1024, "the stage buffers fit in LDS");

// Workgroup barrier without the memory fence __syncthreads adds: the fence
// would wait for every direct load in flight, including the later stages
// the pipeline keeps going; each wave has already waited for what it needs.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
constexpr int64_t kMaxGridY = 65535;

// Issue this wave's share of stage (k step) s's direct loads into LDS buffer
// buf.  Fragment f < kTileM is A block f; the rest are B blocks.  Blocks past
// the matrix edge load the tile's first block instead (their results are
// never stored).
__device__ __forceinline__ void load_stage(const uint8_t* __restrict__ fa, const uint8_t* __restrict__ fb,
                                           int64_t bm0, int64_t bn0, int64_t mb, int64_t nb, int64_t kb, int64_t s,
                                           lds_u8* buf, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
        const int f = wave * kPerWave + q;
        const bool is_a = f < kTileM;
        const int blk = is_a ? f : f - kTileM;
        const int64_t b0 = is_a ? bm0 : bn0, lim = is_a ? mb : nb;
        const int64_t row = b0 + blk < lim ? b0 + blk : b0;
        const uint8_t* src = (is_a ? fa : fb) + (row * kb + s) * kFragBytes + lane * 16;
        __builtin_amdgcn_global_load_lds(src, buf + f * kFragBytes, 16, 0, 0);
    }
}

__global__ __launch_bounds__(kGemmThreads) void k_gemm_frag(const uint8_t* __restrict__ fa,
                                                             const uint8_t* __restrict__ fb, float* __restrict__ c,
                                                             int64_t m, int64_t n, int64_t k, int64_t tile_row0) {
    __shared__ bf16x8 lds_v[kLdsBytes / 16];
    lds_u8* lds = (lds_u8*)(reinterpret_cast<uint8_t*>(lds_v));
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
    const int lane = threadIdx.x % 64;
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int64_t mb = m / 16, nb = n / 16, kb = k / 32;
    const int64_t ty = blockIdx.y, tx = blockIdx.x;
    const int64_t bm0 = (tile_row0 + ty) * kTileM, bn0 = tx * kTileN;
    const int64_t stages = kb;  // one k step per stage

    f32x4 acc[kWbM][kWbN];
#pragma unroll
    for (int x = 0; x < kWbM; ++x)
#pragma unroll
        for (int y = 0; y < kWbN; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Prologue: stage 0 in flight (k = 0 issues nothing: C = 0).
    if (stages > 0) load_stage(fa, fb, bm0, bn0, mb, nb, kb, 0, lds, wave, lane);

    // Ping-pong schedule.  Waves 0-3 and 4-7 share the SIMDs pairwise.  The
    // second half holds each stage's fragments over the next barrier and
    // multiplies them while reading the next stage's, so one wave of each
    // SIMD feeds the matrix unit while the other waits for LDS.  The k steps
    // still accumulate in increasing order.
    const bool lag = wave >= kWaves / 2;
    // Stage s has landed once this wave's loads are done; the barrier then
    // also says every wave is done with stage s - 1, whose buffer the next
    // loads reuse.
    auto begin = [&](int64_t s) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // held fragments have arrived
        stage_barrier();
        if (s + 1 < stages) load_stage(fa, fb, bm0, bn0, mb, nb, kb, s + 1, lds + ((s + 1) % 2) * kBufBytes, wave, lane);
        return lds + (s % 2) * kBufBytes;
    };
    auto frag_a = [&](lds_u8* cur, int x) {
        return *(__attribute__((address_space(3))) bf16x8*)(cur + (wm * kWbM + x) * kFragBytes + lane * 16);
    };
    auto frag_b = [&](lds_u8* cur, int y) {
        return *(__attribute__((address_space(3))) bf16x8*)(cur + (kTileM + wn * kWbN + y) * kFragBytes + lane * 16);
    };
    if (!lag) {
        for (int64_t s = 0; s < stages; ++s) {
            lds_u8* cur = begin(s);
            bf16x8 a[kWbM], b[kWbN];
#pragma unroll
            for (int x = 0; x < kWbM; ++x) a[x] = frag_a(cur, x);
#pragma unroll
            for (int y = 0; y < kWbN; ++y) b[y] = frag_b(cur, y);
#pragma unroll
            for (int x = 0; x < kWbM; ++x)
#pragma unroll
                for (int y = 0; y < kWbN; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[x], b[y], acc[x][y], 0, 0, 0);
        }
    } else {
        bf16x8 ha[kWbM], hb[kWbN];  // the previous stage's fragments, held over the barrier
        for (int64_t s = 0; s < stages; ++s) {
            lds_u8* cur = begin(s);
            bf16x8 na[kWbM];
#pragma unroll
            for (int x = 0; x < kWbM; ++x) na[x] = frag_a(cur, x);
            if (s > 0) {
#pragma unroll
                for (int y = 0; y < kWbN; ++y) {
#pragma unroll
                    for (int x = 0; x < kWbM; ++x)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[x], hb[y], acc[x][y], 0, 0, 0);
                    hb[y] = frag_b(cur, y);
                }
            } else {
#pragma unroll
                for (int y = 0; y < kWbN; ++y) hb[y] = frag_b(cur, y);
            }
#pragma unroll
            for (int x = 0; x < kWbM; ++x) ha[x] = na[x];
        }
        if (stages > 0) {
#pragma unroll
            for (int x = 0; x < kWbM; ++x)
#pragma unroll
                for (int y = 0; y < kWbN; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[x], hb[y], acc[x][y], 0, 0, 0);
        }
    }

    // Epilogue: through each wave's own LDS slice of the (now idle) stage
    // buffers, once every wave is done reading the last stage.
    stage_barrier();
    store_c_blocks<kWbM, kWbN>(acc, (lds_f32*)(lds + wave * epilogue_slice_bytes<kWbN>()), c, n, bm0 + wm * kWbM,
                               bn0 + wn * kWbN, mb, nb, lane);
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
