// Kernel launchers (defined in the .hip files, called by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swz_common.h"

namespace swz {

struct ConvertJob {
    const void* src;
    void* dst;
    int64_t batch, rows, cols;
    LdsLayout layout;
    bool aligned;  // 16-byte vector path allowed (pointers and pitches)
    bool direct;   // direct HBM -> LDS fill (needs aligned and an unpadded layout)
    int order;     // tile order, enum swz_tile_order
};

struct StageJob {
    const void* src;
    void* frag;
    int64_t mn, k;
    LdsLayout layout;
    bool direct;  // direct HBM -> LDS fill
    // A second operand staged by the same launch (src2 == nullptr: none):
    // src2 [mn2][k] into frag2, same k, layout and fill.
    const void* src2 = nullptr;
    void* frag2 = nullptr;
    int64_t mn2 = 0;
};

hipError_t launch_convert(int kind, const ConvertJob& job, hipStream_t stream);
// SWZ_READ_ROWS: whole rows of any width up to 64 columns (kernels_rows.hip).
// A tile is as many whole rows as fit in kRowsTileBytes of LDS, in groups
// of 64 lane-words (a lane-word: 4 bytes of consecutive rows of one column).
// Its run in each output row is shifted to start on a kRowsLine-byte line
// of the output, so it also loads up to kRowsLine / E rows past its own:
// the LDS holds kRowsLdsBytes.
hipError_t launch_rows(int esz, const ConvertJob& job, hipStream_t stream);
constexpr int kRowsTileBytes = 16384;
constexpr int kRowsLine = 64;
// The halo: at most kRowsLine / E rows of at most 64 E bytes.
constexpr int kRowsLdsBytes = kRowsTileBytes + kRowsLine * 64;
inline int64_t rows_halo_rows(int esz) { return kRowsLine / esz; }
inline int64_t rows_tile_rows(int64_t cols, int esz) {
    const int64_t group = 64 * (4 / esz);
    return cols <= 0 || cols * esz > kRowsTileBytes ? 0 : kRowsTileBytes / (cols * esz) / group * group;
}
hipError_t launch_stage(const StageJob& job, hipStream_t stream);
hipError_t launch_gemm_frag(const void* fa, const void* fb, float* c, int64_t m, int64_t n, int64_t k,
                            hipStream_t stream);
hipError_t launch_gemm_tiles(const void* a, const void* bt, void* c, int64_t m, int64_t n, int64_t k,
                             const LdsLayout& layout, bool bf16c, hipStream_t stream);
hipError_t launch_map(const int32_t* in, int32_t* out, int64_t n, swz_params p, hipStream_t stream);

// Up to kMapBatch triples of one batched-map launch, passed by value.
constexpr int kMapBatch = 128;
struct MapParamPack {
    uint8_t B[kMapBatch], M[kMapBatch];
    int8_t S[kMapBatch];
};
hipError_t launch_map_batch(const int32_t* in, int32_t* out, int64_t n, const MapParamPack& pk, int count,
                            hipStream_t stream);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);
hipError_t launch_lds_probe(const uint32_t* addrs, const uint64_t* masks, int n_patterns, int width, bool write,
                            int iters, int waves, uint64_t* cycles, hipStream_t stream);

}  // namespace swz
