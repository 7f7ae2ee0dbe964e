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
// SWZ_READ_ROWS: whole rows of any width up to 128 columns (kernels_rows.hip).
// A tile is as many whole rows as fit in rows_tile_bytes of LDS, in groups
// of 64 lane-words (a lane-word: 4 bytes of consecutive rows of one column,
// so a group is 256 / E rows): 16 KiB and 256 threads up to 64 columns,
// 32 KiB and 512 threads up to 128.  Its run in each output row may be
// shifted to start on a kRowsLine-byte line of the output; it then also
// loads up to kRowsLine / E rows past its own (at most a quarter of the
// tile's bytes), so the LDS holds rows_lds_bytes.
hipError_t launch_rows(int esz, const ConvertJob& job, hipStream_t stream);
constexpr int kRowsLine = 64;
inline int rows_tile_bytes(int64_t cols) { return cols <= 64 ? 16384 : 32768; }
inline int rows_threads(int64_t cols) { return cols <= 64 ? 256 : 512; }
inline int rows_lds_bytes(int64_t cols) { return rows_tile_bytes(cols) + rows_tile_bytes(cols) / 4; }
inline int64_t rows_halo_rows(int esz) { return kRowsLine / esz; }
inline int64_t rows_tile_rows(int64_t cols, int esz) {
    const int64_t group = 64 * (4 / esz);
    return cols <= 0 || cols > 128 ? 0 : rows_tile_bytes(cols) / (cols * esz) / group * group;
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
