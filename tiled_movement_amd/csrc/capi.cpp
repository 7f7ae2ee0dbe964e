// C ABI of libswz.so: argument checks, parameter choice and launches.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "chooser.h"
#include "launch.h"
#include "swz.h"

#define SWZ_API extern "C" __attribute__((visibility("default")))

namespace {

using swz::KindInfo;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + static_cast<uintptr_t>(bbytes) && pb < pa + static_cast<uintptr_t>(abytes);
}

// Whether n elements of esz bytes make a whole number of 16-byte vectors;
// unsigned, so that a huge n wraps instead of overflowing (16 divides 2^64).
bool pitch16(int64_t n, int32_t esz) { return (static_cast<uint64_t>(n) * static_cast<uint64_t>(esz)) % 16 == 0; }

int ilog2(int64_t v) {
    int r = -1;
    while (v > 0) {
        v >>= 1;
        ++r;
    }
    return r;
}

// Parameters and LDS row pitch of a layout for a kind: the caller's swizzle
// or the chooser's for SWIZZLE and SWIZZLE_DIRECT (the direct fill also needs
// S >= B, so that the swizzle is its own inverse), the pad for PAD.
int resolve_layout(int kind, int32_t layout, const swz_params* p, swz_params* q, int* pad) {
    *q = swz_params{0, 0, 0};
    *pad = 0;
    switch (layout) {
        case SWZ_LAYOUT_SWIZZLE:
        case SWZ_LAYOUT_SWIZZLE_DIRECT:
            if (p) {
                if (!swz::params_ok_for_kind(kind, *p)) return SWZ_EINVAL;
                if (layout == SWZ_LAYOUT_SWIZZLE_DIRECT && p->B > 0 && (p->S < 0 ? -p->S : p->S) < p->B)
                    return SWZ_EINVAL;  // only |S| >= B makes the swizzle its own inverse
                *q = *p;
            } else {
                *q = swz::cached_choice(kind);
            }
            return SWZ_OK;
        case SWZ_LAYOUT_PAD: {
            // A row narrower than one 4-byte LDS write cannot get a pad of
            // its own: the write would straddle the gap.
            KindInfo k;
            if (swz::is_narrow(kind) && swz::kind_info(kind, &k) && k.tc * k.esz < 4) return SWZ_EUNSUPPORTED;
            *pad = swz::pad_elems(kind);
            return SWZ_OK;
        }
        case SWZ_LAYOUT_PLAIN: return SWZ_OK;
        default: return SWZ_EINVAL;
    }
}

// Resolve read kind, layout and parameters into a plan; shared by the calls
// and by swz_plan.  aligned_out: pointers and the output row pitch allow
// 16-byte vectors; aligned_in: so does the input row pitch.  Whole-row
// (narrow) tiles are contiguous stretches of the input, so they need only
// the first.
int make_plan(int op, int64_t rows, int64_t cols, int32_t esz, int32_t layout, int32_t read_kind,
              const swz_params* p, bool aligned_out, bool aligned_in, swz_plan_info* out) {
    if (layout < SWZ_LAYOUT_SWIZZLE || layout > SWZ_LAYOUT_SWIZZLE_DIRECT) return SWZ_EINVAL;
    int kind = read_kind;
    if (op == 0) {
        if (esz != 1 && esz != 2 && esz != 4) return SWZ_EINVAL;
        if (kind == SWZ_READ_AUTO) {
            // whole-row tiles: the swizzled kinds for power-of-two widths of
            // 1 to 64 bytes, flat rows for the other widths up to 128 columns
            // (fp32 from 96 columns on only where the last 32 x 32 tile
            // column would hold at most 19 columns: with fuller tiles the
            // tile kind ran faster, x 96 0.79 against 0.72 of a copy, x 120
            // 0.74 against 0.68, x 127 0.69 against 0.58; x 115 0.51
            // against 0.79)
            const bool pow2 = cols >= 1 && (cols & (cols - 1)) == 0;
            const bool narrow = pow2 && cols * esz <= 64;
            const int lc = ilog2(cols);
            const bool flat_rows = !pow2 && cols >= 1 && cols <= swz::kRowsMaxCols &&
                                   (esz != 4 || cols < 96 || (cols % 32 >= 1 && cols % 32 <= 19));
            // Power-of-two widths whose output rows (or pointers) rule out
            // 16-byte vectors: the swizzled narrow kinds then move elements
            // one by one, and flat rows ran faster for every fp32 width,
            // 2-byte widths of 8 to 32 and bytes x 64 (odd row counts, 64
            // MiB, share of a copy: fp32 x 1 0.59 -> 0.90, x 8 0.49 -> 0.75,
            // x 16 0.48 -> 0.74; 2-byte x 16 0.54 -> 0.72; bytes x 64 0.59
            // -> 0.64; narrower 2-byte and byte widths kept their kinds, at
            // 0.73-1.0)
            const bool unaligned_pow2 =
                narrow && !aligned_out && (esz == 4 || (esz == 2 && cols >= 8) || (esz == 1 && cols == 64));
            // (the flat-row kind has no padded or direct layout: those keep
            // the tile kinds)
            const bool rows_layout = layout == SWZ_LAYOUT_SWIZZLE || layout == SWZ_LAYOUT_PLAIN;
            if ((flat_rows || unaligned_pow2) && rows_layout)
                kind = SWZ_READ_ROWS;
            else if (esz == 4)
                kind = narrow ? SWZ_READ_NARROW1 + lc : SWZ_READ_SCALAR_COL;
            else if (esz == 2)
                kind = narrow        ? SWZ_READ_HNARROW1 + lc
                       : cols <= 64  ? SWZ_READ_B64_TR16
                       : cols <= 128 ? SWZ_READ_B128_8X8
                       : cols <= 256 ? SWZ_READ_B64_TR16
                       : rows % 2 == 0 && (!aligned_out || !aligned_in || swz::partial_line_output(rows, esz))
                           ? SWZ_READ_B64_TR16  // see below
                           : SWZ_READ_B64_4X4;
            // (Above 256 columns, for an even number of rows whose pitches
            // or pointers are off 16 bytes or whose output rows are off the
            // 64-byte lines, the transpose read ran faster: 4096 x 4100 0.81
            // -> 0.87 of a copy, 4100 x 4096 0.69 -> 0.73, 67108 x 500 0.63
            // -> 0.66, 111848 x 300 0.53 -> 0.56; with an odd number of rows
            // the 4x4 reads stay ahead: 5801 x 5801 0.67 against 0.56.)
            else
                kind = narrow ? SWZ_READ_BNARROW1 + lc : SWZ_READ_B64_TR8;
        }
        if (kind == SWZ_READ_MFMA_16X16X32) return SWZ_EINVAL;
        if (kind == SWZ_READ_ROWS) {
            // flat whole rows, swizzled on word offsets (M = 0, B <= S <=
            // 11: a bit of the tile's word offset XORs into a lower one;
            // B <= 10, so the XOR stays inside the 20 or 40 KiB of LDS, whole
            // 4 KiB blocks, that tile and halo take), or plain; no padded or
            // direct layout
            if (cols < 1 || cols > swz::kRowsMaxCols) return SWZ_EINVAL;
            if (layout == SWZ_LAYOUT_PAD || layout == SWZ_LAYOUT_SWIZZLE_DIRECT) return SWZ_EUNSUPPORTED;
            if (p && p->B != 0 && (p->B < 0 || p->B > 10 || p->M != 0 || p->S < p->B || p->S > 11))
                return SWZ_EINVAL;
            swz_params q{0, 0, 0};
            if (layout == SWZ_LAYOUT_SWIZZLE) q = p ? (p->B == 0 ? swz_params{0, 0, 0} : *p) : swz::rows_choice(static_cast<int>(cols));
            std::memset(out, 0, sizeof(*out));
            out->params = q;
            out->read_kind = kind;
            out->tile_rows = static_cast<int32_t>(swz::rows_tile_rows(cols, esz));
            out->tile_cols = static_cast<int32_t>(cols);
            out->layout = layout;
            out->lds_bytes = static_cast<int32_t>((out->tile_rows + swz::rows_halo_rows(esz)) * cols * esz);
            out->vec_bytes = 16;
            out->aligned = 1;  // any pitch: unaligned rows take the same accesses
            out->threads = swz::rows_threads(cols);
            out->interior_tiles = 1;
            return SWZ_OK;
        }
    } else {
        if (esz != 2) return SWZ_EINVAL;
        if (kind != SWZ_READ_AUTO && kind != SWZ_READ_MFMA_16X16X32) return SWZ_EINVAL;
        kind = SWZ_READ_MFMA_16X16X32;
    }
    KindInfo k;
    if (!swz::kind_info(kind, &k)) return SWZ_EINVAL;
    if (k.esz != esz) return SWZ_EINVAL;
    if (swz::is_narrow(kind) && cols != k.tc) return SWZ_EINVAL;  // whole rows per tile
    const bool aligned = aligned_out && (aligned_in || swz::is_narrow(kind));

    swz_params q;
    int pad;
    const int st = resolve_layout(kind, layout, p, &q, &pad);
    if (st != SWZ_OK) return st;
    if (layout == SWZ_LAYOUT_SWIZZLE_DIRECT && !aligned) return SWZ_EUNSUPPORTED;
    std::memset(out, 0, sizeof(*out));
    out->read_kind = kind;
    out->tile_rows = k.tr;
    out->tile_cols = k.tc;
    out->layout = layout;
    out->params = q;
    out->pad_elems = pad;
    out->lds_bytes = k.tr * (k.tc + pad) * k.esz;
    out->vec_bytes = layout == SWZ_LAYOUT_SWIZZLE_DIRECT ? (k.esz == 2 ? 16 : 4) : k.vec;
    out->aligned = aligned ? 1 : 0;
    out->threads = k.nt;
    out->interior_tiles = swz::interior_stack(kind) * swz::interior_stack_cols(kind);
    (void)rows;
    return SWZ_OK;
}

swz::LdsLayout layout_of(const swz_plan_info& pl) {
    return swz::LdsLayout{static_cast<uint32_t>(pl.tile_cols + pl.pad_elems), static_cast<uint32_t>(pl.params.B),
                          static_cast<uint32_t>(pl.params.M), pl.params.S};
}

int hip_status(hipError_t e) { return e == hipSuccess ? SWZ_OK : SWZ_EHIP; }

// The order of a shape with none pinned, from sweeps of every order over
// matrices of 32-512 MiB with sides from 1,024 to 16,384 (bench.py
// --order-shapes).  What decides is the source row pitch:
// - not within 1% of a multiple of 4 KiB: slope 1/32.  Workgroups then walk
//   down the block columns nearly in order, so the output rows are written
//   in long runs, while the reads, a pitch apart, still spread over the
//   memory channels.  Over 745 fp32, 723 16-bit and 471 byte such shapes
//   the mean rate rose from 0.85, 0.87 and 0.84 of a copy of the same bytes
//   to 0.95, 0.96 and 0.90; one shape lost more than 1% (a byte matrix, 2.6%).
// - within 1% of a multiple of 4 KiB: reads a pitch apart fall on few
//   channels in that walk and the diagonal is needed; for fp32 matrices
//   with at most 10,240 rows and a side that is not a power of two, slope
//   1/8 did better still (462 shapes: 0.85 -> 0.91; 11 lost 2-6%; beyond
//   10,240 rows it lost up to 8%).
// Where the output rows are not whole 64-byte pieces (at 2,000 rows and
// more), whole tile columns in turn: the grid that serves those shapes has
// workgroups on one XCD take consecutive blocks, and in this order those
// are the neighbours that share the pieces (fp32, 16-bit and byte matrices
// of 2,000-9,000 rows: 0.45-0.60 of a copy before, 0.63-0.75 after; slope
// 1/32 within 1% of it, the diagonal up to 0.17 behind).  The whole-row
// kinds have one tile column, where every order is the same, and keep the
// diagonal.
int default_order(int kind, int64_t rows, int64_t cols) {
    const int esz = kind == SWZ_READ_SCALAR_COL ? 4
                    : kind == SWZ_READ_B64_4X4 || kind == SWZ_READ_B64_TR16 || kind == SWZ_READ_B128_8X8 ? 2
                    : kind == SWZ_READ_B64_TR8                                                          ? 1
                                                                                                        : 0;
    if (esz == 0) return SWZ_ORDER_DIAGONAL;
    // Output rows off the 64-byte pieces (the XCD-grouped grid): neighbours
    // down a block column share those pieces, so they go in turn, unless the
    // matrix is under 16 tiles wide; then the workgroups in flight would
    // crowd a few output rows, and the shallowest slope spreads them (odd row
    // counts, share of a copy, columns against slope 1/32: bytes x 300, 3
    // tiles, 0.30 against 0.42; 2-byte x 500, 8 tiles, 0.50 against 0.63;
    // bytes x 1000, 8 tiles, 0.50 against 0.59; from 16 tiles columns won or
    // tied: fp32 x 500 0.63 against 0.61, 2-byte x 1000 0.60 against 0.58).
    if (swz::partial_line_output(rows, esz)) {
        const int64_t tile_cols = kind == SWZ_READ_SCALAR_COL ? 32 : esz == 2 && kind != SWZ_READ_B128_8X8 ? 64 : 128;
        return (cols + tile_cols - 1) / tile_cols < 16 ? SWZ_ORDER_SLOPE_32 : SWZ_ORDER_COLUMNS;
    }
    const uint64_t pitch = static_cast<uint64_t>(cols) * static_cast<uint64_t>(esz), r = pitch % 4096;
    const uint64_t off = r < 4096 - r ? r : 4096 - r;  // distance to the nearest multiple of 4 KiB
    if (off * 100 > pitch) return SWZ_ORDER_SLOPE_32;
    const bool pow2 = (rows & (rows - 1)) == 0 && (cols & (cols - 1)) == 0;
    return esz == 4 && !pow2 && rows <= 10240 ? SWZ_ORDER_SLOPE_8 : SWZ_ORDER_DIAGONAL;
}

// Tile orders pinned per conversion shape (swz_set_tile_order,
// swz_tune_tile_order); shapes not listed use their default order.
using ShapeKey = std::tuple<int, int64_t, int64_t, int64_t>;  // read kind, batch, rows, cols
std::mutex g_order_mu;
std::map<ShapeKey, int>& order_table() {
    static std::map<ShapeKey, int> t;
    return t;
}
int pinned_order(int kind, int64_t batch, int64_t rows, int64_t cols) {
    std::lock_guard<std::mutex> lock(g_order_mu);
    const auto it = order_table().find(ShapeKey{kind, batch, rows, cols});
    return it == order_table().end() ? default_order(kind, rows, cols) : it->second;
}

}  // namespace

SWZ_API const char* swz_strerror(int status) {
    switch (status) {
        case SWZ_OK: return "ok";
        case SWZ_EINVAL: return "invalid argument";
        case SWZ_EUNSUPPORTED: return "unsupported request";
        case SWZ_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

SWZ_API int swz_map(const int32_t* d_in, int32_t* d_out, int64_t n, swz_params p, void* stream) {
    if (n < 0) return SWZ_EINVAL;
    const int64_t abs_s = p.S < 0 ? -static_cast<int64_t>(p.S) : p.S;
    if (p.B < 0 || p.M < 0 || static_cast<int64_t>(p.B) + p.M + abs_s > 32) return SWZ_EINVAL;
    if (n == 0) return SWZ_OK;
    if (!d_in || !d_out) return SWZ_EINVAL;
    if (reinterpret_cast<uintptr_t>(d_in) % 4 || reinterpret_cast<uintptr_t>(d_out) % 4) return SWZ_EINVAL;
    int64_t bytes;
    if (!mul_ok(n, 4, &bytes)) return SWZ_EINVAL;
    if (d_in != d_out && overlaps(d_in, bytes, d_out, bytes)) return SWZ_EINVAL;
    return hip_status(swz::launch_map(d_in, d_out, n, p, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_map_batch(const int32_t* d_in, int32_t* d_out, int64_t n, const swz_params* h_params,
                          int32_t n_params, void* stream) {
    if (n < 0 || n_params < 0) return SWZ_EINVAL;
    if (n_params > 0 && !h_params) return SWZ_EINVAL;
    for (int32_t j = 0; j < n_params; ++j) {
        const swz_params& p = h_params[j];
        const int64_t abs_s = p.S < 0 ? -static_cast<int64_t>(p.S) : p.S;
        if (p.B < 0 || p.M < 0 || static_cast<int64_t>(p.B) + p.M + abs_s > 32) return SWZ_EINVAL;
    }
    if (n == 0 || n_params == 0) return SWZ_OK;
    if (!d_in || !d_out) return SWZ_EINVAL;
    if (reinterpret_cast<uintptr_t>(d_in) % 4 || reinterpret_cast<uintptr_t>(d_out) % 4) return SWZ_EINVAL;
    int64_t in_bytes, out_elems, out_bytes;
    if (!mul_ok(n, 4, &in_bytes) || !mul_ok(n, n_params, &out_elems) || !mul_ok(out_elems, 4, &out_bytes))
        return SWZ_EINVAL;
    if (overlaps(d_in, in_bytes, d_out, out_bytes)) return SWZ_EINVAL;
    const auto st = static_cast<hipStream_t>(stream);
    for (int32_t j0 = 0; j0 < n_params; j0 += swz::kMapBatch) {
        const int count = n_params - j0 < swz::kMapBatch ? n_params - j0 : swz::kMapBatch;
        swz::MapParamPack pk{};
        for (int k = 0; k < count; ++k) {
            pk.B[k] = static_cast<uint8_t>(h_params[j0 + k].B);
            pk.M[k] = static_cast<uint8_t>(h_params[j0 + k].M);
            pk.S[k] = static_cast<int8_t>(h_params[j0 + k].S);
        }
        const int rc = hip_status(swz::launch_map_batch(d_in, d_out + static_cast<int64_t>(j0) * n, n, pk, count, st));
        if (rc != SWZ_OK) return rc;
    }
    return SWZ_OK;
}

SWZ_API int swz_plan(int32_t op, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t layout, int32_t read_kind,
                     const swz_params* p_or_null, swz_plan_info* out) {
    if (!out || (op != 0 && op != 1) || rows < 0 || cols < 0) return SWZ_EINVAL;
    if (op == 1 && (rows % 16 || cols % 32)) return SWZ_EINVAL;
    // Pointers are taken as 16-byte aligned; the row pitches decide the rest.
    return make_plan(op, rows, cols, elem_bytes, layout, read_kind, p_or_null,
                     op == 1 || pitch16(rows, elem_bytes), op == 1 || pitch16(cols, elem_bytes), out);
}

SWZ_API int swz_convert_layout(const void* d_src, void* d_dst, int64_t batch, int64_t rows, int64_t cols,
                               int32_t elem_bytes, int32_t layout, int32_t read_kind, const swz_params* p_or_null,
                               void* stream) {
    if (batch < 0 || rows < 0 || cols < 0) return SWZ_EINVAL;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return SWZ_EINVAL;
    int64_t n, n2, bytes;
    if (!mul_ok(batch, rows, &n) || !mul_ok(n, cols, &n2) || !mul_ok(n2, elem_bytes, &bytes)) return SWZ_EINVAL;
    const auto ps = reinterpret_cast<uintptr_t>(d_src), pd = reinterpret_cast<uintptr_t>(d_dst);
    swz_plan_info pl;
    const int st = make_plan(0, rows, cols, elem_bytes, layout, read_kind, p_or_null,
                             ps % 16 == 0 && pd % 16 == 0 && pitch16(rows, elem_bytes), pitch16(cols, elem_bytes), &pl);
    if (st != SWZ_OK) return st;
    if (bytes == 0) return SWZ_OK;
    if (!d_src || !d_dst) return SWZ_EINVAL;
    if (ps % elem_bytes || pd % elem_bytes) return SWZ_EINVAL;
    if (overlaps(d_src, bytes, d_dst, bytes)) return SWZ_EINVAL;
    swz::ConvertJob job{d_src, d_dst, batch, rows, cols, layout_of(pl), pl.aligned != 0,
                        layout == SWZ_LAYOUT_SWIZZLE_DIRECT, pinned_order(pl.read_kind, batch, rows, cols)};
    if (pl.read_kind == SWZ_READ_ROWS)
        return hip_status(swz::launch_rows(elem_bytes, job, static_cast<hipStream_t>(stream)));
    return hip_status(swz::launch_convert(pl.read_kind, job, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_transpose(const void* d_src, void* d_dst, int64_t rows, int64_t cols, int32_t elem_bytes,
                          int32_t layout, int32_t read_kind, const swz_params* p_or_null, void* stream) {
    return swz_convert_layout(d_src, d_dst, 1, rows, cols, elem_bytes, layout, read_kind, p_or_null, stream);
}

SWZ_API int swz_set_tile_order(int64_t batch, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t read_kind,
                               int32_t order) {
    if (batch < 0 || rows < 0 || cols < 0) return SWZ_EINVAL;
    if (order < -1 || order > SWZ_ORDER_SLOPE_32) return SWZ_EINVAL;
    swz_plan_info pl;
    const int st = make_plan(0, rows, cols, elem_bytes, SWZ_LAYOUT_SWIZZLE, read_kind, nullptr,
                             pitch16(rows, elem_bytes), pitch16(cols, elem_bytes), &pl);
    if (st != SWZ_OK) return st;
    std::lock_guard<std::mutex> lock(g_order_mu);
    const ShapeKey key{pl.read_kind, batch, rows, cols};
    if (order < 0)
        order_table().erase(key);
    else
        order_table()[key] = order;
    return SWZ_OK;
}

SWZ_API int swz_get_tile_order(int64_t batch, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t read_kind,
                               int32_t* order) {
    if (!order || batch < 0 || rows < 0 || cols < 0) return SWZ_EINVAL;
    swz_plan_info pl;
    const int st = make_plan(0, rows, cols, elem_bytes, SWZ_LAYOUT_SWIZZLE, read_kind, nullptr,
                             pitch16(rows, elem_bytes), pitch16(cols, elem_bytes), &pl);
    if (st != SWZ_OK) return st;
    *order = pinned_order(pl.read_kind, batch, rows, cols);
    return SWZ_OK;
}

SWZ_API int swz_tune_tile_order(const void* d_src, void* d_dst, int64_t batch, int64_t rows, int64_t cols,
                                int32_t elem_bytes, int32_t layout, int32_t read_kind, const swz_params* p_or_null,
                                int32_t reps, int32_t* chosen, void* stream) {
    if (!chosen || reps < 1 || reps > 1000) return SWZ_EINVAL;
    if (batch < 0 || rows < 0 || cols < 0) return SWZ_EINVAL;
    swz_plan_info pl;
    const auto ps = reinterpret_cast<uintptr_t>(d_src), pd = reinterpret_cast<uintptr_t>(d_dst);
    int st = make_plan(0, rows, cols, elem_bytes, layout, read_kind, p_or_null,
                       ps % 16 == 0 && pd % 16 == 0 && pitch16(rows, elem_bytes), pitch16(cols, elem_bytes), &pl);
    if (st != SWZ_OK) return st;
    int64_t n, n2, bytes;
    if (!mul_ok(batch, rows, &n) || !mul_ok(n, cols, &n2) || !mul_ok(n2, elem_bytes, &bytes)) return SWZ_EINVAL;
    const int dflt = default_order(pl.read_kind, rows, cols);
    if (bytes == 0) {
        *chosen = dflt;
        return SWZ_OK;
    }
    if (!d_src || !d_dst) return SWZ_EINVAL;
    const auto strm = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return SWZ_EHIP;
    }
    // Three rounds over the orders (interleaved, so slow drifts of clock or
    // temperature hit them alike), each one untimed and reps timed calls;
    // an order's time is its best round.
    constexpr int kOrders = SWZ_ORDER_SLOPE_32 + 1, kRounds = 3;
    float t[kOrders];
    for (int o = 0; o < kOrders; ++o) t[o] = -1.0f;
    for (int round = 0; round < kRounds && st == SWZ_OK; ++round) {
        for (int order = 0; order < kOrders && st == SWZ_OK; ++order) {
            st = swz_set_tile_order(batch, rows, cols, elem_bytes, pl.read_kind, order);
            for (int r = 0; r <= reps && st == SWZ_OK; ++r) {
                if (r == 1 && hipEventRecord(e0, strm) != hipSuccess) st = SWZ_EHIP;
                if (st == SWZ_OK)
                    st = swz_convert_layout(d_src, d_dst, batch, rows, cols, elem_bytes, layout, read_kind,
                                            p_or_null, stream);
            }
            float ms = 0.0f;
            if (st == SWZ_OK && (hipEventRecord(e1, strm) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                                 hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
                st = SWZ_EHIP;
            if (st == SWZ_OK && (t[order] < 0.0f || ms < t[order])) t[order] = ms;
        }
    }
    // Another order replaces the default one only when it is at least 3%
    // faster: the timed calls reuse one buffer pair, which the caches hold
    // in part, so small differences need not carry over to other buffers.
    int best = dflt;
    for (int o = 0; o < kOrders; ++o)
        if (o != dflt && t[o] >= 0.0f && t[o] < t[best] && (best != dflt || t[o] < 0.97f * t[best])) best = o;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != SWZ_OK) {
        (void)swz_set_tile_order(batch, rows, cols, elem_bytes, pl.read_kind, -1);
        return st;
    }
    // the last call left the result in d_dst; the pinned order gives the same bits
    *chosen = best;
    return swz_set_tile_order(batch, rows, cols, elem_bytes, pl.read_kind, best);
}

SWZ_API int swz_stage_operand(const void* d_src, void* d_frag, int64_t mn, int64_t k, int32_t elem_bytes,
                              int32_t frag_kind, int32_t layout, const swz_params* p_or_null, void* stream) {
    if (mn < 0 || k < 0 || mn % 16 || k % 32) return SWZ_EINVAL;
    if (elem_bytes != 2 || frag_kind != SWZ_FRAG_MFMA_F32_16X16X32_BF16) return SWZ_EINVAL;
    int64_t n, bytes;
    if (!mul_ok(mn, k, &n) || !mul_ok(n, 2, &bytes)) return SWZ_EINVAL;
    swz_plan_info pl;
    const int st = make_plan(1, mn, k, elem_bytes, layout, SWZ_READ_MFMA_16X16X32, p_or_null, true, true, &pl);
    if (st != SWZ_OK) return st;
    if (bytes == 0) return SWZ_OK;
    if (!d_src || !d_frag) return SWZ_EINVAL;
    if (reinterpret_cast<uintptr_t>(d_src) % 16 || reinterpret_cast<uintptr_t>(d_frag) % 16) return SWZ_EINVAL;
    if (overlaps(d_src, bytes, d_frag, bytes)) return SWZ_EINVAL;
    swz::StageJob job{d_src, d_frag, mn, k, layout_of(pl), layout == SWZ_LAYOUT_SWIZZLE_DIRECT};
    return hip_status(swz::launch_stage(job, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_stage_operands(const void* d_a, void* d_fa, int64_t m, const void* d_bt, void* d_fb, int64_t n,
                               int64_t k, int32_t elem_bytes, int32_t frag_kind, int32_t layout,
                               const swz_params* p_or_null, void* stream) {
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 32) return SWZ_EINVAL;
    if (elem_bytes != 2 || frag_kind != SWZ_FRAG_MFMA_F32_16X16X32_BF16) return SWZ_EINVAL;
    int64_t ea, eb, a_bytes, b_bytes;
    if (!mul_ok(m, k, &ea) || !mul_ok(ea, 2, &a_bytes) || !mul_ok(n, k, &eb) || !mul_ok(eb, 2, &b_bytes))
        return SWZ_EINVAL;
    swz_plan_info pl;
    const int st = make_plan(1, m > n ? m : n, k, elem_bytes, layout, SWZ_READ_MFMA_16X16X32, p_or_null, true, true, &pl);
    if (st != SWZ_OK) return st;
    if (a_bytes == 0 && b_bytes == 0) return SWZ_OK;
    if ((a_bytes && (!d_a || !d_fa)) || (b_bytes && (!d_bt || !d_fb))) return SWZ_EINVAL;
    for (const void* q : {d_a, static_cast<const void*>(d_fa), d_bt, static_cast<const void*>(d_fb)})
        if (reinterpret_cast<uintptr_t>(q) % 16) return SWZ_EINVAL;
    // each fragment buffer is disjoint from both sources and from the other
    // one (the sources are only read and may share memory)
    if (overlaps(d_fa, a_bytes, d_a, a_bytes) || overlaps(d_fa, a_bytes, d_bt, b_bytes) ||
        overlaps(d_fb, b_bytes, d_a, a_bytes) || overlaps(d_fb, b_bytes, d_bt, b_bytes) ||
        overlaps(d_fa, a_bytes, d_fb, b_bytes))
        return SWZ_EINVAL;
    swz::StageJob job{d_a, d_fa, m, k, layout_of(pl), layout == SWZ_LAYOUT_SWIZZLE_DIRECT};
    if (a_bytes == 0) {  // only B^T
        job.src = d_bt;
        job.frag = d_fb;
        job.mn = n;
    } else if (b_bytes > 0) {
        job.src2 = d_bt;
        job.frag2 = d_fb;
        job.mn2 = n;
    }
    return hip_status(swz::launch_stage(job, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_gemm_frag(const void* d_fa, const void* d_fb, float* d_c, int64_t m, int64_t n, int64_t k,
                          int32_t frag_kind, void* stream) {
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 32) return SWZ_EINVAL;
    if (frag_kind != SWZ_FRAG_MFMA_F32_16X16X32_BF16) return SWZ_EINVAL;
    int64_t a_elems, b_elems, c_elems, a_bytes, b_bytes, c_bytes;
    if (!mul_ok(m, k, &a_elems) || !mul_ok(n, k, &b_elems) || !mul_ok(m, n, &c_elems)) return SWZ_EINVAL;
    if (!mul_ok(a_elems, 2, &a_bytes) || !mul_ok(b_elems, 2, &b_bytes) || !mul_ok(c_elems, 4, &c_bytes))
        return SWZ_EINVAL;
    if (m == 0 || n == 0) return SWZ_OK;
    if (!d_c) return SWZ_EINVAL;
    if (k > 0 && (!d_fa || !d_fb)) return SWZ_EINVAL;
    const auto pa = reinterpret_cast<uintptr_t>(d_fa), pb = reinterpret_cast<uintptr_t>(d_fb),
               pc = reinterpret_cast<uintptr_t>(d_c);
    if (pa % 16 || pb % 16 || pc % 16) return SWZ_EINVAL;
    if (k > 0 && (overlaps(d_c, c_bytes, d_fa, a_bytes) || overlaps(d_c, c_bytes, d_fb, b_bytes))) return SWZ_EINVAL;
    return hip_status(swz::launch_gemm_frag(d_fa, d_fb, d_c, m, n, k, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_gemm_ex(const void* d_a, const void* d_bt, void* d_c, int64_t m, int64_t n, int64_t k,
                        int32_t layout, const swz_params* p_or_null, int32_t c_type, void* stream) {
    if (c_type != SWZ_C_F32 && c_type != SWZ_C_BF16) return SWZ_EINVAL;
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 32) return SWZ_EINVAL;
    if (layout == SWZ_LAYOUT_PAD) return SWZ_EUNSUPPORTED;  // the direct fill writes whole rows
    swz_plan_info pl;
    const int st = make_plan(1, m, k, 2, layout == SWZ_LAYOUT_SWIZZLE ? SWZ_LAYOUT_SWIZZLE_DIRECT : layout,
                             SWZ_READ_MFMA_16X16X32, p_or_null, true, true, &pl);
    if (st != SWZ_OK) return st;
    int64_t a_elems, b_elems, c_elems, a_bytes, b_bytes, c_bytes;
    if (!mul_ok(m, k, &a_elems) || !mul_ok(n, k, &b_elems) || !mul_ok(m, n, &c_elems)) return SWZ_EINVAL;
    if (!mul_ok(a_elems, 2, &a_bytes) || !mul_ok(b_elems, 2, &b_bytes) ||
        !mul_ok(c_elems, c_type == SWZ_C_BF16 ? 2 : 4, &c_bytes))
        return SWZ_EINVAL;
    if (m == 0 || n == 0) return SWZ_OK;
    if (!d_c) return SWZ_EINVAL;
    if (k > 0 && (!d_a || !d_bt)) return SWZ_EINVAL;
    const auto pa = reinterpret_cast<uintptr_t>(d_a), pb = reinterpret_cast<uintptr_t>(d_bt),
               pc = reinterpret_cast<uintptr_t>(d_c);
    if (pa % 16 || pb % 16 || pc % 16) return SWZ_EINVAL;
    if (k > 0 && (overlaps(d_c, c_bytes, d_a, a_bytes) || overlaps(d_c, c_bytes, d_bt, b_bytes))) return SWZ_EINVAL;
    return hip_status(swz::launch_gemm_tiles(d_a, d_bt, d_c, m, n, k, layout_of(pl), c_type == SWZ_C_BF16,
                                             static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_gemm(const void* d_a, const void* d_bt, float* d_c, int64_t m, int64_t n, int64_t k, int32_t layout,
                     const swz_params* p_or_null, void* stream) {
    return swz_gemm_ex(d_a, d_bt, d_c, m, n, k, layout, p_or_null, SWZ_C_F32, stream);
}

SWZ_API int swz_fold(const swz_params* p, uint32_t base, uint32_t active, uint32_t* collision,
                     uint32_t* folded_base, int64_t* strides) {
    if (!p || !collision) return SWZ_EINVAL;
    const int64_t abs_s = p->S < 0 ? -static_cast<int64_t>(p->S) : p->S;
    if (p->B < 0 || p->M < 0 || p->B + p->M + abs_s > 32) return SWZ_EINVAL;
    if (base & active) return SWZ_EINVAL;
    const auto B = static_cast<uint32_t>(p->B), M = static_cast<uint32_t>(p->M);
    *collision = active & ~swz::swizzle(active, B, M, p->S);
    if (*collision) return SWZ_EUNSUPPORTED;
    const uint32_t sb = swz::swizzle(base, B, M, p->S);
    if (folded_base) *folded_base = sb;
    if (strides) {
        for (int b = 0; b < 32; ++b) {
            strides[b] = 0;
            if (!((active >> b) & 1u)) continue;
            // Flipping bit b flips the bits of swizzle(1 << b) in swizzle(base):
            // each flip adds its power of two where that bit was clear and
            // subtracts it where it was set.  Without collisions the bits
            // flipped by different active bits never meet, so the moves add.
            const uint32_t v = swz::swizzle(1u << b, B, M, p->S);
            int64_t d = 0;
            for (int t = 0; t < 32; ++t)
                if ((v >> t) & 1u) d += ((sb >> t) & 1u) ? -(int64_t(1) << t) : (int64_t(1) << t);
            strides[b] = d;
        }
    }
    return SWZ_OK;
}

SWZ_API int swz_choose(int32_t elem_bytes, int32_t vec_bytes, int32_t tile_rows, int32_t tile_cols, int32_t read_kind,
                       swz_params* out) {
    if (!out) return SWZ_EINVAL;
    KindInfo k;
    if (!swz::kind_info(read_kind, &k)) return SWZ_EINVAL;
    if (k.esz != elem_bytes || k.vec != vec_bytes || k.tr != tile_rows || k.tc != tile_cols) return SWZ_EUNSUPPORTED;
    *out = swz::cached_choice(read_kind);
    return SWZ_OK;
}

SWZ_API int swz_predict_conflicts(int32_t read_kind, int32_t layout, const swz_params* p_or_null, int64_t* wcyc,
                                  int64_t* rcyc) {
    if (!wcyc || !rcyc) return SWZ_EINVAL;
    KindInfo k;
    if (!swz::kind_info(read_kind, &k)) return SWZ_EINVAL;
    swz_params q;
    int pad;
    const int st = resolve_layout(read_kind, layout, p_or_null, &q, &pad);
    if (st != SWZ_OK) return st;
    swz::predict_tile(read_kind, swz::gfx950_bank_model(), static_cast<uint32_t>(k.tc + pad), q, wcyc, rcyc,
                      layout == SWZ_LAYOUT_SWIZZLE_DIRECT);
    return SWZ_OK;
}

SWZ_API int swz_kernel_accesses(int32_t read_kind, int32_t layout, const swz_params* p_or_null, int32_t is_write,
                                int32_t* addrs, int32_t max_accesses, int32_t* n_accesses, int32_t* width) {
    if (!n_accesses || !width || max_accesses < 0 || (max_accesses > 0 && !addrs)) return SWZ_EINVAL;
    if (is_write != 0 && is_write != 1) return SWZ_EINVAL;
    KindInfo k;
    if (!swz::kind_info(read_kind, &k)) return SWZ_EINVAL;
    swz_params q;
    int pad;
    const int st = resolve_layout(read_kind, layout, p_or_null, &q, &pad);
    if (st != SWZ_OK) return st;
    int w = 0;
    *n_accesses = swz::kernel_accesses(read_kind, static_cast<uint32_t>(k.tc + pad), q,
                                       layout == SWZ_LAYOUT_SWIZZLE_DIRECT, is_write != 0, addrs, max_accesses, &w);
    *width = w;
    return SWZ_OK;
}

SWZ_API int swz_copy(const void* d_src, void* d_dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return SWZ_EINVAL;
    if (bytes == 0) return SWZ_OK;
    if (!d_src || !d_dst) return SWZ_EINVAL;
    if (reinterpret_cast<uintptr_t>(d_src) % 16 || reinterpret_cast<uintptr_t>(d_dst) % 16) return SWZ_EINVAL;
    if (overlaps(d_src, bytes, d_dst, bytes)) return SWZ_EINVAL;
    return hip_status(swz::launch_copy(d_src, d_dst, bytes, static_cast<hipStream_t>(stream)));
}

SWZ_API int swz_bank_model_get(swz_bank_model* out) {
    if (!out) return SWZ_EINVAL;
    const swz::BankModel& m = swz::gfx950_bank_model();
    for (int d = 0; d < 2; ++d) {
        for (int w = 0; w < 3; ++w) {
            out->n_banks[d][w] = m.n_banks[d][w];
            out->bank_bytes[d][w] = m.bank_bytes[d][w];
        }
    }
    std::memcpy(out->phase, m.phase, sizeof(out->phase));
    return SWZ_OK;
}

SWZ_API int swz_lds_probe(const uint32_t* d_addrs, const uint64_t* d_masks, int32_t n_patterns, int32_t width_bytes,
                          int32_t is_write, int32_t iters, int32_t waves, uint64_t* d_cycles, void* stream) {
    if (n_patterns < 0 || (width_bytes != 1 && width_bytes != 2 && width_bytes != 4 && width_bytes != 8 &&
                           width_bytes != 16))
        return SWZ_EINVAL;
    if (iters < 1 || iters > (1 << 20) || waves < 1 || waves > 16 || (is_write != 0 && is_write != 1))
        return SWZ_EINVAL;
    if (n_patterns == 0) return SWZ_OK;
    if (!d_addrs || !d_masks || !d_cycles) return SWZ_EINVAL;
    return hip_status(swz::launch_lds_probe(d_addrs, d_masks, n_patterns, width_bytes, is_write != 0, iters, waves,
                                            d_cycles, static_cast<hipStream_t>(stream)));
}
