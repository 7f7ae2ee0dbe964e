/*
 * swz.h -- swizzled on-chip tile movement for AMD gfx950 (MI355X).
 *
 * C ABI of libswz.so.  Plain pointers and sizes only.  Every call that moves
 * data is asynchronous on the caller's HIP stream (a hipStream_t passed as
 * void*; NULL is the default stream), except swz_tune_tile_order, which
 * times conversions on it and waits for them.  Device buffers belong to the caller;
 * the library allocates no device memory and keeps no pointer after a call
 * returns.  Errors are negative return codes, detected on the host before
 * any launch; no call aborts or throws.  All calls are thread-safe.
 *
 * Calls: the swizzle map (swz_map, swz_map_batch); transposes and batched layout
 * conversions of 1-, 2- and 4-byte elements through swizzled, padded or
 * plain LDS tiles (swz_transpose, swz_convert_layout), with a per-shape
 * tile order (swz_set_tile_order, swz_get_tile_order, swz_tune_tile_order);
 * GEMM operand staging
 * into matrix-instruction fragments (swz_stage_operand, and both operands of
 * one GEMM at once: swz_stage_operands) and their consumer
 * (swz_gemm_frag); the GEMM that stages its own operands through swizzled
 * tiles (swz_gemm, swz_gemm_ex for a bf16 result); host-only planning, bank-conflict prediction and layout
 * algebra (swz_choose, swz_plan, swz_predict_conflicts, swz_kernel_accesses,
 * swz_bank_model_get, swz_fold); and two diagnostics (swz_copy,
 * swz_lds_probe).
 *
 * The method follows four pages on CuTe's swizzle:
 *   "NVIDIA CuTe Swizzle", "CuTe Swizzle 学习手册", "cutlass 入门",
 *   "CUDA 013 - Swizzle 的工作原理".
 */
#ifndef SWZ_H
#define SWZ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Swizzle<B,M,S> on element offsets: the B-bit field at bit M+S is XORed
 * into the B-bit field at bit M ("CuTe Swizzle 学习手册", section on the
 * swizzle formula; "CUDA 013 - Swizzle 的工作原理", section 计算公式, where
 * the same triple is written (base, bits, shift) = (M, B, S)).  M counts
 * elements: 2^M consecutive elements stay together.  A negative S moves the
 * field the other way ("NVIDIA CuTe Swizzle", the SShift comment: a negative
 * shift moves the mask to the left): the B-bit field at bit M is XORed into
 * the field at bit M + |S|. */
typedef struct swz_params {
    int32_t B;
    int32_t M;
    int32_t S;
} swz_params;

enum swz_status {
    SWZ_OK = 0,
    SWZ_EINVAL = -1,       /* bad argument: size, pointer, alignment, overlap, parameters */
    SWZ_EUNSUPPORTED = -2, /* valid request this build does not handle */
    SWZ_EHIP = -3          /* the HIP runtime reported an error at launch */
};

/* Layout of a tile in LDS.  PAD and PLAIN are the ablations: PAD adds one
 * LDS store's width to each row: one element where the tile is staged an
 * element at a time (4-byte elements), else one vector (16 bytes for the
 * 2-byte tile kinds, 8 for the 8-bit one, 4 for the narrow-row kinds of
 * smaller elements) ("CUDA 013 - Swizzle 的工作原理", section 如何避免 Bank
 * Conflict, the 32x33 array); SWZ_EUNSUPPORTED for narrow rows under 4
 * bytes (HNARROW1, BNARROW1, BNARROW2), whose 4-byte stores span rows.
 * PLAIN is the row-major tile with no remapping.
 * SWIZZLE_DIRECT is the SWIZZLE layout filled without a trip through
 * registers: the tile moves from HBM straight into LDS (the gfx950 direct
 * load, the role cp.async plays in "NVIDIA CuTe Swizzle" and "CuTe Swizzle
 * 学习手册", usage step 2).  Such a load writes each lane's bytes at
 * consecutive LDS addresses, so the swizzle is applied on the HBM side
 * instead: the lane that fills LDS slot p fetches tile element swizzle(p),
 * which places every element exactly where SWIZZLE puts it (the swizzle is
 * its own inverse when |S| >= B).  It needs |S| >= B (or B = 0, plain rows), and
 * 16-byte aligned pointers and row pitches (SWZ_EUNSUPPORTED otherwise; for
 * the narrow-row kinds (NARROW, HNARROW, BNARROW), whose tiles are
 * contiguous stretches of the input, only the output row pitch counts). */
enum swz_layout {
    SWZ_LAYOUT_SWIZZLE = 0,
    SWZ_LAYOUT_PAD = 1,
    SWZ_LAYOUT_PLAIN = 2,
    SWZ_LAYOUT_SWIZZLE_DIRECT = 3
};

/* How a staged tile is read back from LDS.
 *  SCALAR_COL : 4-byte elements, 32x32 tile, each lane reads one element
 *               of a column (two columns per 64-lane wave).
 *  B64_4X4    : 2-byte elements, 64x64 tile, each lane reads 8-byte row
 *               pieces of 8 rows and transposes 4x4 blocks in registers.
 *  B128_8X8   : 2-byte elements, 64x128 tile, each lane reads 16-byte row
 *               pieces of 8 rows and transposes an 8x8 block in registers.
 *  MFMA_16X16X32 : operand staging; see swz_stage_operand.
 *  B64_TR16   : 2-byte elements, 64x64 tile, read with the gfx950 LDS
 *               transpose read (ds_read_b64_tr_b16, the role ldmatrix .trans
 *               plays in "NVIDIA CuTe Swizzle"): each 16-lane group
 *               addresses 8-byte row pieces and every lane receives four
 *               consecutive rows of one column, so two reads give a lane one
 *               16-byte output piece with no register shuffles.
 *  B64_TR8    : 1-byte elements, 128x128 tile, read with the gfx950 8-bit
 *               transpose read (ds_read_b64_tr_b8): each lane receives eight
 *               consecutive rows of one column per read.  The 1-byte case of
 *               "CUDA 013 - Swizzle 的工作原理", usage example 2 (char rows
 *               with the low bits kept together), here with 8-byte runs.
 *  NARROW1 .. NARROW16 : 4-byte elements in matrices of exactly 1, 2, 4, 8
 *               or 16 columns.  Each tile is 4096 bytes of whole rows
 *               (1024/cols rows), contiguous in the source, and its
 *               transpose is cols output runs of 4096/cols bytes.  A row is
 *               narrower than a bank row, so the swizzle acts on the flat
 *               offset and its source bits come from rows above the ones
 *               that form one 32-element line: it spans several rows
 *               ("CUDA 013 - Swizzle 的工作原理", usage example 4).  Reads as
 *               SCALAR_COL: each lane reads four rows of one column.
 *  HNARROW1 .. HNARROW32 : the same for 2-byte elements in matrices of 1,
 *               2, 4, 8, 16 or 32 columns, staged as 4-byte LDS writes (so
 *               M >= 1).  2 to 16 columns: 4096-byte tiles of 2048/cols
 *               rows, each lane reading eight rows of one column with 2-byte
 *               loads into 16 bytes of one output row.  1 and 32 columns:
 *               each lane reads 4-byte words (eight rows of two columns, or
 *               of the one column) and splits them in registers; tiles of
 *               2048 x 1 and 128 x 32.
 *  BNARROW1 .. BNARROW64 : the same for 1-byte elements in matrices of 1 to
 *               64 columns (powers of two), 4-byte LDS writes (M >= 2):
 *               each lane reads 4-byte words of 16 rows and up to 4 columns
 *               and transposes them in registers into up to four 16-byte
 *               output pieces; tiles of 1 KiB per column up to 4 columns,
 *               8 KiB at 8 and 16 KiB above (64, 128 and 256 lanes).
 *  ROWS       : rows of any width up to 128 columns (any element size):
 *               tiles of as many whole rows as fit in 16 KiB (up to 64
 *               columns, 256 threads) or 32 KiB (65 to 128 columns, 512
 *               threads), at least 64 lane-words' worth (256 / esz rows),
 *               copied flat into LDS, each lane gathering 4 bytes of
 *               consecutive rows of one column, each wave storing 256
 *               contiguous bytes of an output row.  Lanes of a read are cols
 *               words apart: odd widths read conflict-free as they are, even
 *               widths through a swizzle of word offsets, Swizzle<B,0,S> with
 *               B <= 10 and B <= S <= 11 (the chooser's per-width pick unless
 *               given).  Layouts SWIZZLE and PLAIN only.  Where output rows
 *               are not whole 64-byte lines and a tile's run in an output row
 *               is at most 2 KiB, the runs are shifted to start on line
 *               boundaries (the tiles then also read up to 64 / esz rows
 *               past their own).
 *  AUTO       : ROWS for the widths up to 128 that are not powers of two
 *               (4-byte elements from 96 columns on only where cols % 32 is
 *               1 to 19), and for the power-of-two widths below whose output
 *               rows or pointers are not 16-byte aligned (4-byte elements,
 *               2-byte of 8 to 32 columns, 1-byte of 64: the narrow kinds
 *               would move them element by element), in the SWIZZLE and
 *               PLAIN layouts (PAD and SWIZZLE_DIRECT keep the kinds below);
 *               otherwise 4-byte ->
 *               NARROW<cols> when cols is 1,
 *               2, 4, 8 or 16, else SCALAR_COL; 2-byte -> HNARROW<cols> when
 *               cols is a power of two up to 32, else B64_TR16 when
 *               cols <= 64, B128_8X8 when cols <= 128, B64_TR16 when
 *               cols <= 256 and B64_4X4 above (the faster of the two 64x64
 *               kinds at those widths), except B64_TR16 above 256 columns
 *               for an even number of rows whose pitches or pointers are off
 *               16 bytes or whose output rows are off the 64-byte lines;
 *               1-byte -> BNARROW<cols> when cols is
 *               a power of two up to 64, else B64_TR8. */
/* The read kind is an argument of its own (read_kind, just before
 * p_or_null, in swz_transpose, swz_convert_layout, swz_tune_tile_order and
 * the tile-order calls), and it names a kernel, not a class of read.  The
 * problem statement fixes only what moves (a row-major tile read back along
 * columns, or in the matrix-operand pattern); how a column is read back is
 * the kernel's choice, and on gfx950 there are several for one element size
 * (8-byte reads with a 4x4 register transpose, the 16-bit transpose read, a
 * 16-byte 8x8 form, whole-row tiles for narrow matrices), each with its own
 * lane map and so its own conflict-free swizzle.  A single "vector column"
 * value could not say which, so that value became these kinds, AUTO picks
 * one from the element size and width exactly as a caller without the
 * argument would get, and the operand-fragment kind moved to 3.  Callers
 * pass SWZ_READ_AUTO for the behaviour of a call without the argument. */
enum swz_read_kind {
    SWZ_READ_AUTO = -1,
    SWZ_READ_SCALAR_COL = 0,
    SWZ_READ_B64_4X4 = 1,
    SWZ_READ_B128_8X8 = 2,
    SWZ_READ_MFMA_16X16X32 = 3,
    SWZ_READ_B64_TR16 = 4,
    SWZ_READ_B64_TR8 = 5,
    SWZ_READ_NARROW1 = 6,
    SWZ_READ_NARROW2 = 7,
    SWZ_READ_NARROW4 = 8,
    SWZ_READ_NARROW8 = 9,
    SWZ_READ_NARROW16 = 10,
    SWZ_READ_HNARROW1 = 11,
    SWZ_READ_HNARROW2 = 12,
    SWZ_READ_HNARROW4 = 13,
    SWZ_READ_HNARROW8 = 14,
    SWZ_READ_HNARROW16 = 15,
    SWZ_READ_HNARROW32 = 16,
    SWZ_READ_BNARROW1 = 17,
    SWZ_READ_BNARROW2 = 18,
    SWZ_READ_BNARROW4 = 19,
    SWZ_READ_BNARROW8 = 20,
    SWZ_READ_BNARROW16 = 21,
    SWZ_READ_BNARROW32 = 22,
    SWZ_READ_BNARROW64 = 23,
    SWZ_READ_ROWS = 24
};

enum swz_frag_kind { SWZ_FRAG_MFMA_F32_16X16X32_BF16 = 0 };

/* What a call will do: tile shape, read kind, LDS layout and parameters. */
typedef struct swz_plan_info {
    int32_t read_kind;   /* resolved read kind */
    int32_t tile_rows;   /* source rows per tile */
    int32_t tile_cols;   /* source columns per tile */
    int32_t layout;      /* as requested */
    swz_params params;   /* swizzle actually used (B = 0 for PAD / PLAIN) */
    int32_t pad_elems;   /* extra elements per LDS row (PAD only) */
    int32_t lds_bytes;   /* LDS bytes one tile occupies */
    int32_t vec_bytes;   /* width of the LDS stores of the staging pass (the
                            direct fill: bytes each lane's load writes) */
    int32_t aligned;     /* 1 if the 16-byte vector path is used */
    int32_t threads;     /* threads per tile */
    int32_t interior_tiles; /* whole tiles per workgroup of the whole-tile
                            launch (threads x interior_tiles threads); a
                            tile on a ragged edge takes a workgroup alone */
} swz_plan_info;

/* out[i] = Swizzle<B,M,S>(in[i]) for i < n, on the 32-bit bit patterns
 * ("CuTe Swizzle 学习手册", swizzle formula; "CUDA 013 - Swizzle 的工作原理",
 * section 计算公式).
 *   d_in, d_out : device int32 arrays of n elements; may be the same
 *                 pointer (in place) but must not otherwise overlap.
 *   p           : B, M >= 0, any S, and B + M + |S| <= 32; B = 0 is the
 *                 identity (S = 0 with B > 0 clears the field, computed as
 *                 written).
 * Errors: SWZ_EINVAL for n < 0, NULL with n > 0, partial overlap, or
 * parameters out of range. */
int swz_map(const int32_t* d_in, int32_t* d_out, int64_t n, swz_params p, void* stream);

/* out[j][i] = Swizzle<B_j,M_j,S_j>(in[i]) for j < n_params, i < n: one
 * offset range under many triples, one launch per 128 triples (the same
 * formula as swz_map, whose single-triple calls are launch-bound at small
 * n).
 *   d_in     : device int32 array of n elements.
 *   d_out    : device int32 array [n_params][n]; must not overlap d_in.
 *   h_params : host array of n_params triples, each in swz_map's range;
 *              read during the call only.
 * Errors: SWZ_EINVAL for n < 0, n_params < 0, NULL with work to do,
 * misalignment, overlap or any triple out of range (then nothing is
 * launched); SWZ_EHIP if a launch fails (earlier chunks may have run). */
int swz_map_batch(const int32_t* d_in, int32_t* d_out, int64_t n, const swz_params* h_params, int32_t n_params,
                  void* stream);

/* dst = transpose of src: src is [rows][cols] row-major, dst is
 * [cols][rows] row-major (the column-major image of src), bit-exact.  Tiles
 * are loaded with coalesced row reads into LDS in the requested layout, read
 * back along columns, and written out with coalesced row writes
 * ("CuTe Swizzle 学习手册", typical scenario: column access of a row-major
 * tile; "CUDA 013 - Swizzle 的工作原理", sections 如何避免 Bank Conflict and
 * Swizzle 技术).  Exactly swz_convert_layout with batch = 1.
 *   elem_bytes : 1, 2 or 4.
 *   layout     : enum swz_layout.
 *   read_kind  : enum swz_read_kind (AUTO picks by element size and width).
 *   p_or_null  : swizzle to use with SWZ_LAYOUT_SWIZZLE(_DIRECT), or NULL to
 *                let swz_choose pick; ignored for PAD and PLAIN.
 * Any rows, cols >= 0 are accepted (partial edge tiles are handled); 0 is a
 * no-op.  src and dst must not overlap; they must be aligned to elem_bytes.
 * Errors: SWZ_EINVAL (sizes, NULL, overlap, misalignment, a read kind that
 * does not fit elem_bytes, parameters that split a vector or move bits
 * outside the tile, S = 0 with B > 0 (not one-to-one), |S| < B with
 * SWZ_LAYOUT_SWIZZLE_DIRECT, a narrow-row kind whose width differs from
 * cols); negative S is accepted; SWZ_EUNSUPPORTED for
 * SWZ_LAYOUT_SWIZZLE_DIRECT when a pointer or a row pitch (cols * elem_bytes
 * or rows * elem_bytes; only the latter for the narrow-row kinds) is not a
 * multiple of 16 bytes, and for SWZ_LAYOUT_PAD with a narrow-row kind whose
 * rows are narrower than 4 bytes (a padded row needs whole 4-byte writes). */
int swz_transpose(const void* d_src, void* d_dst, int64_t rows, int64_t cols, int32_t elem_bytes,
                  int32_t layout, int32_t read_kind, const swz_params* p_or_null, void* stream);

/* Batched layout conversion src[batch][rows][cols] -> dst[batch][cols][rows],
 * each batch entry transposed as in swz_transpose; same arguments and errors. */
int swz_convert_layout(const void* d_src, void* d_dst, int64_t batch, int64_t rows, int64_t cols,
                       int32_t elem_bytes, int32_t layout, int32_t read_kind,
                       const swz_params* p_or_null, void* stream);

/* Order in which the workgroups of a transpose / conversion visit the tiles
 * (of the stacked blocks of tiles where a launch stacks them): workgroups
 * with consecutive numbers q take consecutive tile rows tr, each with the
 * tile column below.  Which order the HBM system serves fastest depends on
 * the matrix shape, by up to 25% at some shapes; no order is best at all of
 * them.  All orders give the same bits.
 *
 * Shapes with no pinned order (swz_set_tile_order) take a default.  With
 * at least 2,000 rows whose output rows (rows * elem_bytes) are not whole
 * 64-byte pieces: SWZ_ORDER_COLUMNS for matrices at least 16 tiles wide,
 * SWZ_ORDER_SLOPE_32 for narrower ones.  Otherwise it is set by the source
 * row pitch (cols * elem_bytes): SWZ_ORDER_SLOPE_32 when the pitch is not
 * within 1% of a multiple of 4 KiB; otherwise the diagonal, or
 * SWZ_ORDER_SLOPE_8 for fp32 matrices with at most 10,240 rows and a side
 * that is not a power of two.  The whole-row (narrow) kinds take the
 * diagonal.  (Measured over 1,273 fp32, 1,009 16-bit and 597 byte shapes
 * of 32 to 512 MiB against a copy of the same bytes; swz_get_tile_order
 * reads a shape's order.) */
enum swz_tile_order {
    SWZ_ORDER_DIAGONAL = 0,       /* tile row tr, tile column (q + tr) mod tiles */
    SWZ_ORDER_HALF_DIAGONAL = 1,  /* tile column (q + tr / 2) mod tiles */
    SWZ_ORDER_COLUMNS = 2,        /* tile column q: every tile row of one tile column in turn */
    SWZ_ORDER_STEEP_DIAGONAL = 3, /* tile column (q + 3 tr) mod tiles */
    SWZ_ORDER_SLOPE_8 = 4,        /* tile column (q + tr / 8) mod tiles */
    SWZ_ORDER_SLOPE_16 = 5,       /* tile column (q + tr / 16) mod tiles */
    SWZ_ORDER_SLOPE_32 = 6        /* tile column (q + tr / 32) mod tiles */
};

/* Pin the tile order of later swz_transpose / swz_convert_layout calls of
 * this shape (batch, rows, cols, elem_bytes, read kind after AUTO is
 * resolved), in every layout; order = -1 removes the entry (back to the
 * shape's default order).  AUTO is resolved here as swz_plan does, for
 * 16-byte aligned pointers; a call whose pointers are not resolves AUTO
 * with them and may land on another kind, whose own entry then applies
 * (swz_tune_tile_order resolves with its buffers' pointers).  Host only;
 * the table is shared by all threads and devices of the process.
 * Errors: SWZ_EINVAL for negative sizes, an order outside -1..6, or an
 * element size / read kind that swz_convert_layout would refuse. */
int swz_set_tile_order(int64_t batch, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t read_kind,
                       int32_t order);

/* The tile order later conversions of this shape will use (the pinned one,
 * or the shape's default), in *order.  Host only.
 * Errors: SWZ_EINVAL for NULL order or negative sizes; as
 * swz_set_tile_order for the element size and read kind. */
int swz_get_tile_order(int64_t batch, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t read_kind,
                       int32_t* order);

/* Time every tile order on this conversion and pin the fastest: three
 * interleaved rounds over the orders, each one untimed and `reps` timed
 * swz_convert_layout calls with these arguments on the caller's buffers and
 * stream, timed with HIP events; an order counts its best round, and
 * replaces the shape's default order only when at least 3% faster (the
 * calls reuse one buffer pair, which the caches partly hold).  Synchronizes the stream;
 * allocates no device memory.  d_dst ends up holding the conversion of
 * d_src (every order writes the same bits).
 *   reps   : 1..1000.
 *   chosen : receives the pinned order (enum swz_tile_order).
 * Errors: those of swz_convert_layout (then no order is pinned for the
 * shape); SWZ_EINVAL for NULL chosen or reps out of range; SWZ_EHIP if an
 * event call fails. */
int swz_tune_tile_order(const void* d_src, void* d_dst, int64_t batch, int64_t rows, int64_t cols,
                        int32_t elem_bytes, int32_t layout, int32_t read_kind, const swz_params* p_or_null,
                        int32_t reps, int32_t* chosen, void* stream);

/* GEMM operand staging without compute.  d_src is a K-contiguous operand
 * [mn][k] (A row-major, or B column-major, which is B^T row-major), 16-bit
 * elements.  Tiles of 64 x 64 are loaded coalesced into LDS in the requested
 * layout and read back in the operand-register pattern of the 16x16x32
 * 16-bit matrix instruction: lane l holds row l%16 of a 16-row block and
 * k = 8*(l/16) .. +7 of a 32-wide k step.  Each 64-lane fragment is written
 * in lane order:
 *   d_frag[i][j][l][e] = src[16*i + l%16][32*j + 8*(l/16) + e],
 *   i < mn/16, j < k/32, l < 64, e < 8  (same byte count as src).
 * The pages' version of this step is the ldmatrix / WGMMA read of a swizzled
 * tile ("NVIDIA CuTe Swizzle", on cp.async and ldmatrix; "CuTe Swizzle
 * 学习手册", usage steps 3 and 5).
 *   elem_bytes must be 2; frag_kind must be SWZ_FRAG_MFMA_F32_16X16X32_BF16.
 *   mn must be a multiple of 16 and k of 32 (partial 64x64 tiles are fine).
 *   d_src and d_frag must be 16-byte aligned and must not overlap.
 * Errors: SWZ_EINVAL otherwise. */
int swz_stage_operand(const void* d_src, void* d_frag, int64_t mn, int64_t k, int32_t elem_bytes,
                      int32_t frag_kind, int32_t layout, const swz_params* p_or_null, void* stream);

/* Both operands of one GEMM C = A * B^T staged by one launch: A [m][k]
 * row-major into d_fa ([m/16][k/32][64][8]) and B^T [n][k] (B column-major)
 * into d_fb ([n/16][k/32][64][8]), each exactly as swz_stage_operand stages
 * it (the same tiles, layout, parameters and fragments).  One launch instead
 * of two saves one launch's start-up and drain, about 5% of two 64 MiB
 * stagings.  The same operand-read step of the pages as swz_stage_operand.
 *   m and n multiples of 16, k of 32 (m or n may be 0: the other operand
 *   alone); elem_bytes 2; frag_kind SWZ_FRAG_MFMA_F32_16X16X32_BF16.
 *   The four pointers 16-byte aligned; each fragment buffer disjoint from
 *   both sources and from the other fragment buffer (the sources are only
 *   read and may overlap each other).
 * Errors: SWZ_EINVAL otherwise, and as swz_stage_operand for the layout and
 * parameters. */
int swz_stage_operands(const void* d_a, void* d_fa, int64_t m, const void* d_bt, void* d_fb, int64_t n, int64_t k,
                       int32_t elem_bytes, int32_t frag_kind, int32_t layout, const swz_params* p_or_null,
                       void* stream);

/* Consumer of staged fragments: d_c = A * B^T in fp32, where d_fa and d_fb
 * are what swz_stage_operand wrote for A [m][k] and for B^T [n][k] (B
 * column-major), on the 16x16x32 bf16 matrix instruction with fp32
 * accumulation.  The operand read that feeds the matrix unit is the step
 * the pages put after the swizzled staging ("NVIDIA CuTe Swizzle", ldmatrix
 * and WGMMA; "CuTe Swizzle 学习手册", usage step 5); since the fragments are
 * already in lane order, each is one contiguous KiB, loaded straight into
 * LDS and read back lane-linearly (every bank once).
 *   d_c : [m][n] row-major fp32, written (not accumulated into); must not
 *         overlap the inputs.
 *   m, n multiples of 16, k a multiple of 32 (the fragment format); k = 0
 *   writes zeros.  All pointers 16-byte aligned.  frag_kind must be
 *   SWZ_FRAG_MFMA_F32_16X16X32_BF16.
 * The sum over k is taken 32 at a time by the instruction and accumulated
 * in fp32 in increasing k order.
 * Errors: SWZ_EINVAL (sizes, alignment, NULL, overlap, fragment kind). */
int swz_gemm_frag(const void* d_fa, const void* d_fb, float* d_c, int64_t m, int64_t n, int64_t k,
                  int32_t frag_kind, void* stream);

/* GEMM with the staging inside: d_c = A * B^T in fp32 from bf16 operands in
 * their natural layouts, A [m][k] row-major (d_a) and B^T [n][k] row-major
 * (d_bt; B column-major).  This is the use the pages build the swizzle for:
 * each k stage copies a 256 x 64 tile of A and one of B^T from HBM straight
 * into a swizzled LDS tile (the cp.async step), and the operand reads take
 * the 16x16x32 instruction's fragments out of it (the ldmatrix step) --
 * "NVIDIA CuTe Swizzle", cp.async, ldmatrix and the MMA; "CuTe Swizzle
 * 学习手册", usage steps 2, 3 and 5.  The tile is the one swz_stage_operand
 * stages, read in the same pattern.
 *   layout    : SWZ_LAYOUT_SWIZZLE or SWZ_LAYOUT_SWIZZLE_DIRECT (the same
 *               here: the fill is always direct), or SWZ_LAYOUT_PLAIN (the
 *               ablation: row-major tiles, whose fragment reads conflict).
 *               SWZ_LAYOUT_PAD returns SWZ_EUNSUPPORTED (a direct load
 *               writes whole unpadded rows).
 *   p_or_null : the swizzle for the SWIZZLE layouts (|S| >= B, as for
 *               SWZ_LAYOUT_SWIZZLE_DIRECT), or NULL for the chooser's.
 *   d_c       : [m][n] row-major fp32, written (not accumulated into); must
 *               not overlap the inputs.
 *   m, n multiples of 16, k a multiple of 32; k = 0 writes zeros.  All
 *   pointers 16-byte aligned.
 * The products are exact in fp32 and the sum over k is accumulated in fp32,
 * 32 at a time by the instruction, in increasing k order -- the same result
 * as swz_gemm_frag on the staged operands.
 * Errors: SWZ_EINVAL (sizes, alignment, NULL, overlap, parameters),
 * SWZ_EUNSUPPORTED (PAD). */
int swz_gemm(const void* d_a, const void* d_bt, float* d_c, int64_t m, int64_t n, int64_t k, int32_t layout,
             const swz_params* p_or_null, void* stream);

/* Element type of the GEMM result. */
enum swz_c_type { SWZ_C_F32 = 0, SWZ_C_BF16 = 1 };

/* swz_gemm with a choice of result type: c_type SWZ_C_F32 is swz_gemm
 * (d_c float [m][n]); SWZ_C_BF16 writes d_c as bf16 [m][n] (uint16 bit
 * patterns), each element the fp32 result of swz_gemm rounded to nearest
 * with ties to even (NaN stays NaN), half the bytes of C to write.
 * Errors: those of swz_gemm; SWZ_EINVAL for another c_type. */
int swz_gemm_ex(const void* d_a, const void* d_bt, void* d_c, int64_t m, int64_t n, int64_t k, int32_t layout,
                const swz_params* p_or_null, int32_t c_type, void* stream);

/* Host only.  The swizzle the library uses for a tile of tile_rows x
 * tile_cols elements of elem_bytes, staged by vec_bytes-wide stores and read
 * back by read_kind, under the built-in gfx950 LDS bank model:
 * M = log2(vec_bytes / elem_bytes), B = log2(vectors per bank row) (bounded
 * by the tile), S the smallest shift >= B with the fewest predicted
 * bank-conflict cycles over the kernel's write and read lane patterns
 * ("NVIDIA CuTe Swizzle", derivation of the three parameters; "CUDA 013 -
 * Swizzle 的工作原理", section CuTe 通用 swizzle 映射规则解析).  Only the
 * (elem_bytes, vec_bytes, tile, read_kind) combinations the kernels use are
 * accepted; others return SWZ_EUNSUPPORTED. */
int swz_choose(int32_t elem_bytes, int32_t vec_bytes, int32_t tile_rows, int32_t tile_cols,
               int32_t read_kind, swz_params* out);

/* Host only.  Folding a swizzle into a plain layout over a slice ("cutlass
 * 入门", section swizzle 融入 layout 优化).  A slice is the set of offsets
 * base | x with x ranging over the subsets of the bit mask `active` (the bits
 * a slice's coordinates can change; base has none of them).  The page's test:
 * collision = active & ~swizzle(active) marks every target bit whose source
 * bit is also active; when it is zero the swizzle restricted to the slice is
 * a plain (strided) layout:
 *   swizzle(base | x) = swizzle(base) + sum over set bits b of x of strides[b].
 *   p          : the swizzle (S of either sign; B + M + |S| <= 32).
 *   *collision : the collision bits (always written).
 *   *folded_base, strides[32] : swizzle(base) and the signed per-bit strides
 *                (strides[b] = 0 for bits outside `active`), written only
 *                when the slice folds; either may be NULL.
 * Returns SWZ_OK when the slice folds, SWZ_EUNSUPPORTED when it does not
 * (collision != 0), SWZ_EINVAL for bad parameters, base & active != 0 or a
 * NULL collision pointer. */
int swz_fold(const swz_params* p, uint32_t base, uint32_t active, uint32_t* collision, uint32_t* folded_base,
             int64_t* strides);

/* Host only.  Predicted conflict cycles (write + read, summed over one
 * tile) of the kernel pattern for read_kind under the built-in bank model,
 * for the given layout and parameters (params ignored for PAD and PLAIN;
 * with SWIZZLE_DIRECT the writes are the direct fill's lane-linear ones). */
int swz_predict_conflicts(int32_t read_kind, int32_t layout, const swz_params* p_or_null,
                          int64_t* write_cycles, int64_t* read_cycles);

/* Host only.  The LDS accesses one tile of the kernel for read_kind issues,
 * as byte addresses per lane: the staging stores (is_write = 1) or the reads
 * (is_write = 0), one 64-lane access after another (all waves, all steps),
 * in the given layout.  Writes min(count, max_accesses) x 64 addresses to
 * addrs (int32, -1 = lane idle), the total count to *n_accesses and the
 * bytes per lane to *width.  Lets tests and the bank microbenchmark check
 * the exact patterns the kernels use. */
int swz_kernel_accesses(int32_t read_kind, int32_t layout, const swz_params* p_or_null, int32_t is_write,
                        int32_t* addrs, int32_t max_accesses, int32_t* n_accesses, int32_t* width);

/* The LDS bank model the chooser uses, per access direction d (0 = read,
 * 1 = write) and width w (4 << w bytes per lane): n_banks banks of
 * bank_bytes, byte a in bank (a / bank_bytes) % n_banks ("CuTe Swizzle
 * 学习手册", bank structure, gives one geometry, 32 x 4 bytes, for NVIDIA;
 * gfx950's depends on the access and is measured with swz_lds_probe), and
 * phase[d][w][l], the group of lanes served together. */
typedef struct swz_bank_model {
    int32_t n_banks[2][3];
    int32_t bank_bytes[2][3];
    uint8_t phase[2][3][64];
} swz_bank_model;

/* Host only.  Copy the built-in gfx950 model to *out.  SWZ_EINVAL on NULL. */
int swz_bank_model_get(swz_bank_model* out);

/* Host only.  Fill *out with what swz_convert_layout (op = 0) or
 * swz_stage_operand (op = 1) would do for these arguments, without
 * launching anything; pointers are not inspected (they are taken to be
 * 16-byte aligned, so aligned reflects the row pitches).  Same validation and
 * errors as the call. */
int swz_plan(int32_t op, int64_t rows, int64_t cols, int32_t elem_bytes, int32_t layout,
             int32_t read_kind, const swz_params* p_or_null, swz_plan_info* out);

/* Host only.  Static text for a status code. */
const char* swz_strerror(int status);

/* Reference copy (diagnostic): d_dst[0..bytes) = d_src[0..bytes) with plain
 * 16-byte vector loads and stores and the same launch policy as the tile
 * kernels.  It is the read-once / write-once ceiling the tile kernels are
 * compared with, and the kernel of known size HBM byte counters are scaled
 * by.  bytes must be a multiple of 16, pointers 16-byte aligned, buffers
 * disjoint.  Errors: SWZ_EINVAL otherwise. */
int swz_copy(const void* d_src, void* d_dst, int64_t bytes, void* stream);

/* LDS bank microbenchmark (diagnostic; used to measure the bank model the
 * chooser relies on).  Launches n_patterns workgroups of `waves` 64-lane
 * waves.  Workgroup g runs pattern g: lane l of every wave accesses LDS byte
 * d_addrs[64*g + l] (taken modulo the probe's 96 KiB LDS window and aligned
 * down to width_bytes) if bit l of d_masks[g] is set, with ds_read_u8/u16/
 * b32/b64/b128 (is_write = 0) or ds_write_b8/b16/b32/b64/b128
 * (is_write = 1), 8 accesses per iteration for `iters` iterations, and
 * writes the wave's elapsed shader-clock cycles to d_cycles[g * waves + w].
 *   width_bytes: 1, 2, 4, 8 or 16; waves: 1..16; iters: 1..1<<20.
 * Errors: SWZ_EINVAL on any other value or NULL pointer. */
int swz_lds_probe(const uint32_t* d_addrs, const uint64_t* d_masks, int32_t n_patterns,
                  int32_t width_bytes, int32_t is_write, int32_t iters, int32_t waves,
                  uint64_t* d_cycles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWZ_H */
