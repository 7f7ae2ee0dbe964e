// Swizzle parameter chooser and per-tile conflict prediction (host).
#pragma once

#include <stdint.h>

#include "bank_model.h"
#include "swz.h"

namespace swz {

struct KindInfo {
    int esz, tr, tc, nt, vec, rwidth, wsteps, rsteps;
};

// Static facts of a read kind; false for an unknown kind.
bool kind_info(int kind, KindInfo* out);

// Predicted conflict cycles over one tile for the kind's staging writes and
// reads, with LDS row pitch ld and swizzle p (B = 0 for none).  direct: the
// writes are those of the direct fill (lane-linear), not the register fill's.
void predict_tile(int kind, const BankModel& m, uint32_t ld, swz_params p, int64_t* wcyc, int64_t* rcyc,
                  bool direct = false);

// Swizzle of SWZ_READ_ROWS tiles (rows of `cols` elements, 1-64, copied
// flat): word w of the tile lives at w ^ ((w >> S) & (2^B - 1)) (M = 0).
// Lanes of a read are cols words apart, so an even width meets conflicts
// that the XOR of bits above the bank bits into the bank bits removes; odd
// widths need none (B = 0).  Searched against the model's 4-byte reads of
// that pattern and the 4-byte writes of the flat copy; cached per width
// (1 to kRowsMaxCols; none for other widths).
constexpr int kRowsMaxCols = 128;
swz_params rows_choice(int cols);

// Chooser: see swz_choose in swz.h.  Result cached per kind for the gfx950
// model; the model argument form is uncached.
swz_params choose_for_kind(int kind, const BankModel& m, int64_t* cycles);
swz_params cached_choice(int kind);

// The kernel's LDS accesses for one tile (see swz_kernel_accesses).
int kernel_accesses(int kind, uint32_t ld, swz_params p, bool direct, bool write, int32_t* addrs, int max_acc,
                    int* width);

// Pad (elements per LDS row) of the padded layout for a kind.
int pad_elems(int kind);

// Validate caller parameters for a kind: B, M non-negative, fields inside
// 32 bits, S != 0 when B > 0 (S = 0 would not be one-to-one; S may be
// negative), vectors kept whole (2^M >= elements per LDS store and per LDS
// load) and the field that changes inside the tile.
bool params_ok_for_kind(int kind, swz_params p);

}  // namespace swz
