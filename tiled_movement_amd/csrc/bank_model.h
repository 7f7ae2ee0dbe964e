// LDS bank model of gfx950 and a per-wave bank-conflict predictor (host).
#pragma once

#include <stdint.h>

#include <vector>

namespace swz {

// n_banks banks of bank_bytes; byte a lies in bank (a / bank_bytes) % n_banks
// ("CuTe Swizzle 学习手册", bank structure, states this for 32 x 4 B).
// phase[w][lane] numbers the group of lanes the LDS serves together for an
// access of 4 << w bytes per lane (w = 0, 1, 2), separately for reads and
// writes.  Within a phase, lanes asking one bank for different words are
// serialised; the same word is broadcast.
struct BankModel {
    int n_banks;
    int bank_bytes;
    uint8_t read_phase[3][64];
    uint8_t write_phase[3][64];
};

// The model the chooser uses on gfx950.
const BankModel& gfx950_bank_model();

// Contiguous phases of one bank row each: n_banks*bank_bytes/width lanes.
BankModel contiguous_model(int n_banks, int bank_bytes);

// One wave-wide LDS access: byte address per lane, -1 = lane inactive.
struct Access {
    int32_t addr[64];
    int width;  // bytes per lane: 4, 8 or 16
    bool write;
};

// Extra cycles the access costs: sum over phases of (worst words per bank - 1).
int conflict_cycles(const BankModel& m, const Access& a, int* worst_degree = nullptr);

}  // namespace swz
