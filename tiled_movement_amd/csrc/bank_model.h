// LDS bank model of gfx950 and a per-wave bank-conflict predictor (host).
#pragma once

#include <stdint.h>

namespace swz {

// For each access direction (0 = read, 1 = write) and width (4 << w bytes
// per lane, w = 0, 1, 2): n_banks banks of bank_bytes, byte a in bank
// (a / bank_bytes) % n_banks ("CuTe Swizzle 学习手册", bank structure, states
// this with one geometry of 32 x 4 bytes), and phase[d][w][lane], the group
// of lanes the LDS serves together.  Within a phase, lanes asking one bank
// for different words are serialised; the same word is broadcast.
struct BankModel {
    int n_banks[2][3];
    int bank_bytes[2][3];
    uint8_t phase[2][3][64];
};

// The model the chooser uses on gfx950 (measured with swz_lds_probe).
const BankModel& gfx950_bank_model();

// One geometry for every access, phases of one bank row each.
BankModel uniform_model(int n_banks, int bank_bytes);

// One wave-wide LDS access: byte address per lane, -1 = lane inactive.
struct Access {
    int32_t addr[64];
    int width;  // bytes per lane: 4, 8 or 16
    bool write;
};

// Extra cycles the access costs: sum over phases of (worst words per bank - 1).
int conflict_cycles(const BankModel& m, const Access& a, int* worst_degree = nullptr);

}  // namespace swz
