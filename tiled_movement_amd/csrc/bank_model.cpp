// gfx950 LDS bank model and conflict predictor.
#include "bank_model.h"

#include <algorithm>

namespace swz {

BankModel contiguous_model(int n_banks, int bank_bytes) {
    BankModel m{};
    m.n_banks = n_banks;
    m.bank_bytes = bank_bytes;
    for (int w = 0; w < 3; ++w) {
        const int width = 4 << w;
        int per = n_banks * bank_bytes / width;
        if (per < 1) per = 1;
        if (per > 64) per = 64;
        for (int l = 0; l < 64; ++l) {
            m.read_phase[w][l] = static_cast<uint8_t>(l / per);
            m.write_phase[w][l] = static_cast<uint8_t>(l / per);
        }
    }
    return m;
}

const BankModel& gfx950_bank_model() {
    // 64 banks of 4 bytes (256 bytes per bank row), one bank row per phase.
    static const BankModel m = contiguous_model(64, 4);
    return m;
}

int conflict_cycles(const BankModel& m, const Access& a, int* worst_degree) {
    const int w = a.width == 4 ? 0 : a.width == 8 ? 1 : 2;
    const uint8_t* phase = a.write ? m.write_phase[w] : m.read_phase[w];
    int n_phases = 0;
    for (int l = 0; l < 64; ++l) n_phases = std::max(n_phases, phase[l] + 1);

    int cycles = 0, worst = 0;
    // (bank, word) pairs touched in the current phase.
    std::vector<int64_t> words;
    words.reserve(256);
    for (int p = 0; p < n_phases; ++p) {
        words.clear();
        for (int l = 0; l < 64; ++l) {
            if (phase[l] != p || a.addr[l] < 0) continue;
            const int64_t first = a.addr[l] / m.bank_bytes;
            const int64_t last = (a.addr[l] + a.width - 1) / m.bank_bytes;
            for (int64_t wd = first; wd <= last; ++wd) words.push_back(wd);
        }
        if (words.empty()) continue;
        std::sort(words.begin(), words.end());
        words.erase(std::unique(words.begin(), words.end()), words.end());
        // Distinct words per bank; the worst bank sets the phase's passes.
        std::vector<int> per_bank(m.n_banks, 0);
        int degree = 0;
        for (int64_t wd : words) {
            const int b = static_cast<int>(wd % m.n_banks);
            degree = std::max(degree, ++per_bank[b]);
        }
        cycles += degree - 1;
        worst = std::max(worst, degree);
    }
    if (worst_degree) *worst_degree = worst;
    return cycles;
}

}  // namespace swz
