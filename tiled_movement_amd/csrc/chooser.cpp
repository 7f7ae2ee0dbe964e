// Swizzle<B,M,S> chooser for gfx950 LDS (host).
//
// The pages derive the three parameters from the hardware ("NVIDIA CuTe
// Swizzle", derivation of MBase / BBits / SShift; "CUDA 013 - Swizzle 的
// 工作原理", section CuTe 通用 swizzle 映射规则解析): M keeps one vector
// whole, B spans one bank row of vectors, S reaches the row bits.  Their bank
// row is 32 x 4 bytes; here it comes from the measured gfx950 model, and S is
// picked by predicting the conflicts of the kernel's own lane patterns, since
// which row bits vary inside one LDS phase depends on how lanes are assigned.
#include "chooser.h"

#include <mutex>

#include "swz_common.h"

namespace swz {

namespace {

int ilog2(int64_t v) {
    int r = -1;
    while (v > 0) {
        v >>= 1;
        ++r;
    }
    return r;
}

// LDS addresses of the direct fill's load j of one wave (lane-linear).
template <int KIND>
void direct_write(int wave, int j, int32_t* addr) {
    using D = Direct<KIND>;
    for (int l = 0; l < 64; ++l) addr[l] = D::VB * (64 * wave + l + Kind<KIND>::NT * j);
}

template <int KIND>
void predict_kind(const BankModel& m, uint32_t ld, swz_params p, bool direct, int64_t* wcyc, int64_t* rcyc) {
    using K = Kind<KIND>;
    const LdsLayout L{ld, static_cast<uint32_t>(p.B), static_cast<uint32_t>(p.M), p.S};
    int64_t w = 0, r = 0;
    Access a;
    for (int wave = 0; wave < K::NT / 64; ++wave) {
        for (int j = 0; direct && j < Direct<KIND>::LOADS; ++j) {
            a.width = Direct<KIND>::VB;
            a.write = true;
            direct_write<KIND>(wave, j, a.addr);
            w += conflict_cycles(m, a);
        }
        for (int i = 0; !direct && i < K::WSTEPS; ++i) {
            a.width = K::VEC;
            a.write = true;
            for (int l = 0; l < 64; ++l) {
                int rr, cc;
                K::wcoord(wave * 64 + l, i, rr, cc);
                a.addr[l] = static_cast<int32_t>(lds_elem(L, rr, cc) * K::ESZ);
            }
            w += conflict_cycles(m, a);
        }
        for (int i = 0; i < K::RSTEPS; ++i) {
            a.width = K::RWIDTH;
            a.write = false;
            for (int l = 0; l < 64; ++l) {
                int rr, cc;
                K::rcoord(wave * 64 + l, i, rr, cc);
                a.addr[l] = static_cast<int32_t>(lds_elem(L, rr, cc) * K::ESZ);
            }
            r += conflict_cycles(m, a);
        }
    }
    *wcyc = w;
    *rcyc = r;
}

template <int KIND>
int accesses_kind(uint32_t ld, swz_params p, bool direct, bool write, int32_t* addrs, int max_acc, int* width) {
    using K = Kind<KIND>;
    const LdsLayout L{ld, static_cast<uint32_t>(p.B), static_cast<uint32_t>(p.M), p.S};
    const bool dw = direct && write;
    const int steps = dw ? Direct<KIND>::LOADS : write ? K::WSTEPS : K::RSTEPS;
    *width = dw ? Direct<KIND>::VB : write ? K::VEC : K::RWIDTH;
    int n = 0;
    for (int wave = 0; wave < K::NT / 64; ++wave) {
        for (int i = 0; i < steps; ++i, ++n) {
            if (n >= max_acc || !addrs) continue;
            if (dw) {
                direct_write<KIND>(wave, i, addrs + 64 * n);
                continue;
            }
            for (int l = 0; l < 64; ++l) {
                int rr, cc;
                if (write)
                    K::wcoord(wave * 64 + l, i, rr, cc);
                else
                    K::rcoord(wave * 64 + l, i, rr, cc);
                addrs[64 * n + l] = static_cast<int32_t>(lds_elem(L, rr, cc) * K::ESZ);
            }
        }
    }
    return n;
}

}  // namespace

int kernel_accesses(int kind, uint32_t ld, swz_params p, bool direct, bool write, int32_t* addrs, int max_acc,
                    int* width) {
    int n = -1;
    with_kind(kind, [&](auto kd) { n = accesses_kind<decltype(kd)::value>(ld, p, direct, write, addrs, max_acc, width); });
    return n;
}

bool kind_info(int kind, KindInfo* o) {
    return with_kind(kind, [&](auto kd) {
        using K = Kind<decltype(kd)::value>;
        *o = KindInfo{K::ESZ, K::TR, K::TC, K::NT, K::VEC, K::RWIDTH, K::WSTEPS, K::RSTEPS};
    });
}

int pad_elems(int kind) {
    KindInfo k;
    if (!kind_info(kind, &k)) return 0;
    // One element for scalar staging (the 32x33 array of the pages); one
    // 16-byte vector for vector staging so every row stays 16-byte aligned.
    return k.vec == k.esz ? 1 : k.vec / k.esz;
}

void predict_tile(int kind, const BankModel& m, uint32_t ld, swz_params p, int64_t* wcyc, int64_t* rcyc,
                  bool direct) {
    *wcyc = *rcyc = -1;
    with_kind(kind, [&](auto kd) { predict_kind<decltype(kd)::value>(m, ld, p, direct, wcyc, rcyc); });
}

bool params_ok_for_kind(int kind, swz_params p) {
    KindInfo k;
    if (!kind_info(kind, &k)) return false;
    if (p.B < 0 || p.M < 0) return false;
    const int64_t abs_s = p.S < 0 ? -static_cast<int64_t>(p.S) : p.S;
    if (p.B == 0) return p.M + abs_s <= 32;
    if (p.B + p.M + abs_s > 32) return false;
    if (abs_s < 1) return false;
    const int min_vec = k.vec > k.rwidth ? k.vec : k.rwidth;
    if ((1 << p.M) < min_vec / k.esz) return false;
    // The field that changes starts at M (S > 0) or M + |S| (S < 0); it must
    // stay inside the tile.
    const int64_t target = p.S > 0 ? p.M : p.M + abs_s;
    if (target + p.B > ilog2(static_cast<int64_t>(k.tr) * k.tc)) return false;
    return true;
}

swz_params choose_for_kind(int kind, const BankModel& m, int64_t* cycles) {
    KindInfo k;
    swz_params none{0, 0, 0};
    if (!kind_info(kind, &k)) return none;
    const int M = ilog2(k.vec / k.esz);
    const int log_tile = ilog2(static_cast<int64_t>(k.tr) * k.tc);
    const int b_max = (log_tile - M) / 2;
    // B spans one bank row as the reads see it (the layout exists for them).
    const int rw = k.rwidth <= 4 ? 0 : k.rwidth == 8 ? 1 : 2;
    const int row_bytes = m.n_banks[0][rw] * m.bank_bytes[0][rw];
    int b_rule = row_bytes >= k.vec ? ilog2(row_bytes / k.vec) : 0;
    if (b_rule > b_max) b_rule = b_max;

    auto cost = [&](int B, int S) {
        int64_t w, r;
        predict_tile(kind, m, static_cast<uint32_t>(k.tc), swz_params{B, M, S}, &w, &r);
        return w + r;
    };

    swz_params best{b_rule, M, b_rule};
    int64_t best_cyc = -1;
    for (int S = b_rule; S <= log_tile - M - b_rule; ++S) {
        const int64_t c = cost(b_rule, S);
        if (best_cyc < 0 || c < best_cyc) {
            best = swz_params{b_rule, M, S};
            best_cyc = c;
        }
        if (c == 0) {
            if (cycles) *cycles = 0;
            return best;
        }
    }
    // No zero-conflict shift at the rule's B: widest search, ties to the B
    // nearest the rule, then the smaller S.
    for (int B = 1; B <= b_max; ++B) {
        for (int S = B; S <= log_tile - M - B; ++S) {
            const int64_t c = cost(B, S);
            const int db = B > b_rule ? B - b_rule : b_rule - B;
            const int dbest = best.B > b_rule ? best.B - b_rule : b_rule - best.B;
            if (c < best_cyc || (c == best_cyc && (db < dbest || (db == dbest && S < best.S)))) {
                best = swz_params{B, M, S};
                best_cyc = c;
            }
        }
    }
    if (cycles) *cycles = best_cyc;
    return best;
}

namespace {

uint32_t rows_swz(uint32_t w, uint32_t B, uint32_t S) { return w ^ ((w >> S) & ((1u << B) - 1u)); }

// Extra cycles of the reads and writes of one rows tile under (B, S): four
// wave steps of every column offset for the reads; four 64-lane groups of
// 4-byte writes (word j of each lane's 16-byte vector) for a swizzled copy,
// whose 16-byte vector writes are lane-linear (no conflicts) when B = 0.
int64_t rows_cost(int cols, uint32_t B, uint32_t S, const BankModel& m) {
    int64_t cyc = 0;
    Access a{};
    a.width = 4;
    a.write = false;
    for (int s = 0; s < 4; ++s)
        for (int k = 0; k < cols; ++k) {
            for (int t = 0; t < 64; ++t)
                a.addr[t] = static_cast<int32_t>(4 * rows_swz(static_cast<uint32_t>((64 * s + t) * cols + k), B, S));
            cyc += conflict_cycles(m, a);
        }
    if (B == 0) return cyc;
    a.write = true;
    for (int g = 0; g < 4; ++g)
        for (int j = 0; j < 4; ++j) {
            for (int t = 0; t < 64; ++t)
                a.addr[t] = static_cast<int32_t>(4 * rows_swz(static_cast<uint32_t>(4 * (64 * g + t) + j), B, S));
            cyc += cols * conflict_cycles(m, a) / 4;  // as many write as read instructions per tile
        }
    return cyc;
}

}  // namespace

swz_params rows_choice(int cols) {
    if (cols < 1 || cols > kRowsMaxCols) return swz_params{0, 0, 0};
    static std::once_flag once[kRowsMaxCols + 1];
    static swz_params table[kRowsMaxCols + 1];
    std::call_once(once[cols], [cols] {
        const BankModel& m = gfx950_bank_model();
        swz_params best{0, 0, 0};
        int64_t best_cyc = rows_cost(cols, 0, 0, m);
        for (int B = 1; B <= 5 && best_cyc > 0; ++B)
            for (int S = B; S <= 8; ++S) {
                const int64_t cyc = rows_cost(cols, B, S, m);
                if (cyc < best_cyc) {
                    best_cyc = cyc;
                    best = swz_params{B, 0, S};
                }
            }
        table[cols] = best;
    });
    return table[cols];
}

swz_params cached_choice(int kind) {
    static std::once_flag once;
    constexpr int kKinds = kNumKinds;
    static swz_params table[kKinds];
    std::call_once(once, [] {
        for (int kd = 0; kd < kKinds; ++kd) table[kd] = choose_for_kind(kd, gfx950_bank_model(), nullptr);
    });
    if (kind < 0 || kind >= kKinds) return swz_params{0, 0, 0};
    return table[kind];
}

}  // namespace swz
