// Exact division of slot indices by seq_len with a multiply and a shift.
// Host-only, dependency-free (also compiled by a CPU test).
#pragma once

#include <stdint.h>

namespace rlpl {

// Exact division by an invariant divisor d (1 <= d < 2^31) for dividends
// n < 2^31 (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, round-up variant): with l = ceil(log2 d) and
// m = ceil(2^(31+l) / d), floor(n / d) == (n * m) >> (31 + l), because
// m*d - 2^(31+l) < d <= 2^l bounds the error below one for every n < 2^31.
// m < 2^32 since d > 2^(l-1) (or d == 2^l, where m == 2^31).
inline bool row_divisor(uint32_t d, uint32_t* magic, uint32_t* shift) {
    if (d < 1 || d >= (1u << 31)) return false;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << (31 + l)) + d - 1) / d;
    if (m >> 32) return false;
    *magic = uint32_t(m);
    *shift = 31 + l;
    // Self-check at the edges of the domain and around multiples of d.
    const uint32_t probes[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7FFFFFFFu, 0x7FFFFFFFu - d,
                               (0x7FFFFFFFu / d) * d, (0x7FFFFFFFu / d) * d - 1};
    for (uint32_t n : probes) {
        if (n >= (1u << 31)) continue;
        if (uint32_t((uint64_t(n) * m) >> (31 + l)) != n / d) return false;
    }
    return true;
}

}  // namespace rlpl
