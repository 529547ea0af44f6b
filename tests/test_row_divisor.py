"""The slot -> row division used by every kernel (multiply by a magic constant, shift).

Brute force on the CPU: the header is compiled with g++ and checked against
integer division for many divisors, on every dividend near each multiple of
the divisor and near the top of the range (dividends < 2^31).
"""
import os
import subprocess

HDR_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "rl_post_loss_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "row_divisor.h"
int main() {
    std::mt19937_64 rng(12345);
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 5000; ++d) ds.push_back(d);
    for (int e = 12; e <= 30; ++e) { ds.push_back(1u << e); ds.push_back((1u << e) - 1); ds.push_back((1u << e) + 1); }
    ds.push_back(0x7FFFFFFFu);
    for (int i = 0; i < 3000; ++i) ds.push_back(1 + uint32_t(rng() % 0x7FFFFFFEu));
    long checked = 0;
    for (uint32_t d : ds) {
        uint32_t m, sh;
        if (!rlpl::row_divisor(d, &m, &sh)) { std::printf("setup failed d=%u\n", d); return 1; }
        auto check = [&](uint64_t n) {
            if (n >= (1ull << 31)) return true;
            ++checked;
            return uint32_t((n * m) >> sh) == uint32_t(n / d);
        };
        uint64_t top = 0x7FFFFFFFull;
        for (uint64_t k = 0; k < 64; ++k) {
            uint64_t q = k, q2 = top / d - k;
            for (int64_t o = -2; o <= 2; ++o) {
                if (!check(q * d + o) || !check(q2 * d + o)) { std::printf("bad d=%u\n", d); return 1; }
            }
        }
        for (int i = 0; i < 200; ++i)
            if (!check(rng() & 0x7FFFFFFFull)) { std::printf("bad d=%u\n", d); return 1; }
    }
    uint32_t m, sh;
    if (rlpl::row_divisor(0, &m, &sh) || rlpl::row_divisor(0x80000000u, &m, &sh)) return 2;
    std::printf("ok %ld\n", checked);
    return 0;
}
"""


def test_row_divisor_matches_integer_division(tmp_path):
    src = tmp_path / "drv.cpp"
    src.write_text(DRIVER.replace("#include <random>", "#include <random>\n#include <vector>"))
    exe = tmp_path / "drv"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-I", HDR_DIR, str(src), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
