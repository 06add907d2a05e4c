"""The fast division helper of the kernels, checked on the host against plain
integer division (compiled with g++; no GPU)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_re_layout_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.hpp"
using namespace basp;
static int check(uint32_t d, uint32_t n) {
    FastDiv f = make_fastdiv(d);
    if (fastdiv(n, f) != n / d) { std::printf("FAIL d=%u n=%u got=%u\n", d, n, fastdiv(n, f)); return 1; }
    return 0;
}
int main() {
    std::mt19937_64 rng(7);
    const uint32_t top = 0x7fffffffu;
    int bad = 0;
    for (uint32_t d = 1; d <= 4096 && !bad; ++d) {
        for (uint32_t n = 0; n < 4 * d + 64; ++n) bad |= check(d, n);
        for (uint32_t n = top - 4 * d - 64; n <= top - 1; ++n) bad |= check(d, n);
        bad |= check(d, top);
        for (int i = 0; i < 2000; ++i) bad |= check(d, uint32_t(rng() % (uint64_t(top) + 1)));
    }
    for (int i = 0; i < 2000000 && !bad; ++i) {
        uint32_t d = uint32_t(rng() % top) + 1;
        uint32_t n = uint32_t(rng() % (uint64_t(top) + 1));
        bad |= check(d, n);
        bad |= check(d, top);
        bad |= check(d, (n / d) * d);
        if (d > 1) bad |= check(d, (n / d) * d - 1 + (n < d ? d : 0));
    }
    for (uint32_t k = 0; k < 31 && !bad; ++k) {
        uint32_t d = 1u << k;
        for (uint32_t e : {d - 1, d, d + 1})
            if (e >= 1 && e <= top) for (uint32_t n : {0u, 1u, e - 1, e, e + 1, top - 1, top}) bad |= check(e, n);
    }
    std::printf(bad ? "FAIL\n" : "OK\n");
    return bad;
}
"""


def test_fastdiv_exact(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-DBASP_HD=", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout[-2000:]
