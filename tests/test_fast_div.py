"""The repack's division by the chunks per row (tiled_bf16_gemm_amd/csrc/fast_div.hpp: a
multiply-high and shifts, Granlund and Montgomery 1994) against the integer quotient, on the host:
every divisor up to 4096 and random ones up to 2^32 - 1, with the numerators around each multiple
of the divisor and at the ends of the 32-bit range."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = r"""
#include <cstdio>
#include <cstdint>
#include "fast_div.hpp"
static uint64_t s = 88172645463325252ull;
static uint32_t next() { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)(s >> 16); }
static int check(uint32_t d, uint32_t n) {
  const uint32_t q = tbg::fast_div(n, tbg::make_fast_div(d));
  if (q != n / d) { std::printf("d=%u n=%u got %u want %u\n", d, n, q, n / d); return 1; }
  return 0;
}
static int divisor(uint32_t d) {
  int bad = 0;
  const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 0xFFFFFFFFu, 0xFFFFFFFEu, 0x80000000u, 0x7FFFFFFFu};
  for (uint32_t n : edge) bad += check(d, n);
  const uint32_t top = 0xFFFFFFFFu / d;
  for (int i = 0; i < 64; ++i) {
    const uint32_t k = top ? next() % top + 1 : 1;  // a multiple k*d <= 2^32 - 1
    const uint64_t m = (uint64_t)k * d;
    bad += check(d, (uint32_t)(m - 1));
    if (m <= 0xFFFFFFFFu) bad += check(d, (uint32_t)m);
    bad += check(d, next());
  }
  return bad;
}
int main() {
  int bad = 0;
  for (uint32_t d = 1; d <= 4096; ++d) bad += divisor(d);
  for (int i = 0; i < 20000; ++i) bad += divisor(next() | 1u), bad += divisor(next() + 1u > 0 ? next() + 1u : 1u);
  const uint32_t special[] = {65535u, 65536u, 65537u, 0x7FFFFFFFu, 0x80000000u, 0x80000001u, 0xFFFFFFFEu, 0xFFFFFFFFu};
  for (uint32_t d : special) bad += divisor(d);
  std::printf("%d mismatches\n", bad);
  return bad != 0;
}
"""


def test_fast_div_matches_integer_division(tmp_path):
    src = tmp_path / "fast_div_check.cpp"
    src.write_text(HARNESS)
    exe = tmp_path / "fast_div_check"
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "tiled_bf16_gemm_amd", "csrc"), str(src),
                        "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip() == "0 mismatches"
