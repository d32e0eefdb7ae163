"""The launch-time division used to find a position's DCP shard
(csrc/mla_fastdiv.h) against exact integer division, compiled for the host:
every divisor up to 5000 plus large ones, on edge and random dividends."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECK = r'''
#include <cstdio>
#include <cstdint>
#include <random>
#include "mla_fastdiv.h"
int main() {
  std::mt19937_64 g(7);
  long bad = 0, n_checked = 0;
  auto check = [&](uint32_t d) {
    const mla::FastDiv f = mla::make_fastdiv(d);
    const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7FFFFFFFu, 0x80000000u, 0xFFFFFFFFu};
    for (uint32_t n : edge) { bad += mla::fastdiv(n, f) != n / d; ++n_checked; }
    for (int i = 0; i < 2000; ++i) {
      const uint32_t n = (uint32_t)g();
      bad += mla::fastdiv(n, f) != n / d; ++n_checked;
      const uint32_t m = (uint32_t)(g() % 262144);  // positions of long sequences
      bad += mla::fastdiv(m, f) != m / d; ++n_checked;
    }
  };
  for (uint32_t d = 1; d <= 5000; ++d) check(d);
  const uint32_t big[] = {65535u, 65536u, 65537u, 1u << 20, (1u << 31) - 1, 1u << 31, 0xFFFFFFFEu, 0xFFFFFFFFu};
  for (uint32_t d : big) check(d);
  printf("%ld %ld\n", bad, n_checked);
  return bad != 0;
}
'''


def test_fastdiv_is_exact(tmp_path):
    src = tmp_path / "check.cpp"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "latent_decode_attention_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    bad, checked = map(int, out.stdout.split())
    assert out.returncode == 0 and bad == 0 and checked > 20_000_000
