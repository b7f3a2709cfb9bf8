"""The library's division by invariant integers (`make_fastdiv` in the internal header,
Granlund and Montgomery's round-up method): the kernels take q = (umulhi(n, m) + n) >> s
as n / d for every 32-bit n and divisors 1 <= d <= 2^31. A host program built from the
library's own header checks the constants it makes against the integer quotient over
every divisor below 4096 and a spread of larger ones, for edge numerators (0, multiples
of d and their neighbours, the top of the 32-bit range, the 2^29-block limit) and
pseudo-random ones. No GPU is used."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "nvfp4_internal.h"

static uint32_t q_of(const nvfp4::FastDiv &f, uint32_t n) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (uint32_t)(((uint64_t)t + n) >> f.s);
}

int main() {
  std::vector<uint32_t> divs;
  for (uint32_t d = 1; d < 4096; ++d) divs.push_back(d);
  for (uint64_t d = 4096; d <= (1ull << 31); d = d * 3 / 2 + 7) divs.push_back((uint32_t)d);
  for (int k = 12; k <= 31; ++k) {
    divs.push_back((1u << k) - 1);
    divs.push_back(1u << k);
    divs.push_back((1u << k) + 1);
  }
  divs.push_back(0x7FFFFFFFu);
  divs.push_back(0x80000000u);
  uint64_t lcg = 0x9E3779B97F4A7C15ull, checked = 0, bad = 0;
  for (uint32_t d : divs) {
    const nvfp4::FastDiv f = nvfp4::make_fastdiv(d);
    std::vector<uint32_t> ns = {0u, 1u, d - 1u, d, d + 1u, 0xFFFFFFFFu, 0xFFFFFFFEu,
                                (1u << 29) - 1u, 1u << 29, (1u << 31) - 1u, 1u << 31};
    const uint64_t top = 0xFFFFFFFFull / d;
    for (uint64_t k : {top, top - 1, top / 2, (uint64_t)1 << 16, (uint64_t)3}) {
      if (k == 0 || k > top) continue;
      const uint64_t m = k * d;
      ns.push_back((uint32_t)m);
      ns.push_back((uint32_t)(m - 1));
      if (m + 1 <= 0xFFFFFFFFull) ns.push_back((uint32_t)(m + 1));
      if (m + d - 1 <= 0xFFFFFFFFull) ns.push_back((uint32_t)(m + d - 1));
    }
    for (int i = 0; i < 256; ++i) {
      lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
      ns.push_back((uint32_t)(lcg >> 32));
    }
    for (uint32_t n : ns) {
      ++checked;
      if (q_of(f, n) != n / d) {
        if (bad < 8) std::printf("bad d=%u n=%u got %u want %u\n", d, n, q_of(f, n), n / d);
        ++bad;
      }
    }
  }
  std::printf("checked %llu bad %llu\n", (unsigned long long)checked, (unsigned long long)bad);
  return bad != 0;
}
"""


def test_fastdiv_constants_give_the_integer_quotient(tmp_path):
    from microscaling_fp4_block_amd import build

    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(DRIVER)
    exe = str(tmp_path / "fastdiv_check")
    cmd = [build.hipcc(), "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950",
           "-I", build.CSRC, str(src), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("bad 0"), r.stdout
