"""Host check of the shared-row kernels' work-unit mapping (unit_map / unit_of_block in
csrc/e2f_device.hpp): compiled for the host with hipcc, every schedule slot of [0, N) must land
in exactly one unit, for many N, unit sizes and closing fractions (CPU only)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "interatomic_potentials_amd", "csrc")

PROG = r'''
#include "e2f_device.hpp"
#include <cstdio>
#include <cstdint>
#include <vector>
int main() {
  const int64_t Ns[] = {1, 2, 7, 63, 64, 100, 4097, 5000, 32767, 32768, 100003, 131071};
  const int cases[][3] = {{4, 16, 2}, {4, 8, 2}, {4, 16, 1}, {3, 16, 2}, {3, 0, 2}, {2, 16, 1},
                          {4, 0, 2}, {2, 0, 1}};
  for (int64_t N : Ns)
    for (const auto& c : cases) {
      const int T = c[0], den = c[1], tt = c[2];
      const e2f::UnitMap u = e2f::unit_map(N, T, den, tt);
      std::vector<int> seen(N, 0);
      for (int64_t blk = 0; blk < u.per_xcd * e2f::kXcds; ++blk) {
        int64_t slot0, xend;
        int cnt;
        e2f::unit_of_block(u, blk, T, tt, slot0, cnt, xend);
        if (slot0 >= N) continue;
        for (int t = 0; t < T; ++t) {
          const int64_t sl = slot0 + t;
          if (t < cnt && sl < N && sl < xend) ++seen[sl];
        }
      }
      for (int64_t s = 0; s < N; ++s)
        if (seen[s] != 1) {
          std::printf("N=%ld T=%d den=%d tt=%d slot %ld seen %d\n", N, T, den, tt, s, seen[s]);
          return 1;
        }
    }
  std::printf("ok\n");
  return 0;
}
'''


def test_every_slot_in_exactly_one_unit(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "unit_map.hip"
    src.write_text(PROG)
    exe = tmp_path / "unit_map"
    subprocess.run([hipcc, "-std=c++17", "-O1", f"-I{CSRC}", "--offload-arch=gfx950", str(src),
                    "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout
