"""The persistent kernels' work schedule, checked on the host: the header's
schedule functions (schedule_item / schedule_phase) are compiled for the CPU
(hipcc, host pass only) into a small program that checks, for every tile
count up to 3000 per XCD and the 32 workers of an XCD, in both phases, that
every tile is covered exactly once, either whole or as both of its column
halves.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = textwrap.dedent(r"""
    #include <cstdio>
    #include <vector>
    #include "wgrad_kernels.hpp"
    using namespace forge;

    // Every even worker count per XCD a device can give (the launch uses
    // whole pairs per XCD, up to 32 compute units per XCD).
    static int check_persistent() {
      for (int nw = 2; nw <= 32; nw += 2)
      for (int R = 1; R <= 3000; ++R) {
        for (int phase = 0; phase < 2; ++phase) {
          if (phase && forge::schedule_phase(1, R, nw) == 0) continue;
          std::vector<int> cover(2 * R, 0);
          for (int j = 0; j < nw; ++j) {
            int tile, half;
            for (int k = 0; forge::schedule_item(k, j, nw, R, phase, tile, half); ++k) {
              if (tile < 0 || tile >= R) { printf("persistent: tile %d out of range R=%d\n", tile, R); return 1; }
              if (half < 0) { cover[2 * tile]++; cover[2 * tile + 1]++; }
              else cover[2 * tile + half]++;
            }
          }
          for (int i = 0; i < 2 * R; ++i)
            if (cover[i] != 1) { printf("persistent: nw=%d R=%d phase %d half-tile %d covered %d times\n", nw, R, phase, i, cover[i]); return 1; }
        }
      }
      return 0;
    }

    int main() {
      if (check_persistent()) return 1;
      printf("OK\n");
      return 0;
    }
""")


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def test_schedules_cover_every_tile_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "sched.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "sched"
    csrc = os.path.join(ROOT, "weight_gradient_gemm_amd", "csrc")
    subprocess.run([hipcc, "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout + out.stderr
