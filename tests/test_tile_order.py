"""The workgroup order of the tiled kernels (xcd_remap then tile_order, from
the device header, compiled for the host): for every grid shape it must be a
bijection from workgroup ids onto (unit, tile) pairs, or tiles would be
computed twice or not at all. Also checks the two properties the order is
for: with causal masking each XCD's share issues tile ranks in non-decreasing
order (longest first), and when the units come in groups of `together` whose
count is a multiple of 8, a group's tiles stay on one XCD while consecutive
groups go to different XCDs."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "forward_backward_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "attn_device.hpp"
int main() {
  long bad = 0, cases = 0;
  const int units_list[] = {1, 2, 3, 5, 7, 8, 9, 16, 24, 31, 32, 33, 64, 96, 128, 256, 512};
  const int tiles_list[] = {1, 2, 3, 5, 8, 17, 32, 64};
  const int together_list[] = {1, 2, 4, 8, 16};
  for (int nunits : units_list)
    for (int ntiles : tiles_list)
      for (int lf = 0; lf < 2; ++lf)
        for (int tog : together_list) {
          const int n = nunits * ntiles;
          std::vector<int> seen(n, 0), xcd_of_unit(nunits, -1);
          int last_rank[8];
          for (int x = 0; x < 8; ++x) last_rank[x] = -1;
          bool ok = true;
          for (int b = 0; b < n; ++b) {  // hardware ids in dispatch order
            int u, t;
            attn::tile_order(attn::xcd_remap(b, n), ntiles, nunits, lf != 0, u, t, tog);
            if (u < 0 || u >= nunits || t < 0 || t >= ntiles) { ok = false; break; }
            seen[u * ntiles + t]++;
            const int x = b % 8;
            if (lf && nunits % 8 == 0) {
              if (t < last_rank[x]) ok = false;  // longest first within each XCD's share
              last_rank[x] = t;
            }
            if (nunits % tog == 0 && (nunits / tog) % 8 == 0) {
              const int g = u / tog;
              if (xcd_of_unit[g] < 0) xcd_of_unit[g] = x;
              else if (xcd_of_unit[g] != x) ok = false;  // a group stays on one XCD
            }
          }
          for (int i = 0; i < n && ok; ++i) ok = seen[i] == 1;
          if (ok && nunits % tog == 0 && (nunits / tog) % 8 == 0)
            for (int g = 0; g + 1 < nunits / tog; ++g)
              if (xcd_of_unit[g] == xcd_of_unit[g + 1]) ok = false;  // consecutive groups spread
          ++cases;
          if (!ok) {
            ++bad;
            std::printf("FAIL units %d tiles %d longest_first %d together %d\n", nunits, ntiles, lf, tog);
          }
        }
  std::printf("cases %ld bad %ld\n", cases, bad);
  return bad != 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_grid_order_is_a_bijection_with_its_placement_properties(tmp_path):
    src = tmp_path / "order.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "order"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout[-2000:])
    assert run.returncode == 0, run.stdout[-2000:]
    assert "bad 0" in run.stdout
