"""The debug build's address test (dbg_in_ranges of attn_internal.h, compiled
for the host): an access of `bytes` bytes at `addr` passes only when it lies
wholly inside one registered range, including at the ends of the address
space where addr + bytes would wrap."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "forward_backward_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "attn_internal.h"
using attn::DbgRange;
using attn::dbg_in_ranges;
int main() {
  const unsigned long long top = ~0ull;
  const DbgRange r[3] = {{1000, 1064}, {4096, 8192}, {top - 64, top}};
  struct T { unsigned long long addr; unsigned bytes; int n; bool want; } t[] = {
      {1000, 16, 3, true},      // first bytes of a range
      {1048, 16, 3, true},      // last 16 bytes of a range
      {1049, 16, 3, false},     // one byte past its end
      {999, 16, 3, false},      // one byte before its start
      {1064, 1, 3, false},      // the end itself
      {1060, 4, 3, true},
      {5000, 16, 3, true},      // second range
      {2000, 16, 3, false},     // between ranges
      {1056, 16, 3, false},     // straddles the end of the first range
      {top - 16, 16, 3, true},  // ends exactly at the top range's end
      {top - 8, 16, 3, false},  // would wrap past the top
      {top, 16, 3, false},
      {1000, 16, 0, false},     // empty table
      {5000, 16, 1, false},     // range 2 not in a table of one
  };
  int bad = 0;
  for (const T& c : t) {
    const bool got = dbg_in_ranges(c.addr, c.bytes, r, c.n);
    if (got != c.want) {
      ++bad;
      std::printf("FAIL addr %llu bytes %u n %d: got %d\n", c.addr, c.bytes, c.n, (int)got);
    }
  }
  std::printf("bad %d\n", bad);
  return bad != 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_address_ranges(tmp_path):
    src = tmp_path / "ranges.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "ranges"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(run.stdout)
    assert run.returncode == 0 and "bad 0" in run.stdout, run.stdout
