"""Bounds model of the tile-copy address arithmetic, compiled for the host from
the device header (no GPU).

The kernels copy [ROWS, D] tiles into LDS with per-lane 32-bit byte offsets
from a wave-uniform 64-bit base (TileCopy), or, for a tile that runs past
the valid rows, with each lane's row clamped below the limit (dma_tile). The
model runs the same helpers (TileGeom, join_halves, key_lo / key_hi /
clamp_len) on the host and checks, for every (head_dim, rows, threads) the
kernels could use:

- every 16-byte chunk of the tile is copied exactly once, to the LDS place
  the readers' swizzle expects;
- the 32-bit lane offsets do not wrap at the largest row stride the API
  accepts (heads * head_dim = 2^22), nor at four times it (at 2^26 they
  would, which shows the check can fail);
- a clamped row stays inside [0, rlim) for rlim down to 1, and a tile is
  copied whole only when all its rows are valid;
- the base address survives its split into two 32-bit halves with bit 31 of
  either half set (the signed widening that once faulted on the device fails
  this check);
- over edge shapes (ragged lengths, KV lengths -3, 0, 1, T - 1, T, T + 50,
  causal and window masks), the key range of every query tile lies inside
  the KV length, so every element a tile copy reads is inside its tensor.
"""

import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "forward_backward_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <vector>
#include "attn_device.hpp"

static long bad = 0, checks = 0;
#define CHECK(cond, ...) do { ++checks; if (!(cond)) { ++bad; if (bad < 20) std::printf(__VA_ARGS__); } } while (0)

template <int D, int ROWS, int THREADS>
void geometry() {
  using G = attn::TileGeom<D, ROWS, THREADS>;
  std::vector<int> lds(ROWS * D / 8, 0), src(ROWS * D / 8, 0);
  for (int wave = 0; wave < G::WAVES; ++wave)
    for (int i = 0; i < G::ITERS; ++i)
      for (int lane = 0; lane < 64; ++lane) {
        const int r = G::row(i, wave, lane);
        const int c = G::chunk(r, lane);
        CHECK(r >= 0 && r < ROWS && c >= 0 && c < D / 8, "D%d R%d T%d: row %d chunk %d\n", D, ROWS, THREADS, r, c);
        const int dst = G::block(i, wave) * 1024 + 16 * lane;  // LDS byte of the lane's 16 bytes
        CHECK(dst >= 0 && dst + 16 <= ROWS * D * 2, "D%d: LDS byte %d outside the tile\n", D, dst);
        // the readers find logical (r, 8 c) at swz_off
        CHECK(2 * attn::swz_off<D>(r, 8 * c) == dst, "D%d R%d T%d: swizzle mismatch at row %d chunk %d\n", D, ROWS,
              THREADS, r, c);
        lds[dst / 16]++;
        src[r * (D / 8) + c]++;
      }
  for (size_t k = 0; k < lds.size(); ++k) {
    CHECK(lds[k] == 1, "D%d R%d T%d: LDS chunk %zu written %d times\n", D, ROWS, THREADS, k, lds[k]);
    CHECK(src[k] == 1, "D%d R%d T%d: source chunk %zu read %d times\n", D, ROWS, THREADS, k, src[k]);
  }
  // 32-bit lane offsets at the largest row stride the API takes, and past it.
  for (long rs : {(long)D, 1L << 22, 1L << 24, 1L << 26}) {
    bool wraps = false;
    for (int wave = 0; wave < G::WAVES; ++wave)
      for (int i = 0; i < G::ITERS; ++i)
        for (int lane = 0; lane < 64; ++lane) {
          const int r = G::row(i, wave, lane);
          const long exact = G::elem(r, r, lane, rs) * 2;
          if ((long)G::voff(i, wave, lane, rs) != exact) wraps = true;
          CHECK(exact + 16 <= ((long)ROWS - 1) * rs * 2 + 2 * D, "D%d: lane offset past the tile's rows\n", D);
        }
    // No wrap up to four times the API's bound; at 2^26 a 64-row tile's offsets do wrap (the check can fail).
    if (rs <= (1L << 24)) CHECK(!wraps, "D%d R%d: 32-bit lane offset wraps at row stride %ld\n", D, ROWS, rs);
    if (rs == (1L << 26) && ROWS >= 64) CHECK(wraps, "D%d R%d: expected a wrap at row stride 2^26\n", D, ROWS);
  }
  // Clamped rows of partial tiles.
  for (int rlim : {1, 2, 3, ROWS - 1, ROWS, ROWS + 1, 1000})
    for (int r0 : {0, 1, ROWS / 2, ROWS, 999})
      for (int r = 0; r < ROWS; ++r) {
        const int gr = G::clamp_row(r0, r, rlim);
        CHECK(gr >= 0 && gr < rlim, "clamp r0 %d r %d rlim %d -> %d\n", r0, r, rlim, gr);
        if (r0 + ROWS <= rlim) CHECK(gr == r0 + r, "a whole tile's rows must not be clamped\n");
      }
}

void halves() {
  const uint64_t addrs[] = {0x0000'7f00'8000'0000ull, 0x0000'7fff'ffff'fff0ull, 0x0000'0001'8000'0010ull,
                            0x0000'7f12'3456'7890ull, 0x0000'0000'ffff'ff00ull, 0x8000'0000'8000'0000ull};
  for (uint64_t a : addrs) {
    // readfirstlane hands each half back as a signed int
    const int32_t lo = (int32_t)(uint32_t)a, hi = (int32_t)(uint32_t)(a >> 32);
    CHECK(attn::join_halves((uint32_t)lo, (uint32_t)hi) == a, "address %llx not rebuilt\n", (unsigned long long)a);
    const uint64_t signed_widening = ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(int64_t)lo;
    if ((uint32_t)a & 0x80000000u)
      CHECK(signed_widening != a, "the signed widening should have corrupted %llx\n", (unsigned long long)a);
  }
}

// Key ranges of query tiles over edge shapes: what the kernels copy.
void key_ranges() {
  const int Ts[] = {1, 63, 64, 65, 127, 129, 333, 1000};
  for (int T : Ts)
    for (int kvl : {-3, 0, 1, 2, T - 1, T, T + 50})
      for (int causal = 0; causal < 2; ++causal)
        for (int w = 0; w < 4; ++w) {
          const int left = w == 1 ? 0 : (w == 2 ? 17 : -1), right = w == 3 ? 5 : (w == 1 ? 0 : -1);
          const int32_t lens[1] = {kvl};
          const int kvlim = attn::clamp_len(lens, 0, T);
          CHECK(kvlim >= 0 && kvlim <= T, "clamp_len %d of %d -> %d\n", kvl, T, kvlim);
          for (int BM : {32, 64, 128})
            for (int q0 = 0; q0 < T; q0 += BM) {
              const int q1 = q0 + BM - 1 < T ? q0 + BM - 1 : T - 1;
              const int lo = attn::key_lo(q0, left);
              const int hi = attn::key_hi(q1, kvlim, causal, right);  // kv_end - 1 of the tile
              if (hi < lo) continue;  // no tile is copied
              CHECK(lo >= 0 && hi < kvlim && hi < T, "T %d kv %d causal %d window %d,%d: keys [%d, %d]\n", T, kvl,
                    causal, left, right, lo, hi);
              for (int i = q0; i <= q1; ++i) {
                const int rl = attn::key_lo(i, left), rh = attn::key_hi(i, kvlim, causal, right);
                if (rh >= rl) CHECK(rl >= lo && rh <= hi, "row %d's keys outside its tile's range\n", i);
              }
            }
        }
}

int main() {
  geometry<32, 64, 256>();  geometry<32, 128, 512>(); geometry<32, 128, 256>();
  geometry<64, 64, 256>();  geometry<64, 64, 512>();  geometry<64, 128, 256>(); geometry<64, 32, 256>();
  geometry<128, 64, 256>(); geometry<128, 64, 512>(); geometry<128, 128, 512>(); geometry<128, 32, 256>();
  geometry<256, 32, 256>(); geometry<256, 64, 256>(); geometry<256, 32, 512>(); geometry<256, 64, 512>();
  halves();
  key_ranges();
  std::printf("checks %ld bad %ld\n", checks, bad);
  return bad != 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_tile_copy_addresses_stay_in_bounds(tmp_path):
    src = tmp_path / "bounds.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "bounds"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout[-3000:])
    assert run.returncode == 0, run.stdout[-3000:]
    assert "bad 0" in run.stdout


def test_api_bounds_the_row_stride_that_keeps_lane_offsets_in_32_bits():
    """heads * head_dim up to 2^22 is accepted; one head more is refused before any launch."""
    from forward_backward_amd import attn
    if not os.path.exists(attn.LIB_PATH):
        pytest.skip("libattn.so not built")
    L = attn.lib()
    for D in (32, 64, 128, 256):
        for op in (attn.OP_FWD, attn.OP_BWD, attn.OP_DECODE):
            ok = attn.make_params(1, 1, 1, (1 << 22) // D, 1, D)
            assert L.attn_validate(ctypes.byref(ok), op) == attn.ATTN_OK
            over = attn.make_params(1, 1, 1, (1 << 22) // D + 1, 1, D)
            assert L.attn_validate(ctypes.byref(over), op) == attn.ATTN_ERR_UNSUPPORTED
            kv_over = attn.make_params(1, 1, 1, 2 * ((1 << 22) // D + 1), (1 << 22) // D + 1, D)
            assert L.attn_validate(ctypes.byref(kv_over), op) == attn.ATTN_ERR_UNSUPPORTED
