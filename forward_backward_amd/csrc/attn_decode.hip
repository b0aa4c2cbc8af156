// Split-KV decode for few queries over a long KV cache, bf16, gfx950.
//
// Method: probjax pages, "Attention performance", section "Grouped-query
// attention and decoding". A handful of queries gives the tiled forward too
// few workgroups (its grid is batch x heads x query tiles), so this path
// divides each cache along its keys instead. One workgroup owns a key range
// of one (batch, KV head) and all query rows that read that KV head, stacked
// as one 64-row operand; each range yields a normalised partial output
// with its log-sum-exp, and a second kernel merges the ranges of a row,
// weighting each by its log-sum-exp. The range schedule, row packing and merge
// order are described below.
//
// Packed row p = i * G + g is query i of query head KV_head * G + g. A
// segment is one (batch, KV head, block of 64 packed rows); its n_b =
// ceil(kv_len[b] / 64) key tiles are cut into k_b = min(n_b, ceil(n_b * P / U))
// near-equal ranges, U being the key tiles of all segments and P the split
// budget. Every range therefore holds at most ceil(U / P) tiles whatever the
// KV lengths are, and there are at most P + (number of segments) ranges; the
// schedule is computed on the device from kv_lens by both kernels. Range
// number r (counting segments in order, then ranges within a segment) is
// workgroup r of the split kernel and partial slot r of the workspace.
//
// Split kernel: four waves; wave w handles packed rows 32 * (w % 2) .. + 31
// and key block w / 2 of every 64-key tile. K/V tiles stream through a
// four-stage LDS ring filled by direct global->LDS copies (three tiles in
// flight while one is computed); keys at or past the length are never read.
// The two waves of a row block merge their (max, sum, O) through LDS at the
// end and write the normalised fp32 partial output with its natural-log LSE.
//
// Combine kernel: for each output row the ranges of its segment are merged
// in ascending order with a running maximum: LSE = log sum_r exp(LSE_r),
// O = sum_r exp(LSE_r - LSE) O_r. A row with no valid key gets O = 0 and
// LSE = -inf. With a split budget of 1 every segment is one range: the split
// kernel then writes O (bf16) and the LSE itself, the bits the combine would
// make of a single range, and no combine is launched.
#include <mutex>

#include "../../include/attn.h"
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

template <int D>
struct DecCfg {
  static constexpr int ROWS = kDecodeRows;    // packed rows per workgroup
  static constexpr int BN = kDecodeTileN;     // 64 keys per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BN * D;         // elements of one K or V tile (swizzled, unpadded)
  static constexpr int NST = D > 128 ? 2 : 4;  // LDS ring stages (two 64 KiB stages at head_dim 256)
  // Global->LDS copy instructions per wave per stage (K and V): 1 KiB each.
  static constexpr int COPIES = 2 * TILE * 2 / 1024 / (THREADS / 64);
  // LDS for the final merge: per row block, O (16 * DB floats per lane) plus max and sum.
  static constexpr int MERGE_FLOATS = 2 * 64 * (16 * DB + 2);
  static_assert(MERGE_FLOATS * 4 <= NST * 2 * TILE * 2, "merge area must fit in the ring");
  static_assert(ROWS == 64, "two row blocks of 32");
};

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most min(later, MAXL) tiles of COPIES copies each are in flight.
template <int MAXL, int COPIES>
__device__ __forceinline__ void wait_tile(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      wait_vmem_le<MAXL * COPIES>();
      return;
    }
    wait_tile<MAXL - 1, COPIES>(later);
  } else {
    wait_vmem_le<0>();
  }
}

__device__ __forceinline__ int key_tiles(const DecodeArgs& a, int b) {
  return (clamp_len(a.kv_lens, b, a.Tkv) + kDecodeTileN - 1) / kDecodeTileN;
}

// Ranges of a segment with n tiles out of U in total: min(n, ceil(n * P / U)).
__device__ __forceinline__ unsigned num_ranges(unsigned n, unsigned P, unsigned U) {
  if (n == 0) return 0;
  const unsigned long long num = (unsigned long long)n * P + (U - 1);
  const unsigned long long k = (num >> 32) == 0 ? (unsigned)num / U : num / U;
  return k < n ? (unsigned)k : n;
}

// Inclusive sum over the 64 lanes of a wave (every lane active): sums within
// each 16-lane row by shifts of 1, 2, 4 and 8 lanes, then the last lane of
// rows 0 and 2 added to rows 1 and 3, and the last lane of row 1 to rows 2
// and 3 (row broadcasts). Lanes whose source lies outside the row add 0.
__device__ __forceinline__ unsigned wave_scan(unsigned v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return (unsigned)x;
}
__device__ __forceinline__ unsigned lane_value(unsigned x, int lane) {
  return (unsigned)__builtin_amdgcn_readlane((int)x, lane);
}

// The schedule is evaluated by every wave on its own, lane i taking batch
// b0 + i of each chunk of 64 batches, so its cost grows with B / 64. Counts
// are 32-bit: the host bounds the key tiles of all segments below 2^31.
// U: key tiles of all segments; P: the split budget.
struct Sched {
  unsigned U, P;
};

// Key tiles of batch b0 + lane (0 past the last batch).
__device__ __forceinline__ unsigned chunk_tiles(const DecodeArgs& a, int b0, int lane) {
  const int bb = b0 + lane;
  return bb < a.B ? (unsigned)key_tiles(a, bb) : 0u;
}

// n0: this lane's key tiles in the first chunk of batches.
__device__ __forceinline__ Sched schedule(const DecodeArgs& a, unsigned n0, int lane) {
  unsigned n_tot = lane_value(wave_scan(n0), 63);
  for (int b0 = 64; b0 < a.B; b0 += 64) n_tot += lane_value(wave_scan(chunk_tiles(a, b0, lane)), 63);
  Sched s;
  s.U = n_tot * (unsigned)(a.Hkv * a.num_rblocks);
  s.P = (unsigned)a.budget;
  return s;
}

// Batch b's first slot (ranges of earlier batches) and its ranges per
// segment; b may differ between lanes.
__device__ __forceinline__ void batch_slots(const DecodeArgs& a, const Sched& sc, unsigned n0, int b, int lane,
                                            unsigned& first, unsigned& k) {
  const unsigned S = (unsigned)(a.Hkv * a.num_rblocks);
  unsigned cum = 0;
  first = 0;
  k = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const unsigned kb = num_ranges(b0 == 0 ? n0 : chunk_tiles(a, b0, lane), sc.P, sc.U);
    const unsigned incl = wave_scan(S * kb) + cum;
    const int src = b - b0 < 0 ? 0 : (b - b0 > 63 ? 63 : b - b0);
    const unsigned excl_src = (unsigned)__shfl((int)(incl - S * kb), src, 64);
    const unsigned k_src = (unsigned)__shfl((int)kb, src, 64);
    if (b >= b0 && b < b0 + 64) {
      first = excl_src;
      k = k_src;
    }
    cum = lane_value(incl, 63);
  }
}

// With one range per segment (split budget 1) the split kernel writes the
// output itself, and the workgroups past the ranges write the rows of the
// segments without keys: workgroup `e` past the last range takes the e-th such
// segment (counting batches with no valid key in order, then their segments)
// and writes O = 0 and LSE = -inf for its rows. A grid of 1 + segments
// workgroups leaves one for every segment.
template <int D>
__device__ __forceinline__ void zero_empty_segment(const DecodeArgs& a, unsigned e, unsigned n0, int lane, int tid) {
  const unsigned S = (unsigned)(a.Hkv * a.num_rblocks);
  unsigned cum = 0, local = 0;
  int b = -1;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const unsigned nb = b0 == 0 ? n0 : chunk_tiles(a, b0, lane);
    const unsigned cnt = (b0 + lane < a.B && nb == 0) ? S : 0u;
    const unsigned incl = wave_scan(cnt) + cum;
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(e < incl);
    if (hit != 0) {
      const int L = __builtin_ctzll(hit);
      b = b0 + L;
      local = e - (lane_value(incl, L) - S);
      break;
    }
    cum = lane_value(incl, 63);
  }
  if (b < 0) return;
  b = __builtin_amdgcn_readfirstlane(b);
  local = __builtin_amdgcn_readfirstlane(local);
  const int kh = (int)local / a.num_rblocks;
  const int rbi = (int)local % a.num_rblocks;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int p0 = rbi * kDecodeRows;
  const int np = R - p0 < kDecodeRows ? R - p0 : kDecodeRows;
  for (int idx = tid; idx < np * (D / 4); idx += 256) {
    const int p = p0 + idx / (D / 4), part = idx % (D / 4);
    const int i = p / G, h = kh * G + p % G;
    *(u32x2_t*)((uint16_t*)a.o + (((long)b * a.Tq + i) * a.Hq + h) * D + 4 * part) = u32x2_t{0u, 0u};
    if (a.lse != nullptr && part == 0) a.lse[((long)b * a.Hq + h) * a.Tq + i] = -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(DecodeArgs a) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t ring[C::NST * 2 * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int rb = wave & 1;   // row block
  const int kk = wave >> 1;  // key block within each tile

  // Find this workgroup's range (the same in every wave).
  const unsigned n0 = chunk_tiles(a, 0, lane);
  const Sched sc = schedule(a, n0, lane);
  if (sc.U == 0 && !a.direct) return;
  const unsigned slot = blockIdx.x;
  int b = -1, n = 0, k = 0, local = 0;
  {
    const unsigned S = (unsigned)(a.Hkv * a.num_rblocks);
    unsigned cum = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const unsigned nb = b0 == 0 ? n0 : chunk_tiles(a, b0, lane);
      const unsigned kb = num_ranges(nb, sc.P, sc.U);
      const unsigned incl = wave_scan(S * kb) + cum;
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(slot < incl);
      if (hit != 0) {
        const int L = __builtin_ctzll(hit);
        b = b0 + L;
        n = (int)lane_value(nb, L);
        k = (int)lane_value(kb, L);
        local = (int)(slot - (lane_value(incl, L) - S * (unsigned)k));
        break;
      }
      cum = lane_value(incl, 63);
    }
    if (b < 0) {
      // Past the last range (cum ranges in all).
      if (a.direct) zero_empty_segment<D>(a, slot - cum, n0, lane, tid);
      return;
    }
  }
  b = __builtin_amdgcn_readfirstlane(b);
  n = __builtin_amdgcn_readfirstlane(n);
  k = __builtin_amdgcn_readfirstlane(k);
  local = __builtin_amdgcn_readfirstlane(local);
  const int seg = local / k;       // (KV head, row block) within the batch
  const int j = local % k;         // range within the segment
  const int kh = seg / a.num_rblocks;
  const int rbi = seg % a.num_rblocks;
  const int t_begin = (int)((long)j * n / k);
  const int t_end = (int)((long)(j + 1) * n / k);
  const int ntiles = t_end - t_begin;  // >= 1 since k <= n
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);

  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const long krs = (long)a.Hkv * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  // Q of the 64 packed rows goes to the ring's last stage (free until the
  // loop's first copy) ahead of the first tiles, so that it has landed with
  // tile 0 (through registers it would have waited for every copy issued
  // before it); rows past the packed rows re-read the last one (never stored).
  uint16_t* const q_lds = ring + (C::NST - 1) * 2 * C::TILE;
  static_assert(C::ROWS * D * 2 <= 2 * C::TILE * 2, "Q fits in one stage");
  {
    constexpr int QB = C::ROWS * D * 2 / 1024;  // 1 KiB blocks of Q
#pragma unroll
    for (int i = 0; i < QB / 4; ++i) {
      const int blk = 4 * i + wave;
      const int off = blk * 1024 + lane * 16;    // byte offset in the [ROWS][D] tile
      const int row = off / (2 * D);
      int p = rbi * C::ROWS + row;
      p = p < R ? p : R - 1;
      const uint16_t* src =
          (const uint16_t*)a.q + (((long)b * a.Tq + p / G) * a.Hq + kh * G + p % G) * D + (off % (2 * D)) / 2;
      dma16(src, lds_addr(q_lds) + blk * 1024);
    }
  }

  const TileCopy<D, C::BN, C::THREADS> kvcopy(krs, tid);
  auto issue = [&](int t) {
    uint16_t* st = ring + ((t - t_begin) % C::NST) * 2 * C::TILE;
    // The cache is read once: non-temporal copies (3.8% faster at 16 queries
    // over 16384 keys, B4, 32 query heads over 8 KV heads).
    if ((t + 1) * C::BN <= kvlim) {
      kvcopy.template copy2<C::TILE * 2, true>(st, kb, vb, krs, t * C::BN);
    } else {
      dma_tile<D, C::BN, C::THREADS, false, true>(st, kb, krs, t * C::BN, kvlim, tid);
      dma_tile<D, C::BN, C::THREADS, false, true>(st + C::TILE, vb, krs, t * C::BN, kvlim, tid);
    }
  };
  // Fill the ring before anything else so that the first tiles are on their
  // way while Q is loaded.
#pragma unroll
  for (int i = 0; i < C::NST - 1; ++i)
    if (i < ntiles) issue(t_begin + i);

  const int prow = rbi * C::ROWS + 32 * rb + l32;  // packed row of this lane
  const bool row_ok = prow < R;
  // Q has landed once tile 0 has (or every copy, without tiles); the second
  // barrier keeps the last stage from being refilled before all waves read it.
  if (ntiles > 0)
    wait_tile<C::NST - 2, C::COPIES>(ntiles - 1);
  else
    wait_vmem();
  __syncthreads();
  u32x4_t qf[C::KS];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) qf[t] = lds_read16(q_lds + (32 * rb + l32) * D + 16 * t + 8 * hh);
  __syncthreads();

  f32x16_t o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;

  // Swizzled LDS offsets of this lane's reads; the key block (32 rows) and
  // the 16-row steps keep the swizzle, which depends on the row's low 4 bits.
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int nrm[C::KS], trd[C::DB][2];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh) + 32 * kk * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col) + 32 * kk * D;
    trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col) + 32 * kk * D;
  }

  for (int it = 0; it < ntiles; ++it) {
    // Tile `it` has landed once at most the copies of the (up to NST - 2)
    // later tiles already issued are outstanding; the barrier makes every wave's
    // share visible and retires the stage the next copy overwrites.
    wait_tile<C::NST - 2, C::COPIES>(ntiles - 1 - it);
    __syncthreads();
    if (it + C::NST - 1 < ntiles) issue(t_begin + it + C::NST - 1);

    const uint16_t* kl = ring + (it % C::NST) * 2 * C::TILE;
    const uint16_t* vl = kl + C::TILE;
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::KS; ++t) sc = mfma_bf16(lds_read16(kl + nrm[t]), qf[t], sc);

    const int kblk = (t_begin + it) * C::BN + 32 * kk;
    if (kblk + 32 > kvlim) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kblk + 8 * (r >> 2) + 4 * hh + (r & 3);
        sc[r] = key < kvlim ? sc[r] : -INFINITY;
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = half_max(mt);
    const float mnew = fmaxf(m, mt);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - mref) * c);
    const float nb = -mref * c;
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(sc[r], c, nb));
      sc[r] = p;
      ps += p;
    }
    lsum = lsum * alpha + ps;
    m = mnew;
#pragma unroll
    for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 8 * u;
      const u32x4_t pf = u32x4_t{pack_bf16(sc[r0 + 0], sc[r0 + 1]), pack_bf16(sc[r0 + 2], sc[r0 + 3]),
                                 pack_bf16(sc[r0 + 4], sc[r0 + 5]), pack_bf16(sc[r0 + 6], sc[r0 + 7])};
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2_t lo = lds_read_tr(vl + trd[db][0] + 16 * u * D);
        const u32x2_t hi = lds_read_tr(vl + trd[db][1] + 16 * u * D);
        o[db] = mfma_bf16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
      }
    }
  }

  // Merge the two key blocks of each row block (waves rb and rb + 2). Every
  // copy has completed (the last iteration waited for all of them).
  __syncthreads();
  float* mg = reinterpret_cast<float*>(ring) + rb * 64 * (16 * C::DB + 2);
  if (kk == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) mg[(16 * db + r) * 64 + lane] = o[db][r];
    mg[(16 * C::DB) * 64 + lane] = m;
    mg[(16 * C::DB + 1) * 64 + lane] = lsum;
  }
  __syncthreads();
  if (kk == 0) {
    const float m1 = mg[(16 * C::DB) * 64 + lane];
    const float l1 = mg[(16 * C::DB + 1) * 64 + lane];
    const float mt = fmaxf(m, m1);
    const float mref = (mt == -INFINITY) ? 0.f : mt;
    const float a0 = (m == -INFINITY) ? 0.f : fast_exp2((m - mref) * c);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2((m1 - mref) * c);
    const float ltot = half_sum(lsum * a0 + l1 * a1);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (row_ok && a.direct) {
      // The segment's only range: its normalised partial is the output (the
      // combine would weight it by 1 and divide by 1), bf16, and its LSE.
      const int i = prow / G, h = kh * G + prow % G;
      uint16_t* op = (uint16_t*)a.o + (((long)b * a.Tq + i) * a.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float w[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * g + x;
            w[x] = (o[db][r] * a0 + mg[(16 * db + r) * 64 + lane] * a1) * inv;
          }
          *(u32x2_t*)(op + 32 * db + 8 * g + 4 * hh) = u32x2_t{pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3])};
        }
      if (hh == 0 && a.lse != nullptr)
        a.lse[((long)b * a.Hq + h) * a.Tq + i] = ltot > 0.f ? mt * a.scale + __logf(ltot) : -INFINITY;
    } else if (row_ok) {
      const long prt = (long)slot * C::ROWS + 32 * rb + l32;
      float* po = a.part_o + prt * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t w;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * g + x;
            w[x] = (o[db][r] * a0 + mg[(16 * db + r) * 64 + lane] * a1) * inv;
          }
          *(f32x4_t*)(po + 32 * db + 8 * g + 4 * hh) = w;
        }
      if (hh == 0) a.part_lse[prt] = ltot > 0.f ? mt * a.scale + __logf(ltot) : -INFINITY;
    }
  }
}

// One group of D/4 threads per output row (packed order), 4 head_dim
// elements per thread; the segment's ranges are merged in ascending order.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
  const long nrows = (long)a.B * a.Hkv * R;
  // Threads past the last row stay until the schedule (a whole-wave
  // computation) is done.
  const bool row_ok = gt / TPR < nrows;
  const long row = row_ok ? gt / TPR : nrows - 1;  // ((b * Hkv + kh) * R + p)
  const int part = (int)(gt % TPR);
  const int p = (int)(row % R);
  const int kh = (int)((row / R) % a.Hkv);
  const int b = (int)(row / ((long)R * a.Hkv));
  const int rbi = p / kDecodeRows;

  // First slot and number of ranges of this row's segment (same schedule as
  // the split kernel).
  const int lane = threadIdx.x & 63;
  const unsigned n0 = chunk_tiles(a, 0, lane);
  const Sched sc = schedule(a, n0, lane);
  long first = 0;
  int k = 0;
  if (sc.U > 0) {
    unsigned f = 0, kk = 0;
    batch_slots(a, sc, n0, b, lane, f, kk);
    k = (int)kk;
    first = (long)f + (long)(kh * a.num_rblocks + rbi) * k;
  }
  if (!row_ok) return;

  // Ranges in chunks of 8 whose loads are all issued before any is used
  // (one memory round trip per chunk); running maximum across chunks.
  constexpr int CH = 8;
  const int prow = p % kDecodeRows;
  float lmax = -INFINITY, tot = 0.f;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < k; r0 += CH) {
    float ls[CH];
    f32x4_t v[CH];
#pragma unroll
    for (int x = 0; x < CH; ++x) {
      const bool ok = r0 + x < k;
      const long pr = (first + (ok ? r0 + x : r0)) * kDecodeRows + prow;
      ls[x] = ok ? a.part_lse[pr] : -INFINITY;
      v[x] = ok ? *(const f32x4_t*)(a.part_o + pr * D + 4 * part) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float cm = -INFINITY;
#pragma unroll
    for (int x = 0; x < CH; ++x) cm = fmaxf(cm, ls[x]);
    const float mnew = fmaxf(lmax, cm);
    if (mnew == -INFINITY) continue;
    const float s_old = lmax == -INFINITY ? 0.f : __expf(lmax - mnew);
    acc *= s_old;
    tot *= s_old;
#pragma unroll
    for (int x = 0; x < CH; ++x) {
      const float w = ls[x] == -INFINITY ? 0.f : __expf(ls[x] - mnew);
      acc += w * v[x];
      tot += w;
    }
    lmax = mnew;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int i = p / G, g = p % G;
  const int h = kh * G + g;
  uint16_t* op = (uint16_t*)a.o + (((long)b * a.Tq + i) * a.Hq + h) * D + 4 * part;
  *(u32x2_t*)op = u32x2_t{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  if (a.lse != nullptr && part == 0)
    a.lse[((long)b * a.Hq + h) * a.Tq + i] = tot > 0.f ? lmax + __logf(tot) : -INFINITY;
}

template <int D>
void launch_decode(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const long R = (long)a.Tq * G;
  if (R == 0 || a.B == 0) return;
  if (a.direct) {
    hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3((unsigned)a.num_slots), dim3(256), 0, st, a);
    return;
  }
  if (a.Tkv > 0)
    hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3((unsigned)a.num_slots), dim3(256), 0, st, a);
  const long threads = (long)a.B * a.Hkv * R * (D / 4);
  hipLaunchKernelGGL(attn_decode_combine_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
}

}  // namespace

// Scratch of attn_decode_noalloc: the partial outputs and LSEs of the key
// ranges, in place of a caller's workspace. Each device holds its own copy of
// the array until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device below and only that address is handed to kernels. Calls that
// overlap on one device share the array and race.
static __device__ __align__(256) char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int D, hipStream_t s) {
  if (D == 128)
    launch_decode<128>(a, s);
  else if (D == 256)
    launch_decode<256>(a, s);
  else if (D == 64)
    launch_decode<64>(a, s);
  else
    launch_decode<32>(a, s);
  return hipGetLastError();
}

}  // namespace attn
