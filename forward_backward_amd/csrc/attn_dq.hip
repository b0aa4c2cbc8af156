// dQ pass of the backward, bf16, gfx950 (the other passes are in
// attn_bwd.hip): per (batch, head, 128-row query tile), for each 64-key tile
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T
// with P recomputed from the forward's LSE (probjax pages, "Attention
// performance", section "When to use which": the two-pass kernels give
// bitwise reproducible gradients). A file of its own so that the build can
// schedule it with its own options (see build.py).
#include <type_traits>

#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

// Single-pair dQ kernel (head_dim 32 and 256; 64 and 128 run the wave-pair
// kernel further below): four waves of 32 query rows, each processing both
// 32-key blocks of every 64-key tile.

template <int D>
struct DqCfg {
  static constexpr int BM = kBwdBlockM;     // 128 query rows, 32 per wave
  static constexpr int BN = 64;             // keys per tile (2 blocks of 32)
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BN * D;       // K and V tiles: swizzled, unpadded
};

template <int D>
__global__ __launch_bounds__(256) void attn_dq_bf16_kernel(BwdArgs a) {
  using C = DqCfg<D>;
  // Two pipeline stages of the K and V tiles in one array (one per-lane
  // offset plus a constant addresses every stage).
  __shared__ __attribute__((aligned(16))) uint16_t tiles[4 * C::TILE];
  uint16_t* const k_s0 = tiles;
  uint16_t* const v_s0 = tiles + C::TILE;
  uint16_t* const k_s1 = tiles + 2 * C::TILE;
  uint16_t* const v_s1 = tiles + 3 * C::TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int nqt = (a.Tq + C::BM - 1) / C::BM;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, rank;
  tile_order(bid, nqt, a.B * a.Hq, a.causal, bh, rank, a.Hq / a.Hkv);
  const int qt = nqt - 1 - rank;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kh = h / (a.Hq / a.Hkv);
  const int q0 = qt * C::BM;

  const long qrs = (long)a.Hq * D;
  const long krs = (long)a.Hkv * D;
  const long qoff = ((long)b * a.Tq * a.Hq + h) * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  // Keys any row of the tile sees: [key_lo(first row), key_hi(last row)].
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;  // first key tile
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  const int qrow = q0 + 32 * wave + l32;
  const bool row_ok = qrow < a.Tq;
  u32x4_t qf[C::KS], gf[C::KS];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    qf[t] = row_ok ? gload16((const uint16_t*)a.q + qoff + qrow * qrs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
    gf[t] = row_ok ? gload16((const uint16_t*)a.dout + qoff + qrow * qrs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
  }
  const long stat = ((long)b * a.Hq + h) * a.Tq + qrow;
  const float lse2 = row_ok ? a.lse2[stat] : INFINITY;
  const float dlt = row_ok ? a.delta[stat] : 0.f;
  const float c = a.scale_log2;

  f32x16_t acc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) acc[i] = f32x16_t{};

  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wave_min_row = q0 + 32 * wave;
  // Visible keys of this lane's row, and the keys every row of the wave sees.
  const int row_lo = key_lo(qrow, a.win_left);
  const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
  const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
  const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);
  int nrm[C::KS], trd[C::DB][2];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col);
    trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col);
  }

  auto issue = [&](int it, uint16_t* ks, uint16_t* vs) {
    const int k0 = (j0 + it) * C::BN;
    dma_tile<D, C::BN, C::THREADS, true>(ks, kb, krs, k0, kv_end, tid);
    dma_tile<D, C::BN, C::THREADS, true>(vs, vb, krs, k0, kv_end, tid);
  };

  // Row fragments of key block j (32 keys) for S^T = K Q^T and dP^T = V dO^T.
  auto read_kv = [&](const uint16_t* kl, const uint16_t* vl, int j, u32x4_t* ka, u32x4_t* va) {
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
      ka[t] = lds_read16(kl + 32 * j * D + nrm[t]);
      va[t] = lds_read16(vl + 32 * j * D + nrm[t]);
    }
  };
  // Transposed K fragments of key block j for dQ^T += K^T dS^T.
  auto read_kt = [&](const uint16_t* kl, int j, u32x2_t (*kt)[C::DB][2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        kt[u][db][0] = lds_read_tr(kl + (32 * j + 16 * u) * D + trd[db][0]);
        kt[u][db][1] = lds_read_tr(kl + (32 * j + 16 * u) * D + trd[db][1]);
      }
  };
  auto sdp = [&](const u32x4_t* ka, const u32x4_t* va, f32x16_t& s, f32x16_t& dp) {
    s = f32x16_t{};
    dp = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
      s = mfma_bf16(ka[t], qf[t], s);
      dp = mfma_bf16(va[t], gf[t], dp);
    }
  };
  // dS^T of key block j as bf16 B operands; MASK selects the element-wise mask.
  auto softmax = [&](auto mask_tag, int kblk0, const f32x16_t& s, const f32x16_t& dp, u32x4_t* dsb) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float dsv[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int r = 8 * u + x;
        float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
        if constexpr (MASK) {
          const int kk = kblk0 + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = (kk >= row_lo) & (kk <= row_hi);
          p = ok ? p : 0.f;
        }
        dsv[x] = p * (dp[r] - dlt);
      }
      dsb[u] = u32x4_t{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                       pack_bf16(dsv[6], dsv[7])};
    }
  };
  auto dq_mfma = [&](u32x2_t (*kt)[C::DB][2], const u32x4_t* dsb) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        acc[db] = mfma_bf16(u32x4_t{kt[u][db][0][0], kt[u][db][0][1], kt[u][db][1][0], kt[u][db][1][1]}, dsb[u],
                            acc[db]);
  };

  // One 64-key tile as a two-block software pipeline: the S/dP products of
  // block 1 are interleaved with the softmax of block 0, so that the vector
  // work runs while the matrix core is busy.
  auto compute = [&](int it, const uint16_t* kl, const uint16_t* vl, auto&& issue_next) {
    const int k0 = (j0 + it) * C::BN;
    const bool mask_tile = (k0 < wave_all_lo) || (k0 + C::BN - 1 > wave_all_hi);
    auto body = [&](auto mask_tag) {
      u32x4_t ka[C::KS], va[C::KS];
      f32x16_t s0, dp0, s1, dp1;
      u32x2_t kt[2][C::DB][2];
      u32x4_t dsb[2];
      read_kv(kl, vl, 0, ka, va);
      sdp(ka, va, s0, dp0);
      read_kv(kl, vl, 1, ka, va);
      read_kt(kl, 0, kt);
      __builtin_amdgcn_sched_barrier(0);
      // The next tile's loads start after the first block's transpose reads
      // (transpose reads issued while they are in flight wait for them).
      issue_next();
      sdp(ka, va, s1, dp1);
      softmax(mask_tag, k0, s0, dp0, dsb);
#pragma unroll
      for (int i = 0; i < 2 * C::KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then vector ALU work
      }
      __builtin_amdgcn_sched_barrier(0);
      dq_mfma(kt, dsb);
      read_kt(kl, 1, kt);
      softmax(mask_tag, k0 + 32, s1, dp1, dsb);
      dq_mfma(kt, dsb);
    };
    // head_dim 256: a block's K/V fragments alone would take 128 registers,
    // so they stream through a two-deep ring and the transposed K fragments
    // are read per 16-key half; one block at a time.
    auto body_wide = [&](auto mask_tag) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint16_t* krow = kl + 32 * j * D;
        const uint16_t* vrow = vl + 32 * j * D;
        u32x4_t ka[2], va[2];
        ka[0] = lds_read16(krow + nrm[0]);
        va[0] = lds_read16(vrow + nrm[0]);
        ka[1] = lds_read16(krow + nrm[1]);
        va[1] = lds_read16(vrow + nrm[1]);
        f32x16_t sj = f32x16_t{}, dpj = f32x16_t{};
#pragma unroll
        for (int t = 0; t < C::KS; ++t) {
          sj = mfma_bf16(ka[t & 1], qf[t], sj);
          dpj = mfma_bf16(va[t & 1], gf[t], dpj);
          if (t + 2 < C::KS) {
            ka[t & 1] = lds_read16(krow + nrm[t + 2]);
            va[t & 1] = lds_read16(vrow + nrm[t + 2]);
          }
        }
        u32x4_t dsb[2];
        softmax(mask_tag, k0 + 32 * j, sj, dpj, dsb);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x2_t kt[C::DB][2];
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            kt[db][0] = lds_read_tr(krow + 16 * u * D + trd[db][0]);
            kt[db][1] = lds_read_tr(krow + 16 * u * D + trd[db][1]);
          }
          if (j == 0 && u == 0) issue_next();
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
            acc[db] = mfma_bf16(u32x4_t{kt[db][0][0], kt[db][0][1], kt[db][1][0], kt[db][1][1]}, dsb[u], acc[db]);
        }
      }
    };
    if constexpr (D > 128) {
      if (mask_tile)
        body_wide(std::true_type{});
      else
        body_wide(std::false_type{});
    } else {
      if (mask_tile)
        body(std::true_type{});
      else
        body(std::false_type{});
    }
  };

  auto step = [&](int it, uint16_t* nk, uint16_t* nv, const uint16_t* ck, const uint16_t* cv) {
    compute(it, ck, cv, [&]() {
      if (it + 1 < ntiles) issue(it + 1, nk, nv);
    });
    wait_vmem();
    __syncthreads();
  };

  if (ntiles > 0) issue(0, k_s0, v_s0);
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < ntiles; it += 2) {
    step(it, k_s1, v_s1, k_s0, v_s0);
    if (it + 1 >= ntiles) break;
    step(it + 1, k_s0, v_s0, k_s1, v_s1);
  }

  if (row_ok) {
    uint16_t* dqp = (uint16_t*)a.dq + qoff + qrow * qrs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        *(u32x2_t*)(dqp + d) = u32x2_t{pack_bf16(acc[db][4 * g] * a.scale, acc[db][4 * g + 1] * a.scale),
                                       pack_bf16(acc[db][4 * g + 2] * a.scale, acc[db][4 * g + 3] * a.scale)};
      }
  }
}

// dQ with the two 32-key blocks of each tile split over a pair of waves that
// share the same 32 query rows: wave w takes block 0 and wave w + 4 block 1 of
// every tile, each with its own dQ^T partial, and the pair adds the two
// partials in that order at the end (deterministic). Without the two-block
// software pipeline of the single-pair kernel a wave needs well under 256
// registers, so two waves share each SIMD. Per block: S^T = K Q^T and
// dP^T = V dO^T (lane = query row), dS^T = P (dP - D), dQ^T += K^T dS^T.
template <int D>
struct DqPairCfg {
  static constexpr int BM = kBwdBlockM;     // 128 query rows, 32 per wave pair
  static constexpr int BN = 64;             // keys per tile (one 32-key block per wave of a pair)
  static constexpr int THREADS = 512;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int R = 2;               // depth of the fragment read-ahead
  // Head_dim 64: two tiles per step and barrier (four stages: two read, two in
  // flight); head_dim 128: one tile per step, copies two tiles ahead (three
  // stages; the two-tile step measured 2% slower there at 256 registers).
  static constexpr bool TWO = D <= 64;
  static constexpr int NST = TWO ? 4 : 3;
  static constexpr int TILE = BN * D;
};

template <int D>
__global__ __launch_bounds__(512) void attn_dq_pair_kernel(BwdArgs a) {
  using C = DqPairCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2 * C::NST * C::TILE];  // stage s: K at 2s, V at 2s + 1
  __shared__ __attribute__((aligned(16))) uint16_t rows_x[2 * C::BM * D];         // the tile's dO rows, then O rows
  static_assert(2 * C::NST * C::TILE * 2 >= 4 * 64 * 16 * C::DB * 4, "the partial hand-over reuses the tiles");
  static_assert(C::NST >= 3 && 2 * C::TILE == C::BM * D, "the tile's Q rows fill ring stage 2");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2;               // key block of each tile
  const int w4 = wave & 3;                  // row block
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int nqt = (a.Tq + C::BM - 1) / C::BM;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, rank;
  tile_order(bid, nqt, a.B * a.Hq, a.causal, bh, rank, a.Hq / a.Hkv);
  const int qt = nqt - 1 - rank;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kh = h / (a.Hq / a.Hkv);
  const int q0 = qt * C::BM;

  const long qrs = (long)a.Hq * D;
  const long krs = (long)a.Hkv * D;
  const long qoff = ((long)b * a.Tq * a.Hq + h) * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  // Copies of tile `it` into stage `st`. They go through inline assembly, which
  // the compiler does not see writing LDS: the waits before each step's
  // barrier order them (CP copy instructions per wave and tile, full or partial).
  const TileCopy<D, C::BN, C::THREADS> kvcopy(krs, tid);
  [[maybe_unused]] constexpr int CP = 2 * TileCopy<D, C::BN, C::THREADS>::ITERS;
  auto issue = [&](int it, int st) {
    uint16_t* ks = tiles + st * 2 * C::TILE;
    const int k0 = (j0 + it) * C::BN;
    if (k0 + C::BN <= kv_end) {
      // One copy at a time here: one batch for both tiles measured 1% slower.
      kvcopy.copy(ks, kb, krs, k0);
      kvcopy.copy(ks + C::TILE, vb, krs, k0);
    } else {
      dma_tile<D, C::BN, C::THREADS>(ks, kb, krs, k0, kv_end, tid);
      dma_tile<D, C::BN, C::THREADS>(ks + C::TILE, vb, krs, k0, kv_end, tid);
    }
  };

  // The tile's Q, dO and O rows stream into LDS together with the first two
  // K/V tiles, so that the start of a tile costs one memory round trip: Q into
  // ring stage 2 (refilled only after the loop's first barrier), dO and O into
  // rows_x, by the same coalesced 1 KiB copies in the swizzled tile layout as
  // the K/V tiles. (Loaded straight into registers, each 16-byte fragment load
  // touched 32 rows per instruction, and the rows took about 9 us per tile to
  // arrive under load.) Rows past Tq re-read the last row; their lanes are
  // zeroed below.
  uint16_t* const q_lds = tiles + 2 * 2 * C::TILE;
  {
    const TileCopy<D, C::BM, C::THREADS> rcopy(qrs, tid);
    auto rows = [&](uint16_t* dst, const void* src) {
      const uint16_t* g = (const uint16_t*)src + qoff;
      if (q0 + C::BM <= a.Tq)
        rcopy.copy1(dst, g, qrs, q0);
      else
        dma_tile<D, C::BM, C::THREADS>(dst, g, qrs, q0, a.Tq, tid);
    };
    rows(q_lds, a.q);
    rows(rows_x, a.dout);
    if (a.dq_stats) rows(rows_x + C::BM * D, a.o);
  }
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);

  const int qrow = q0 + 32 * w4 + l32;
  const bool row_ok = qrow < a.Tq;
  const long stat = ((long)b * a.Hq + h) * a.Tq + qrow;
  // The rows' statistics (compiler-visible loads, issued after the copies: the
  // wait for them below is a wait for everything, rows and first tiles alike).
  float lse_in = 0.f, lse2_in = INFINITY, dlt_in = 0.f;
  if (row_ok) {
    if (a.dq_stats) {
      lse_in = a.lse[stat];
    } else {
      lse2_in = a.lse2[stat];
      dlt_in = a.delta[stat];
    }
  }
  wait_vmem();
  __syncthreads();
  u32x4_t qf[C::KS], gf[C::KS];
  const int lrow = 32 * w4 + l32;  // the lane's row in the tile
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    const int off = swz_off<D>(lrow, 16 * t + 8 * hh);
    qf[t] = row_ok ? lds_read16(q_lds + off) : u32x4_t{0, 0, 0, 0};
    gf[t] = row_ok ? lds_read16(rows_x + off) : u32x4_t{0, 0, 0, 0};
  }
  float lse2, dlt;
  if (a.dq_stats) {
    // D of the lane's row from its O and dO fragments (the pre-kernel's
    // chain, so the same bits), and the statistics the dK/dV pass reads:
    // written once per row, by the block-0 wave of the pair.
    u32x4_t of[C::KS];
#pragma unroll
    for (int t = 0; t < C::KS; ++t)
      of[t] = row_ok ? lds_read16(rows_x + C::BM * D + swz_off<D>(lrow, 16 * t + 8 * hh)) : u32x4_t{0, 0, 0, 0};
    const float dsum = half_sum(row_dot_half<C::KS>(of, gf));
    const float lse = lse_in;
    if (row_ok && half == 0 && hh == 0) write_row_stats(a, stat, dsum, lse);
    lse2 = row_ok ? lse * 1.4426950408889634f : INFINITY;
    dlt = row_ok ? dsum : 0.f;
    if (blockIdx.x == 0 && tid < kBwdQueueWords && a.queue != nullptr) a.queue[tid] = 0u;
  } else {
    lse2 = lse2_in;
    dlt = dlt_in;
  }
  const float c = a.scale_log2;

  f32x16_t acc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) acc[i] = f32x16_t{};

  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wave_min_row = q0 + 32 * w4;
  const int row_lo = key_lo(qrow, a.win_left);
  const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
  const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
  const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);
  // Lane offsets (elements) inside a stage, for this wave's key block.
  int nrm[C::KS], trd[C::DB][2];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh) + 32 * half * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col) + 32 * half * D;
    trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col) + 32 * half * D;
  }

  // One 32-key block: S^T, dP^T, the masked dS^T, then dQ^T += K^T dS^T. The
  // element-wise mask is a select-only fix-up under a uniform branch (a
  // branch between two whole block bodies made the register allocator copy
  // the accumulators).
  auto block = [&](bool mask, const uint16_t* kl, const uint16_t* vl, int kblk0) {
    u32x4_t ka[C::R], va[C::R];
#pragma unroll
    for (int m = 0; m < C::R; ++m) {
      ka[m] = lds_read16(kl + nrm[m]);
      va[m] = lds_read16(vl + nrm[m]);
    }
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
    // At head_dim 64 the row products run at raised wave priority: the wave
    // that gets to them first keeps the matrix core while its partner works
    // through its softmax (3-4% faster at B4 H8 T4096; slower at 128).
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
      s = mfma_bf16(ka[t % C::R], qf[t], s);
      dp = mfma_bf16(va[t % C::R], gf[t], dp);
      if (t + C::R < C::KS) {
        ka[t % C::R] = lds_read16(kl + nrm[t + C::R]);
        va[t % C::R] = lds_read16(vl + nrm[t + C::R]);
      }
    }
    if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
    u32x2_t kt[1][C::DB][2];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      kt[0][db][0] = lds_read_tr(kl + trd[db][0]);
      kt[0][db][1] = lds_read_tr(kl + trd[db][1]);
    }
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
    if (mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kblk0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        pv[r] = ((key >= row_lo) & (key <= row_hi)) ? pv[r] : 0.f;
      }
    }
    u32x4_t dsb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float dsv[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) dsv[x] = pv[8 * u + x] * (dp[8 * u + x] - dlt);
      dsb[u] = u32x4_t{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                       pack_bf16(dsv[6], dsv[7])};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          kt[0][db][0] = lds_read_tr(kl + 16 * D + trd[db][0]);
          kt[0][db][1] = lds_read_tr(kl + 16 * D + trd[db][1]);
        }
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        acc[db] = mfma_bf16(u32x4_t{kt[0][db][0][0], kt[0][db][0][1], kt[0][db][1][0], kt[0][db][1][1]}, dsb[u],
                            acc[db]);
    }
  };

  if constexpr (C::TWO) {
    // Two tiles per step and one barrier: tile t sits in stage t % 4; the
    // copies of the next step's two tiles start after the step's barrier, once
    // every wave is done with the two tiles before, and land before its end.
    // The first tiles landed in the prologue.
    for (int it = 0; it < ntiles; it += 2) {
      __syncthreads();  // tiles it, it + 1 visible; tiles it - 2, it - 1 read by every wave
      if (it + 2 < ntiles) issue(it + 2, (it + 2) % C::NST);
      if (it + 3 < ntiles) issue(it + 3, (it + 3) % C::NST);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (u == 1 && it + 1 >= ntiles) break;
        const uint16_t* kl = tiles + ((it + u) % C::NST) * 2 * C::TILE;
        const int kblk0 = (j0 + it + u) * C::BN + 32 * half;
        const bool mask = (kblk0 < wave_all_lo) || (kblk0 + 31 > wave_all_hi);
        block(mask, kl, kl + C::TILE, kblk0);
      }
      wait_vmem();  // the next step's tiles have landed
    }
  } else {
    // The first tiles landed in the prologue.
    int st_rd = 0, st_wr = 2;
    for (int it = 0; it < ntiles; ++it) {
      // Tile it has landed once at most the copies of tile it + 1 are in flight.
      if (it + 1 < ntiles)
        wait_vmcnt<CP>();
      else
        wait_vmem();
      __syncthreads();  // tile it visible; every wave is done with tile it - 1, whose stage is refilled next
      if (it + 2 < ntiles) issue(it + 2, st_wr);
      const uint16_t* kl = tiles + st_rd * 2 * C::TILE;
      const int k0 = (j0 + it) * C::BN;
      const int kblk0 = k0 + 32 * half;
      const bool mask = (kblk0 < wave_all_lo) || (kblk0 + 31 > wave_all_hi);
      block(mask, kl, kl + C::TILE, kblk0);
      st_rd = st_rd + 1 == C::NST ? 0 : st_rd + 1;
      st_wr = st_wr + 1 == C::NST ? 0 : st_wr + 1;
    }
  }

  // The pair's partials: block-1 waves hand theirs over through LDS, block-0
  // waves add them (block 0 + block 1) and store.
  __syncthreads();
  float* xf = reinterpret_cast<float*>(tiles) + w4 * (16 * C::DB * 64);
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xf[(16 * db + r) * 64 + lane] = acc[db][r];
  }
  __syncthreads();
  // The sums go to a bf16 tile in LDS (rows_x, free by now; the swizzled
  // layout of the copies), and from there to dQ in whole 256-byte rows, 16
  // bytes per lane: stored straight from the fragments, each instruction would
  // write 8 bytes to each of 32 rows.
  if (half == 0) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * g + x;
          v[x] = (acc[db][r] + xf[(16 * db + r) * 64 + lane]) * a.scale;
        }
        const int d = 32 * db + 8 * g + 4 * hh;
        *(u32x2_t*)(rows_x + swz_off<D>(lrow, d)) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      }
  }
  __syncthreads();
  {
    using Gm = TileGeom<D, C::BM, C::THREADS>;
    uint16_t* const dqb = (uint16_t*)a.dq + qoff;
#pragma unroll
    for (int i = 0; i < Gm::ITERS; ++i) {
      const int r = Gm::row(i, wave, lane);
      if (q0 + r < a.Tq)
        *(u32x4_t*)(dqb + Gm::elem(q0 + r, r, lane, qrs)) = lds_read16(rows_x + Gm::block(i, wave) * 512 + lane * 8);
    }
  }
}

}  // namespace

void launch_dq_bf16(const BwdArgs& a, int D, hipStream_t s) {
  const long nqt = (a.Tq + kBwdBlockM - 1) / kBwdBlockM;
  const long qblocks = nqt * a.Hq * a.B;
  if (qblocks <= 0) return;
  const dim3 grid((unsigned)qblocks);
  if (D == 128)
    hipLaunchKernelGGL(attn_dq_pair_kernel<128>, grid, dim3(DqPairCfg<128>::THREADS), 0, s, a);
  else if (D == 64)
    hipLaunchKernelGGL(attn_dq_pair_kernel<64>, grid, dim3(DqPairCfg<64>::THREADS), 0, s, a);
  else if (D == 256)
    hipLaunchKernelGGL(attn_dq_bf16_kernel<256>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_dq_bf16_kernel<32>, grid, dim3(256), 0, s, a);
}

}  // namespace attn
