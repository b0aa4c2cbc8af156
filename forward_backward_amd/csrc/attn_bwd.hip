// Backward pass of fused exact attention, bf16, gfx950.
//
// Deterministic two-pass scheme without atomics (probjax pages,
// "Attention performance", section "When to use which": the two-pass
// kernels give bitwise reproducible gradients; "H100 (Hopper)", section
// "Why": the split backward is the robust choice). With P recomputed from
// the forward's LSE (the residuals are O and LSE only):
//   pre-kernel:  D_i = sum_d dO_id O_id                       (attn_fp32.hip)
//   dK/dV:       per (batch, KV head, 128-key tile), for each query head of
//                the group and each 64-row query tile in ascending order:
//                  S = Q K^T, P = exp2(S*c - LSE2), dP = dO V^T,
//                  dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS
//   dQ:          per (batch, head, 128-row query tile), for each 64-key tile:
//                  S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D),
//                  dQ^T += K^T dS^T
// In both kernels the product whose accumulator becomes the next B operand
// is arranged so the register layouts line up (see attn_device.hpp), and the
// transposed operand (dO^T, Q^T, K^T) is read with the LDS transpose read.
// KV tiles wholly past kv_len store zeros without running their loop.
#include <type_traits>

#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
void launch_delta_any(const BwdArgs& a, int D, bool bf16, hipStream_t s);

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------- dK / dV
//
// One workgroup per (batch, KV head, 128 keys), 4 waves of 32 keys; K and V
// rows of the wave's keys stay in registers as B operands. For each query
// head of the group and each 64-row query tile, in a fixed order:
//   S = Q K^T, dP = dO V^T       (lane = key, registers = query rows)
//   P = exp2(S*c - LSE2), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS  (dO^T, Q^T by transpose reads)
// The tile of four 32-row blocks is a software pipeline: block j+1's S/dP
// products are interleaved with block j's softmax, so the vector work runs
// under the matrix work.

template <int D>
struct DkvCfg {
  static constexpr int BN = kBwdBlockN;     // 128 keys, 32 per wave
  static constexpr int BM = 64;             // query rows per LDS tile
  static constexpr int NB = BM / 32;        // 32-row blocks per tile (pipeline depth)
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BM * D;       // swizzled, unpadded (read row-wise and transposed)
};

template <int D>
__global__ __launch_bounds__(256) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using C = DkvCfg<D>;
  // Two pipeline stages of the Q and dO tiles in one array, so that one
  // per-lane offset plus a constant addresses every stage.
  __shared__ __attribute__((aligned(16))) uint16_t tiles[4 * C::TILE];
  __shared__ __attribute__((aligned(16))) float l_s0[C::BM], l_s1[C::BM];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float d_s0[C::BM], d_s1[C::BM];  // D = rowsum(dO * O)
  uint16_t* const q_s0 = tiles;
  uint16_t* const g_s0 = tiles + C::TILE;   // dO tiles
  uint16_t* const q_s1 = tiles + 2 * C::TILE;
  uint16_t* const g_s1 = tiles + 3 * C::TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = bid % a.num_ktiles;
  const int bkh = bid / a.num_ktiles;
  const int kh = bkh % a.Hkv;
  const int b = bkh / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int k0 = kt * C::BN;
  const int key = k0 + 32 * wave + l32;      // this lane's key

  const long krs = (long)a.Hkv * D;
  const long qrs = (long)a.Hq * D;
  const long kvoff = ((long)b * a.Tkv * a.Hkv + kh) * D;
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);

  f32x16_t dk[C::DB], dv[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) {
    dk[i] = f32x16_t{};
    dv[i] = f32x16_t{};
  }

  if (k0 < kvlim) {
    // K and V rows of this lane's key as B operands (k = head_dim).
    u32x4_t kf[C::KS], vf[C::KS];
    const bool key_ok = key < kvlim;
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
      kf[t] = key_ok ? gload16((const uint16_t*)a.k + kvoff + key * krs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
      vf[t] = key_ok ? gload16((const uint16_t*)a.v + kvoff + key * krs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
    }
    const float c = a.scale_log2;
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int wave_min_key = k0 + 32 * wave;
    const int wave_max_key = wave_min_key + 31;
    const int qt_begin = a.causal ? k0 / C::BM : 0;
    const int nqt = (a.Tq + C::BM - 1) / C::BM;
    const int nq = nqt - qt_begin;
    const int ntiles = G * nq;  // (query head, query tile) pairs in a fixed order

    // Per-lane swizzled offsets (elements); the row block and stage parts are
    // compile-time constants (swz_f depends only on the low 4 bits of the row).
    int nrm[C::KS], trd[C::DB][2];
#pragma unroll
    for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col);
      trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col);
    }

    const TileCopy<D, C::BM, C::THREADS> qcopy(qrs, tid);
    auto issue = [&](int idx, uint16_t* qs, uint16_t* gs, float* ls, float* ds) {
      const int h = kh * G + idx / nq;
      const int q0 = (qt_begin + idx % nq) * C::BM;
      const long hoff = ((long)b * a.Tq * a.Hq + h) * D;
      if (q0 + C::BM <= a.Tq) {
        qcopy.copy(qs, (const uint16_t*)a.q + hoff, qrs, q0);
        qcopy.copy(gs, (const uint16_t*)a.dout + hoff, qrs, q0);
      } else {
        dma_tile<D, C::BM, C::THREADS>(qs, (const uint16_t*)a.q + hoff, qrs, q0, a.Tq, tid);
        dma_tile<D, C::BM, C::THREADS>(gs, (const uint16_t*)a.dout + hoff, qrs, q0, a.Tq, tid);
      }
      const long stat0 = ((long)b * a.Hq + h) * a.Tq;
      static_assert(C::BM == 64, "row statistics are copied by two waves of 64 lanes");
      if (wave == 0) dma_row64(ls, a.lse2 + stat0, q0, a.Tq, lane);
      if (wave == 1) dma_row64(ds, a.delta + stat0, q0, a.Tq, lane);
    };

    // S = Q K^T and dP = dO V^T of block qb, with the row fragments read
    // through a two-deep register ring (the reads of step t + 2 are issued as
    // soon as the products of step t have taken their operands).
    auto sdp = [&](const uint16_t* qsb, const uint16_t* gsb, int qb, f32x16_t& s, f32x16_t& dp) {
      const uint16_t* qrow = qsb + 32 * qb * D;
      const uint16_t* grow = gsb + 32 * qb * D;
      u32x4_t qa[2], ga[2];
      qa[0] = lds_read16(qrow + nrm[0]);
      ga[0] = lds_read16(grow + nrm[0]);
      qa[1] = lds_read16(qrow + nrm[1]);
      ga[1] = lds_read16(grow + nrm[1]);
      s = f32x16_t{};
      dp = f32x16_t{};
#pragma unroll
      for (int t = 0; t < C::KS; ++t) {
        s = mfma_bf16(qa[t & 1], kf[t], s);
        dp = mfma_bf16(ga[t & 1], vf[t], dp);
        if (t + 2 < C::KS) {
          qa[t & 1] = lds_read16(qrow + nrm[t + 2]);
          ga[t & 1] = lds_read16(grow + nrm[t + 2]);
        }
      }
    };
    // P and dS of block qb as bf16 B operands (16 query rows each).
    auto softmax = [&](auto mask_tag, const float* ls, const float* ds, int q0, int qb, const f32x16_t& s,
                       const f32x16_t& dp, u32x4_t* pb, u32x4_t* dsb) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x4_t lv[4], dl[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lv[g] = *(const f32x4_t*)(ls + 32 * qb + 8 * g + 4 * hh);
        dl[g] = *(const f32x4_t*)(ds + 32 * qb + 8 * g + 4 * hh);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float pv[8], dsv[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int r = 8 * u + x;
          float p = fast_exp2(__builtin_fmaf(s[r], c, -lv[r >> 2][r & 3]));
          if constexpr (MASK) {
            const int ql = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = (key < kvlim) & (!a.causal | (key <= ql)) & (ql < a.Tq);
            p = ok ? p : 0.f;
          }
          pv[x] = p;
          dsv[x] = p * (dp[r] - dl[r >> 2][r & 3]);
        }
        pb[u] = u32x4_t{pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                        pack_bf16(pv[6], pv[7])};
        dsb[u] = u32x4_t{pack_bf16(dsv[0], dsv[1]), pack_bf16(dsv[2], dsv[3]), pack_bf16(dsv[4], dsv[5]),
                         pack_bf16(dsv[6], dsv[7])};
      }
    };
    // dV^T += dO^T P and dK^T += Q^T dS for half u (16 query rows) of block qb:
    // transpose reads of dO and Q, then the products.
    struct TrFrags {
      u32x2_t g[C::DB][2], x[C::DB][2];
    };
    auto read_tr = [&](const uint16_t* qsb, const uint16_t* gsb, int qb, int u, TrFrags& f) {
      const uint16_t* gblk = gsb + (32 * qb + 16 * u) * D;
      const uint16_t* qblk = qsb + (32 * qb + 16 * u) * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        f.g[db][0] = lds_read_tr(gblk + trd[db][0]);
        f.g[db][1] = lds_read_tr(gblk + trd[db][1]);
        f.x[db][0] = lds_read_tr(qblk + trd[db][0]);
        f.x[db][1] = lds_read_tr(qblk + trd[db][1]);
      }
    };
    auto dvdk_half = [&](const TrFrags& f, const u32x4_t& p, const u32x4_t& dsv) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        dv[db] = mfma_bf16(u32x4_t{f.g[db][0][0], f.g[db][0][1], f.g[db][1][0], f.g[db][1][1]}, p, dv[db]);
        dk[db] = mfma_bf16(u32x4_t{f.x[db][0][0], f.x[db][0][1], f.x[db][1][0], f.x[db][1][1]}, dsv, dk[db]);
      }
    };

    // One query tile from stage (qsb, gsb, ls, ds); the next tile's loads into
    // the other stage start at the top.
    auto tile = [&](int idx, const uint16_t* qsb, const uint16_t* gsb, const float* ls, const float* ds,
                    auto&& issue_next) {
      const int q0 = (qt_begin + idx % nq) * C::BM;
      issue_next();
      const bool mask_tile =
          (wave_max_key >= kvlim) || (a.causal && q0 < wave_max_key) || (q0 + C::BM > a.Tq);
      // Pipeline over the two 32-row blocks:
      //   S/dP(0);  [S/dP(1) | softmax(0)];  [dV/dK(0) | softmax(1)];  dV/dK(1)
      // where [x | y] interleaves the products x with the vector work y.
      auto body = [&](auto mask_tag) {
        f32x16_t s0, dp0, s1, dp1;
        u32x4_t pb0[2], ds0[2], pb1[2], ds1[2];
        TrFrags tf;
        sdp(qsb, gsb, 0, s0, dp0);
        __builtin_amdgcn_sched_barrier(0);
        sdp(qsb, gsb, 1, s1, dp1);
        softmax(mask_tag, ls, ds, q0, 0, s0, dp0, pb0, ds0);
#pragma unroll
        for (int i = 0; i < 2 * C::KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then vector ALU work
        }
        __builtin_amdgcn_sched_barrier(0);
        read_tr(qsb, gsb, 0, 0, tf);
        __builtin_amdgcn_sched_barrier(0);
        dvdk_half(tf, pb0[0], ds0[0]);
        read_tr(qsb, gsb, 0, 1, tf);
        softmax(mask_tag, ls, ds, q0, 1, s1, dp1, pb1, ds1);
        for (int i = 0; i < 2 * C::DB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two transpose reads
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // then vector ALU work
        }
        __builtin_amdgcn_sched_barrier(0);
        dvdk_half(tf, pb0[1], ds0[1]);
        read_tr(qsb, gsb, 1, 0, tf);
        dvdk_half(tf, pb1[0], ds1[0]);
        read_tr(qsb, gsb, 1, 1, tf);
        dvdk_half(tf, pb1[1], ds1[1]);
      };
      if (mask_tile)
        body(std::true_type{});
      else
        body(std::false_type{});
      wait_vmem();
      __syncthreads();
    };

    if (ntiles > 0) issue(0, q_s0, g_s0, l_s0, d_s0);
    wait_vmem();
    __syncthreads();
    for (int idx = 0; idx < ntiles; idx += 2) {
      tile(idx, q_s0, g_s0, l_s0, d_s0, [&]() {
        if (idx + 1 < ntiles) issue(idx + 1, q_s1, g_s1, l_s1, d_s1);
      });
      if (idx + 1 >= ntiles) break;
      tile(idx + 1, q_s1, g_s1, l_s1, d_s1, [&]() {
        if (idx + 2 < ntiles) issue(idx + 2, q_s0, g_s0, l_s0, d_s0);
      });
    }
  }

  // Store: lane = key, register r of block db = head_dim 32*db + 8*(r/4) + 4*hh + r%4.
  if (key < a.Tkv) {
    uint16_t* dkp = (uint16_t*)a.dk + kvoff + key * krs;
    uint16_t* dvp = (uint16_t*)a.dv + kvoff + key * krs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        *(u32x2_t*)(dkp + d) = u32x2_t{pack_bf16(dk[db][4 * g] * a.scale, dk[db][4 * g + 1] * a.scale),
                                       pack_bf16(dk[db][4 * g + 2] * a.scale, dk[db][4 * g + 3] * a.scale)};
        *(u32x2_t*)(dvp + d) = u32x2_t{pack_bf16(dv[db][4 * g], dv[db][4 * g + 1]),
                                       pack_bf16(dv[db][4 * g + 2], dv[db][4 * g + 3])};
      }
  }
}

// --------------------------------------------------------------------- dQ

template <int D>
struct DqCfg {
  static constexpr int BM = 128;            // query rows, 32 per wave
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
  const int qt = nqt - 1 - (bid % nqt);
  const int bh = bid / nqt;
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
  int kv_end = kvlim;
  if (a.causal) kv_end = min(kv_end, q0 + C::BM);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

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
  int nrm[C::KS], trd[C::DB][2];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col);
    trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col);
  }

  auto issue = [&](int it, uint16_t* ks, uint16_t* vs) {
    const int k0 = it * C::BN;
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
          const bool ok = (kk < kvlim) & (!a.causal | (kk <= qrow));
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
    const int k0 = it * C::BN;
    const bool mask_tile = (k0 + C::BN > kvlim) || (a.causal && k0 + C::BN - 1 > wave_min_row);
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
    if (mask_tile)
      body(std::true_type{});
    else
      body(std::false_type{});
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

template <int D>
void launch_pass(const BwdArgs& a, int pass, hipStream_t s) {
  if (pass == kBwdPre) {
    launch_delta_any(a, D, true, s);
  } else if (pass == kBwdDkdv) {
    const long kblocks = (long)a.num_ktiles * a.Hkv * a.B;
    if (kblocks > 0)
      hipLaunchKernelGGL(attn_dkdv_bf16_kernel<D>, dim3((unsigned)kblocks), dim3(DkvCfg<D>::THREADS), 0, s, a);
  } else {
    const long nqt = (a.Tq + DqCfg<D>::BM - 1) / DqCfg<D>::BM;
    const long qblocks = nqt * a.Hq * a.B;
    if (qblocks > 0) hipLaunchKernelGGL(attn_dq_bf16_kernel<D>, dim3((unsigned)qblocks), dim3(256), 0, s, a);
  }
}

}  // namespace

hipError_t launch_bwd_pass_bf16(const BwdArgs& a, int D, int pass, hipStream_t s) {
  if (D == 128)
    launch_pass<128>(a, pass, s);
  else
    launch_pass<64>(a, pass, s);
  return hipGetLastError();
}

}  // namespace attn
