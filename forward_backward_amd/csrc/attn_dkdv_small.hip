// dK/dV pass of the backward at head_dim 32 and 64, bf16, gfx950: the
// single-role kernel, in which every wave holds both K and V rows of its keys
// and both dK and dV (head_dim 128 and 256 run the wave-pair kernel of
// attn_bwd.hip). Deterministic, without atomics (probjax pages, "Attention
// performance", section "When to use which"). A file of its own so that the
// build can compile it with its own options (see build.py).
#include <type_traits>

#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

// ----------------------------------------------------------------- dK / dV
//
// One workgroup per (batch, KV head, 128 keys), 4 waves of 32 keys; K and V
// rows of the wave's keys stay in registers as B operands. The query rows of
// the G heads of the group are visited in a fixed order, in 64-row tiles of
// two 32-row blocks. Per block:
//   S = Q K^T, dP = dO V^T        (lane = key, registers = query rows)
//   P = exp2(S*c - LSE2), dS = P (dP - D)
//   dV^T += dO^T P, dK^T += Q^T dS  (dO^T, Q^T by transpose reads)
// The blocks form a three-deep software pipeline: step i issues the S/dP
// products of block i and the dV/dK products of block i - 2 on the matrix
// core while the vector unit runs the softmax of block i - 1, so every step
// has the same 4*D/16 products to hide its vector work under. Tiles stream
// through a three-stage LDS ring (a tile is read by four consecutive steps);
// the copy of tile t + 2 starts once tile t - 1 has been read for the last
// time. The pipeline runs one step before the first block and one after the
// last on a zero-filled stage and on discarded results, so every step has
// the same shape.

template <int D>
struct DkvCfg {
  static constexpr int BN = kBwdBlockN;     // 128 keys, 32 per wave
  static constexpr int BM = 64;             // query rows per LDS tile
  static constexpr int NST = 3;             // LDS stages
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;         // k-steps of S and dP; also the dV/dK product pairs per block
  static constexpr int DB = D / 32;
  static constexpr int EPS = 16 / KS;       // softmax elements per k-step
  static constexpr int R = 2;               // depth of the fragment read-ahead (k-steps)
  static constexpr int TILE = BM * D;       // swizzled, unpadded (read row-wise and transposed)
};

template <int D>
__global__ __launch_bounds__(256) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using C = DkvCfg<D>;
  // One LDS array: [row-term stages | Q stages | dO stages], so that every
  // read is a lane register plus an immediate below 64 KiB.
  constexpr int TB = C::TILE * 2;                 // bytes of one tile
  constexpr int R_OFF = 0;                        // row terms: 16 bytes per query row
  constexpr int Q_OFF = C::NST * C::BM * 16;      // Q stages
  constexpr int G_OFF = Q_OFF + C::NST * TB;      // dO stages
  __shared__ __attribute__((aligned(16))) char smem[G_OFF + C::NST * TB];
  uint16_t* const q_st = (uint16_t*)(smem + Q_OFF);
  uint16_t* const g_st = (uint16_t*)(smem + G_OFF);
  uint16_t* const r_st = (uint16_t*)(smem + R_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int kt, rest;  // rank 0: the first key tile, the most query rows when causal
  tile_order(bid, a.num_ktiles, a.kv_split * a.B * a.Hkv, a.causal, rest, kt);
  const int kh = rest % a.Hkv;
  rest /= a.Hkv;
  const int b = rest % a.B;
  const int split = rest / a.B;              // which share of the group's query heads
  const int G = a.Hq / a.Hkv;
  const int h_lo = split * a.heads_per_split;
  const int nh = min(a.heads_per_split, G - h_lo);
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

  // Query rows that see some key of [k0, kmax]: key_hi(i) >= k0 from i_lo on,
  // key_lo(i) <= kmax up to i_hi.
  const int kmax = min(k0 + C::BN, kvlim) - 1;
  int i_lo = a.causal ? k0 : 0;
  if (a.win_right >= 0) i_lo = max(i_lo, k0 - a.win_right);
  int i_hi = a.Tq - 1;
  if (a.win_left >= 0) i_hi = min(i_hi, kmax + a.win_left);
  const int qt_begin = i_lo / C::BM;
  const int nq = i_hi >= i_lo ? i_hi / C::BM + 1 - qt_begin : 0;
  const int ntiles = nh * nq;  // (query head, query tile) pairs in a fixed order

  if (k0 < kvlim && ntiles > 0) {
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

    // Byte offsets of this lane's reads inside a tile (swizzled layout).
    uint32_t row_off[C::KS], tr_off[C::DB][2];
#pragma unroll
    for (int t = 0; t < C::KS; ++t) row_off[t] = 2 * swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      tr_off[db][0] = 2 * swz_off<D>(tr_row, 32 * db + tr_col);
      tr_off[db][1] = 2 * swz_off<D>(tr_row + 8, 32 * db + tr_col);
    }

    // The stage of "tile -1" (the last one) starts as zeros: the two steps
    // before the first block compute with it, and zeros add nothing.
    {
      constexpr int ZS = C::NST - 1;
      const u32x4_t z = {0, 0, 0, 0};
      for (int e = tid * 8; e < C::TILE; e += C::THREADS * 8) {
        lds_write16(q_st + ZS * C::TILE + e, z);
        lds_write16(g_st + ZS * C::TILE + e, z);
      }
      if (tid < C::BM) lds_write16(r_st + (ZS * C::BM + tid) * 8, z);
    }

    const TileCopy<D, C::BM, C::THREADS> qcopy(qrs, tid);
    auto tile_q0 = [&](int t) { return (qt_begin + t % nq) * C::BM; };
    auto issue = [&](int t, int st) {
      const int h = kh * G + h_lo + t / nq;
      const int q0 = tile_q0(t);
      const long hoff = ((long)b * a.Tq * a.Hq + h) * D;
      uint16_t* qs = q_st + st * C::TILE;
      uint16_t* gs = g_st + st * C::TILE;
      if (q0 + C::BM <= a.Tq) {
        qcopy.template copy2<G_OFF - Q_OFF>(qs, (const uint16_t*)a.q + hoff, (const uint16_t*)a.dout + hoff, qrs, q0);
      } else {
        dma_tile<D, C::BM, C::THREADS>(qs, (const uint16_t*)a.q + hoff, qrs, q0, a.Tq, tid);
        dma_tile<D, C::BM, C::THREADS>(gs, (const uint16_t*)a.dout + hoff, qrs, q0, a.Tq, tid);
      }
      // Row terms: one 16-byte row per lane of wave 0 (rows past Tq repeat
      // the last row; their elements are masked).
      static_assert(C::BM == 64, "row terms are copied by one wave of 64 lanes");
      if (wave == 0) {
        int i = q0 + lane;
        i = i < a.Tq ? i : a.Tq - 1;
        dma16(a.rowstat + (((long)b * a.Hq + h) * a.Tq + i) * 8, lds_addr(r_st + st * C::BM * 8));
      }
    };
    // Whether tile t needs the element-wise mask (a KV length, causal or
    // window bound inside the wave's keys, or a ragged last query tile). The pipeline's extra
    // tiles (t < 0, t >= ntiles) compute on zeros or are discarded.
    auto mask_tile = [&](int t) {
      if (t < 0 || t >= ntiles) return false;
      const int q0 = tile_q0(t);
      return (wave_min_key < key_lo(q0 + C::BM - 1, a.win_left)) ||
             (wave_max_key > key_hi(q0, kvlim, a.causal, a.win_right)) || (q0 + C::BM > a.Tq);
    };

    // Pipeline registers: S/dP accumulators and the packed P/dS operands,
    // two sets each (set = block parity).
    f32x16_t sacc[2], pacc[2];
    u32x4_t pk_p[2][2], pk_d[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      sacc[x] = f32x16_t{};
      pacc[x] = f32x16_t{};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pk_p[x][u] = u32x4_t{0, 0, 0, 0};
        pk_d[x][u] = u32x4_t{0, 0, 0, 0};
      }
    }

    // Lane byte offsets of the current pair of steps: row reads go to the
    // stage of tile p, transpose reads to the stage of tile p - 1.
    uint32_t rcur[C::KS], tprev[C::DB][2];

    // Row terms enter S and dP through one extra k-step each: the A operand
    // is the query row's 16 bytes of terms (-LSE/scale in elements 0..2, -D in
    // 4..6, read by both lane halves), the B operand selects them with ones in
    // the first lane half (k = 0..7): S' = S - LSE/scale, dP' = dP - D, so
    // that P = exp2(c * S') and dS = P * dP'.
    const unsigned one2 = 0x3F803F80u, one1 = 0x00003F80u;
    const u32x4_t sel_s = hh == 0 ? u32x4_t{one2, one1, 0, 0} : u32x4_t{0, 0, 0, 0};
    const u32x4_t sel_d = hh == 0 ? u32x4_t{0, 0, one2, one1} : u32x4_t{0, 0, 0, 0};

    // One pipeline step: RB is the 32-row block of tile p whose S/dP are
    // formed (into accumulator set RB); the softmax takes block 1 - RB of
    // tile p - 1 (RB = 0) or block 0 of tile p (RB = 1) from set 1 - RB; the
    // dV/dK products take block RB of tile p - 1 (transposed) with packed set
    // RB. `rterm` is this lane's row-term offset (bytes) for block RB.
    auto step = [&](auto rb_, bool mask, int q0m, uint32_t rterm) {
      constexpr int RB = decltype(rb_)::value;
      constexpr int A = RB;        // accumulator set written by this step
      constexpr int P = 1 - RB;    // set read by the softmax
      constexpr int SB = 1 - RB;   // block of the softmax's rows within its tile
      u32x4_t qa[C::R], ga[C::R];
      u32x2_t tg[C::R][2], tx[C::R][2];
      auto read_rows = [&](int m, int slot) {
        qa[slot] = lds_read16((const uint16_t*)(smem + rcur[m] + Q_OFF + 32 * RB * D * 2));
        ga[slot] = lds_read16((const uint16_t*)(smem + rcur[m] + G_OFF + 32 * RB * D * 2));
      };
      // Transposed operands of dV/dK product pair m: half u = m / DB (16
      // query rows), head_dim block db = m % DB.
      auto read_tr = [&](int m, int slot) {
        const int u = m / C::DB, db = m % C::DB;
        const int boff = (32 * RB + 16 * u) * D * 2;
        tg[slot][0] = lds_read_tr((const uint16_t*)(smem + tprev[db][0] + G_OFF + boff));
        tg[slot][1] = lds_read_tr((const uint16_t*)(smem + tprev[db][1] + G_OFF + boff));
        tx[slot][0] = lds_read_tr((const uint16_t*)(smem + tprev[db][0] + Q_OFF + boff));
        tx[slot][1] = lds_read_tr((const uint16_t*)(smem + tprev[db][1] + Q_OFF + boff));
      };
#pragma unroll
      for (int m = 0; m < C::R; ++m) {
        read_rows(m, m);
        read_tr(m, m);
      }
      f32x16_t& s = sacc[A];
      f32x16_t& dp = pacc[A];
      s = f32x16_t{};
      dp = f32x16_t{};
      const f32x16_t& sin = sacc[P];
      const f32x16_t& din = pacc[P];
      const u32x4_t terms = lds_read16((const uint16_t*)(smem + rterm));
      float pv[16], dsv[16];
#pragma unroll
      for (int m = 0; m < C::KS; ++m) {
        const int slot = m % C::R;
        s = mfma_bf16(qa[slot], kf[m], s);
        dp = mfma_bf16(ga[slot], vf[m], dp);
        {
          const int u = m / C::DB, db = m % C::DB;
          dv[db] = mfma_bf16(u32x4_t{tg[slot][0][0], tg[slot][0][1], tg[slot][1][0], tg[slot][1][1]}, pk_p[A][u],
                             dv[db]);
          dk[db] = mfma_bf16(u32x4_t{tx[slot][0][0], tx[slot][0][1], tx[slot][1][0], tx[slot][1][1]}, pk_d[A][u],
                             dk[db]);
        }
        if (m + C::R < C::KS) {
          read_rows(m + C::R, slot);
          read_tr(m + C::R, slot);
        }
        if (m == C::KS - 1) {
          s = mfma_bf16(terms, sel_s, s);
          dp = mfma_bf16(terms, sel_d, dp);
        }
#pragma unroll
        for (int e = 0; e < C::EPS; ++e) {
          const int r = C::EPS * m + e;
          const float p = fast_exp2(sin[r] * c);
          pv[r] = p;
          dsv[r] = p * din[r];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // Element-wise mask, only on tiles that cross a key, causal or row
      // bound. A select (not a product) so that the non-finite values of
      // invalid elements cannot leak.
      if (mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = q0m + 32 * SB + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = (key >= key_lo(ql, a.win_left)) & (key <= key_hi(ql, kvlim, a.causal, a.win_right)) &
                          (ql < a.Tq);
          pv[r] = ok ? pv[r] : 0.f;
          dsv[r] = ok ? dsv[r] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pk_p[P][u] = u32x4_t{pack_bf16(pv[8 * u + 0], pv[8 * u + 1]), pack_bf16(pv[8 * u + 2], pv[8 * u + 3]),
                             pack_bf16(pv[8 * u + 4], pv[8 * u + 5]), pack_bf16(pv[8 * u + 6], pv[8 * u + 7])};
        pk_d[P][u] = u32x4_t{pack_bf16(dsv[8 * u + 0], dsv[8 * u + 1]), pack_bf16(dsv[8 * u + 2], dsv[8 * u + 3]),
                             pack_bf16(dsv[8 * u + 4], dsv[8 * u + 5]), pack_bf16(dsv[8 * u + 6], dsv[8 * u + 7])};
      }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    issue(0, 0);
    if (ntiles > 1) issue(1, 1);
    wait_vmem();
    __syncthreads();
    // Steps 2p and 2p + 1 (tile p in stage p % 3, tile p - 1 in the stage
    // before), then the ring advances: tile p + 1 must have landed and tile
    // p - 1 is free for tile p + 2. One pair past the last tile drains the
    // pipeline.
    int scur = 0;
    for (int p = 0; p <= ntiles; ++p) {
      const int sprev = scur == 0 ? C::NST - 1 : scur - 1;
#pragma unroll
      for (int t = 0; t < C::KS; ++t) rcur[t] = row_off[t] + scur * TB;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        tprev[db][0] = tr_off[db][0] + sprev * TB;
        tprev[db][1] = tr_off[db][1] + sprev * TB;
      }
      const uint32_t rterm = R_OFF + (scur * C::BM + l32) * 16;
      step(I0{}, mask_tile(p - 1), tile_q0(p - 1 < 0 ? 0 : p - 1), rterm);
      step(I1{}, mask_tile(p), tile_q0(p), rterm + 32 * 16);
      wait_vmem();
      __syncthreads();
      if (p + 2 < ntiles) issue(p + 2, sprev);
      scur = scur == C::NST - 1 ? 0 : scur + 1;
    }
  }

  // Store: lane = key, register r of block db = head_dim 32*db + 8*(r/4) + 4*hh + r%4.
  if (a.kv_split > 1) {
    // Partial sums over this workgroup's query heads (dK unscaled); the
    // reduction adds the splits in order and rounds.
    if (key < a.Tkv) {
      const long part = (long)a.B * a.Tkv * krs;  // elements of one [B, Tkv, Hkv, D] partial
      float* dkp = a.dkv_part + split * part + kvoff + key * krs;
      float* dvp = dkp + (long)a.kv_split * part;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * hh;
          *(f32x4_t*)(dkp + d) = f32x4_t{dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]};
          *(f32x4_t*)(dvp + d) = f32x4_t{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
        }
    }
    return;
  }
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

}  // namespace

void launch_dkdv_bf16_small(const BwdArgs& a, int D, hipStream_t s) {
  const long kblocks = (long)a.kv_split * a.num_ktiles * a.Hkv * a.B;
  if (kblocks <= 0) return;
  if (D == 64)
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<64>, dim3((unsigned)kblocks), dim3(DkvCfg<64>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<32>, dim3((unsigned)kblocks), dim3(DkvCfg<32>::THREADS), 0, s, a);
}

}  // namespace attn
