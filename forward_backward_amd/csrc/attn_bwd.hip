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
//                  dQ^T += K^T dS^T                            (attn_dq.hip)
// In both kernels the product whose accumulator becomes the next B operand
// is arranged so the register layouts line up (see attn_device.hpp), and the
// transposed operand (dO^T, Q^T, K^T) is read with the LDS transpose read.
// KV tiles wholly past kv_len store zeros without running their loop.
#include <type_traits>

#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
void launch_delta_any(const BwdArgs& a, int D, bool bf16, hipStream_t s);
void launch_dq_bf16(const BwdArgs& a, int D, hipStream_t s);  // attn_dq.hip
void launch_dkdv_bf16_small(const BwdArgs& a, int D, hipStream_t s);  // head_dim 32 and 64, attn_dkdv_small.hip
void launch_dkdv_queue(const BwdArgs& a, hipStream_t s);  // head_dim 128, attn_dkdv_queue.hip

namespace {

// dK/dV at head_dim 256 with the work of each 32-key block split over a pair
// of waves, so that every wave holds half the state (K or V rows, dV or dK):
// one wave per SIMD holds all 256 columns of its dV or dK, so S and dP are
// formed once per block:
//   S wave:  K rows (B operand) and dV^T; per 32-row block S = Q K^T,
//            P = exp2(c S'), P (bf16) to LDS for its partner,
//            dV^T += dO^T P
//   dP wave: V rows and dK^T; dP = dO V^T, P from LDS,
//            dS = P dP', dK^T += Q^T dS
// Both roles run the same products: in step i the row product (S or dP) of
// block i + 1 beside the transposed product (dV or dK) of block i, whose B
// operand (P or dS) came from the previous step; one workgroup barrier per
// step hands P over (double-buffered). Head_dim 128 runs the same split of
// work in the persistent kernel of attn_dkdv_queue.hip.
template <int D>
struct DkvPairCfg {
  // 2 pairs (one wave per SIMD: a wave holds 64 registers of K or V and 128
  // of dV or dK), 32-row tiles, 4 stages.
  static_assert(D == 256, "the wave-pair kernel runs head_dim 256");
  static constexpr int NP = 2;                      // wave pairs, 32 keys each
  static constexpr int BN = 32 * NP;                // keys per workgroup
  static constexpr int BM = 32;                     // query rows per LDS tile
  static constexpr int BPT = BM / 32;               // 32-row blocks per tile
  static constexpr int NST = 4;                     // LDS stages
  static constexpr int THREADS = 128 * NP;          // NP S waves, then NP dP waves
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int R = 4;                       // depth of the fragment read-ahead
  static constexpr int TILE = BM * D;
  static_assert(kBwdBlockN % BN == 0, "a 128-key tile splits into whole workgroups");
};

template <int D>
__global__ __launch_bounds__(DkvPairCfg<D>::THREADS) void attn_dkdv_pair_kernel(BwdArgs a) {
  using C = DkvPairCfg<D>;
  constexpr int TB = C::TILE * 2;                 // bytes of one tile
  constexpr int BB = 32 * D * 2;                  // bytes of one 32-row block
  constexpr int R_OFF = 0;                        // row terms: 16 bytes per query row
  constexpr int Q_OFF = C::NST * C::BM * 16;      // Q stages
  constexpr int G_OFF = Q_OFF + C::NST * TB;      // dO stages
  constexpr int XN = 2;                           // hand-over slots
  constexpr int X_OFF = G_OFF + C::NST * TB;      // P hand-over: [XN][NP waves][2 halves][64 lanes] x 16 B
  constexpr int XB = C::NP * 2 * 1024;            // bytes of one hand-over slot
  __shared__ __attribute__((aligned(16))) char smem[X_OFF + XN * XB];
  uint16_t* const q_st = (uint16_t*)(smem + Q_OFF);
  uint16_t* const g_st = (uint16_t*)(smem + G_OFF);
  uint16_t* const r_st = (uint16_t*)(smem + R_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave / C::NP;              // 0: S, P, dV; 1: dP, dS, dK
  const int w4 = wave % C::NP;               // key block of the pair
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int nkt = a.num_ktiles * (kBwdBlockN / C::BN);  // workgroups per (batch, KV head, split)
  int kt, rest;  // rank 0: the first key tile, the most query rows when causal
  tile_order(bid, nkt, a.kv_split * a.B * a.Hkv, a.causal, rest, kt);
  const int kh = rest % a.Hkv;
  rest /= a.Hkv;
  const int b = rest % a.B;
  const int split = rest / a.B;
  const int G = a.Hq / a.Hkv;
  const int h_lo = split * a.heads_per_split;
  const int nh = min(a.heads_per_split, G - h_lo);
  const int k0 = kt * C::BN;
  const int key = k0 + 32 * w4 + l32;

  const long krs = (long)a.Hkv * D;
  const long qrs = (long)a.Hq * D;
  const long kvoff = ((long)b * a.Tkv * a.Hkv + kh) * D;
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);

  f32x16_t acc[C::DB];  // dV^T (S wave) or dK^T (dP wave)
#pragma unroll
  for (int i = 0; i < C::DB; ++i) acc[i] = f32x16_t{};

  const int kmax = min(k0 + C::BN, kvlim) - 1;
  int i_lo = a.causal ? k0 : 0;
  if (a.win_right >= 0) i_lo = max(i_lo, k0 - a.win_right);
  int i_hi = a.Tq - 1;
  if (a.win_left >= 0) i_hi = min(i_hi, kmax + a.win_left);
  const int qt_begin = i_lo / C::BM;
  const int nq = i_hi >= i_lo ? i_hi / C::BM + 1 - qt_begin : 0;
  const int ntiles = nh * nq;

  if (k0 < kvlim && ntiles > 0) {
    // K (S wave) or V (dP wave) rows of this lane's key as B operands.
    u32x4_t frag[C::KS];
    const bool key_ok = key < kvlim;
    {
      const uint16_t* src = role == 0 ? (const uint16_t*)a.k : (const uint16_t*)a.v;
#pragma unroll
      for (int t = 0; t < C::KS; ++t)
        frag[t] = key_ok ? gload16(src + kvoff + key * krs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
    }
    const float c = a.scale_log2;
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int wave_min_key = k0 + 32 * w4;
    const int wave_max_key = wave_min_key + 31;

    // Lane byte offsets: the row operand is Q (S wave) or dO (dP wave), the
    // transposed operand the other one.
    const uint32_t row_base = role == 0 ? Q_OFF : G_OFF;
    const uint32_t tr_base = role == 0 ? G_OFF : Q_OFF;
    uint32_t row_off[C::KS], tr_off[C::DB][2];
#pragma unroll
    for (int t = 0; t < C::KS; ++t) row_off[t] = row_base + 2 * swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      tr_off[db][0] = tr_base + 2 * swz_off<D>(tr_row, 32 * db + tr_col);
      tr_off[db][1] = tr_base + 2 * swz_off<D>(tr_row + 8, 32 * db + tr_col);
    }
    const uint32_t x_off = X_OFF + (w4 * 2 * 64 + lane) * 16;  // + buffer * XB + half * 1024 (XB per buffer)

    const TileCopy<D, C::BM, C::THREADS> qcopy(qrs, tid);
    auto tile_q0 = [&](int t) { return (qt_begin + t % nq) * C::BM; };
    auto issue = [&](int t) {
      const int st = t % C::NST;
      const int h = kh * G + h_lo + t / nq;
      const int q0 = tile_q0(t);
      const long hoff = ((long)b * a.Tq * a.Hq + h) * D;
      uint16_t* qs = q_st + st * C::TILE;
      uint16_t* gs = g_st + st * C::TILE;
      if (q0 + C::BM <= a.Tq) {
        qcopy.copy(qs, (const uint16_t*)a.q + hoff, qrs, q0);
        qcopy.copy(gs, (const uint16_t*)a.dout + hoff, qrs, q0);
      } else {
        dma_tile<D, C::BM, C::THREADS>(qs, (const uint16_t*)a.q + hoff, qrs, q0, a.Tq, tid);
        dma_tile<D, C::BM, C::THREADS>(gs, (const uint16_t*)a.dout + hoff, qrs, q0, a.Tq, tid);
      }
      // Row terms: one 16-byte row per lane of wave 0 (one copy instruction).
      if (wave == 0 && lane < C::BM) {
        int i = q0 + lane;
        i = i < a.Tq ? i : a.Tq - 1;
        dma16(a.rowstat + (((long)b * a.Hq + h) * a.Tq + i) * 8, lds_addr(r_st + st * C::BM * 8));
      }
    };
    auto mask_tile = [&](int t) {
      if (t >= ntiles) return false;
      const int q0 = tile_q0(t);
      return (wave_min_key < key_lo(q0 + C::BM - 1, a.win_left)) ||
             (wave_max_key > key_hi(q0, kvlim, a.causal, a.win_right)) || (q0 + C::BM > a.Tq);
    };
    // The byte offset of a 32-row block in the ring (its tile's stage and its
    // place in the tile) is made one wave-uniform value, so that each read adds
    // it to its lane offset in one instruction.

    // Row terms as one extra k-step (see the single-role kernel): the S wave
    // selects -LSE/scale, the dP wave -D.
    const unsigned one2 = 0x3F803F80u, one1 = 0x00003F80u;
    const u32x4_t sel = hh != 0 ? u32x4_t{0, 0, 0, 0}
                        : role == 0 ? u32x4_t{one2, one1, 0, 0} : u32x4_t{0, 0, one2, one1};

    // Row product of block `half` of the tile in stage `st`: S (S wave) or dP
    // (dP wave), row terms included.
    auto row_product_at = [&](int st, int half) {
      const uint32_t bo = (uint32_t)__builtin_amdgcn_readfirstlane(st * TB + half * BB);
      const u32x4_t terms = lds_read16((const uint16_t*)(smem + R_OFF + (st * C::BM + 32 * half + l32) * 16));
      u32x4_t ra[C::R];
#pragma unroll
      for (int m = 0; m < C::R; ++m) ra[m] = lds_read16((const uint16_t*)(smem + row_off[m] + bo));
      f32x16_t r = f32x16_t{};
#pragma unroll
      for (int m = 0; m < C::KS; ++m) {
        r = mfma_bf16(ra[m % C::R], frag[m], r);
        if (m + C::R < C::KS) ra[m % C::R] = lds_read16((const uint16_t*)(smem + row_off[m + C::R] + bo));
      }
      return mfma_bf16(terms, sel, r);
    };
    auto row_product = [&](int blk) { return row_product_at((blk / C::BPT) % C::NST, blk % C::BPT); };
    // Transposed product of block `half` of the tile in stage `st`:
    // acc += (dO or Q)^T x packed B operand.
    auto tr_product_at = [&](int st, int half, const u32x4_t (&pk)[2]) {
      const uint32_t bo = (uint32_t)__builtin_amdgcn_readfirstlane(st * TB + half * BB);
      u32x2_t tra[C::R][2];
      auto rd = [&](int m, int slot) {
        const int u = m / C::DB, db = m % C::DB;
        tra[slot][0] = lds_read_tr((const uint16_t*)(smem + tr_off[db][0] + bo + 16 * u * D * 2));
        tra[slot][1] = lds_read_tr((const uint16_t*)(smem + tr_off[db][1] + bo + 16 * u * D * 2));
      };
#pragma unroll
      for (int m = 0; m < C::R; ++m) rd(m, m);
#pragma unroll
      for (int m = 0; m < C::KS; ++m) {
        const int u = m / C::DB, db = m % C::DB, slot = m % C::R;
        acc[db] = mfma_bf16(u32x4_t{tra[slot][0][0], tra[slot][0][1], tra[slot][1][0], tra[slot][1][1]}, pk[u],
                            acc[db]);
        if (m + C::R < C::KS) rd(m + C::R, slot);
      }
    };
    auto tr_product = [&](int blk, const u32x4_t (&pk)[2]) {
      tr_product_at((blk / C::BPT) % C::NST, blk % C::BPT, pk);
    };
    auto pack8 = [](const float* v) {
      return u32x4_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    };

    for (int t = 0; t < C::NST - 1 && t < ntiles; ++t) issue(t);
    wait_vmem();
    __syncthreads();
    const int nb = C::BPT * ntiles;  // 32-row blocks
    // Ring bookkeeping shared by both roles (same barriers in the same order).
    // Step i reads blocks (tiles) i and i + 1. At the first step of tile t,
    // tile t - 1 has been read for the last time and tile t - 1 + NST takes
    // its stage, two steps before its first use; the waits below make it land
    // in time.
    auto step_begin = [&](int i) {
      if (i - 1 + C::NST < ntiles) issue(i - 1 + C::NST);
    };
    auto step_end = [&](int i) {
      // Tile i + 2 (issued at step i - 1) must land; the copies of tile i + 3
      // issued at this step may stay in flight.
      constexpr int CP = 2 * TileCopy<D, C::BM, C::THREADS>::ITERS;  // copy instructions per wave and tile
      if (i + 3 < ntiles) {
        if (wave == 0)
          wait_vmcnt<CP + 1>();
        else
          wait_vmcnt<CP>();
      } else {
        wait_vmem();
      }
      __syncthreads();
    };

    if (role == 0) {
      // P of block blk: exp2 of the row product, masked, packed, handed over.
      u32x4_t pk[2];
      // P of block blk of the tile at query row qt0 (masked when msk).
      auto softmax_at = [&](int blk, const f32x16_t& s, bool msk, int qt0) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(s[r] * c);
        if (msk) {
          const int q0 = qt0 + 32 * (blk % C::BPT);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = (key >= key_lo(ql, a.win_left)) & (key <= key_hi(ql, kvlim, a.causal, a.win_right)) &
                            (ql < a.Tq);
            pv[r] = ok ? pv[r] : 0.f;
          }
        }
        pk[0] = pack8(pv);
        pk[1] = pack8(pv + 8);
        const uint32_t xo = x_off + (blk % XN) * XB;
        lds_write16((uint16_t*)(smem + xo), pk[0]);
        lds_write16((uint16_t*)(smem + xo + 1024), pk[1]);
      };
      auto softmax = [&](int blk, const f32x16_t& s) {
        const int t = blk / C::BPT;
        softmax_at(blk, s, mask_tile(t), t < ntiles ? tile_q0(t) : 0);
      };
      softmax(0, row_product(0));
      __syncthreads();
      for (int i = 0; i < nb; ++i) {
        step_begin(i);
        const f32x16_t s = row_product(i + 1);
        tr_product(i, pk);
        softmax(i + 1, s);
        step_end(i);
      }
    } else {
      f32x16_t dp = row_product(0);
      __syncthreads();
      for (int i = 0; i < nb; ++i) {
        step_begin(i);
        // dS of block i from the handed-over P and the previous step's dP'.
        const uint32_t xo = x_off + (i & 1) * XB;
        const u32x4_t p0 = lds_read16((const uint16_t*)(smem + xo));
        const u32x4_t p1 = lds_read16((const uint16_t*)(smem + xo + 1024));
        float dsv[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dsv[2 * w] = bf16_lo(p0[w]) * dp[2 * w];
          dsv[2 * w + 1] = bf16_hi(p0[w]) * dp[2 * w + 1];
          dsv[8 + 2 * w] = bf16_lo(p1[w]) * dp[8 + 2 * w];
          dsv[8 + 2 * w + 1] = bf16_hi(p1[w]) * dp[8 + 2 * w + 1];
        }
        const u32x4_t pk[2] = {pack8(dsv), pack8(dsv + 8)};
        dp = row_product(i + 1);
        tr_product(i, pk);
        step_end(i);
      }
    }
  }

  // Store: lane = key, register r of block db = head_dim 32*db + 8*(r/4) + 4*hh + r%4;
  // the S wave holds dV, the dP wave dK.
  const bool is_dk = role == 1;
  if (a.kv_split > 1) {
    if (key < a.Tkv) {
      const long part = (long)a.B * a.Tkv * krs;
      float* dst = a.dkv_part + (is_dk ? split : a.kv_split + split) * part + kvoff + key * krs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * hh;
          *(f32x4_t*)(dst + d) = f32x4_t{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        }
    }
    return;
  }
  if (key < a.Tkv) {
    const float f = is_dk ? a.scale : 1.f;
    uint16_t* dst = (uint16_t*)(is_dk ? a.dk : a.dv) + kvoff + key * krs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        *(u32x2_t*)(dst + d) = u32x2_t{pack_bf16(acc[db][4 * g] * f, acc[db][4 * g + 1] * f),
                                       pack_bf16(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f)};
      }
  }
}


// Sum of the kv_split partial dK/dV in split order, rounded to bf16 (dK
// scaled). Each thread handles 8 consecutive elements of [B, Tkv, Hkv, D].
__global__ __launch_bounds__(256) void attn_dkdv_reduce_kernel(BwdArgs a, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const long part = n8 * 8;
  float sk[8] = {}, sv[8] = {};
  for (int s = 0; s < a.kv_split; ++s) {
    const f32x4_t* pk = (const f32x4_t*)(a.dkv_part + s * part) + 2 * i;
    const f32x4_t* pv = (const f32x4_t*)(a.dkv_part + (a.kv_split + s) * part) + 2 * i;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t xk = pk[h], xv = pv[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[4 * h + e] += xk[e];
        sv[4 * h + e] += xv[e];
      }
    }
  }
  u32x4_t wk, wv;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wk[w] = pack_bf16(sk[2 * w] * a.scale, sk[2 * w + 1] * a.scale);
    wv[w] = pack_bf16(sv[2 * w], sv[2 * w + 1]);
  }
  *((u32x4_t*)a.dk + i) = wk;
  *((u32x4_t*)a.dv + i) = wv;
}


template <int D>
void launch_pass(const BwdArgs& a, int pass, hipStream_t s) {
  if (pass == kBwdPre) {
    launch_delta_any(a, D, true, s);
  } else if (pass == kBwdDkdv) {
    const long kblocks = (long)a.kv_split * a.num_ktiles * a.Hkv * a.B;
    if (kblocks > 0) {
      if constexpr (D == 128) {
        launch_dkdv_queue(a, s);
      } else if constexpr (D == 256) {
        hipLaunchKernelGGL(attn_dkdv_pair_kernel<D>, dim3((unsigned)(kblocks * (kBwdBlockN / DkvPairCfg<D>::BN))),
                           dim3(DkvPairCfg<D>::THREADS), 0, s, a);
      } else {
        launch_dkdv_bf16_small(a, D, s);
      }
      if (a.kv_split > 1) {
        const long n8 = (long)a.B * a.Tkv * a.Hkv * D / 8;
        hipLaunchKernelGGL(attn_dkdv_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, a, n8);
      }
    }
  } else {
    launch_dq_bf16(a, D, s);
  }
}

}  // namespace

hipError_t launch_bwd_pass_bf16(const BwdArgs& a, int D, int pass, hipStream_t s) {
  if (D == 128)
    launch_pass<128>(a, pass, s);
  else if (D == 256)
    launch_pass<256>(a, pass, s);
  else if (D == 64)
    launch_pass<64>(a, pass, s);
  else
    launch_pass<32>(a, pass, s);
  return hipGetLastError();
}

}  // namespace attn
