// Forward pass of fused exact attention at head_dim 256, bf16, gfx950: the
// same method as attn_fwd.hip (probjax pages, "Attention performance": the
// kernels keep only O and the LSE, memory linear in T), with each 32-row
// block's work split over a pair of waves. A file of its own so that the
// build can schedule the other forward kernels with their own options (see
// build.py).
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr float kRescaleLog2 = 8.f;  // rescale O only when a row max grows by > 2^8

// Forward with each 32-row block's work split over a pair of waves by role,
// for head_dim 256 (where one wave holding Q and O would take 192 registers
// and run alone on its SIMD):
//   S wave: Q rows (B operand); per 32-key block S^T = K Q^T, the online
//           softmax (mask, row max, lazy rescale decision), P = exp2(c S - m)
//           packed to bf16 and handed over with the rescale factor of each row
//   O wave: O^T; one block later, O *= alpha (when some row rescaled) and
//           O^T += V^T P^T with V by transpose reads
// Both hold under 256 registers, so two waves share each SIMD. One workgroup
// barrier per step hands P over (double-buffered). K and V stream in 32-key
// tiles through a four-stage ring: tile u is read in steps u (K) and u + 1
// (V); the copy of tile j + 2 starts at step j and must have landed by the
// end of step j + 1 (only the copies issued at that step may still be in
// flight). At the end the S wave hands over 1 / (row sum) and writes the LSE.
template <int D>
struct FwdPairCfg {
  static constexpr int NP = 4;                // wave pairs, 32 query rows each
  static constexpr int BM = 32 * NP;          // 128 query rows
  static constexpr int BN = 32;               // keys per tile
  static constexpr int NST = 4;               // LDS stages (K and V of one tile each)
  static constexpr int THREADS = 128 * NP;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int R = 4;                 // fragment read-ahead
  static constexpr int TILE = BN * D;         // elements of one K or V tile
  static_assert(BM == kFwdBlockM, "the host sizes the grid with kFwdBlockM");
};

template <int D>
__global__ __launch_bounds__(FwdPairCfg<D>::THREADS) void attn_fwd_pair_kernel(FwdArgs a) {
  using C = FwdPairCfg<D>;
  constexpr int TB = C::TILE * 2;                   // bytes of one K or V tile
  constexpr int X_OFF = C::NST * 2 * TB;            // P hand-over: [2][NP][2 halves][64 lanes] x 16 B
  constexpr int XB = C::NP * 2 * 1024;
  constexpr int A_OFF = X_OFF + 2 * XB;             // rescale factors: [2][NP][64 lanes] floats
  constexpr int AB = C::NP * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[A_OFF + 2 * AB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave / C::NP;                    // 0: S and softmax; 1: O
  const int w4 = wave % C::NP;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, rank;
  tile_order(bid, a.num_qtiles, a.B * a.Hq, a.causal, bh, rank, a.Hq / a.Hkv);
  const int qt = a.num_qtiles - 1 - rank;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kh = h / (a.Hq / a.Hkv);
  const int q0 = qt * C::BM;

  const long qrs = (long)a.Hq * D;
  const long krs = (long)a.Hkv * D;
  const uint16_t* qb = (const uint16_t*)a.q + ((long)b * a.Tq * a.Hq + h) * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  const TileCopy<D, C::BN, C::THREADS> kvcopy(krs, tid);
  auto issue = [&](int j) {
    char* st = smem + (j % C::NST) * 2 * TB;
    const int k0 = (j0 + j) * C::BN;
    if (k0 + C::BN <= kv_end) {
      kvcopy.template copy2<TB>((uint16_t*)st, kb, vb, krs, k0);
    } else {
      dma_tile<D, C::BN, C::THREADS>((uint16_t*)st, kb, krs, k0, kv_end, tid);
      dma_tile<D, C::BN, C::THREADS>((uint16_t*)(st + TB), vb, krs, k0, kv_end, tid);
    }
  };
  constexpr int CP = 2 * TileCopy<D, C::BN, C::THREADS>::ITERS;  // copy instructions per wave and tile
  for (int j = 0; j < 2 && j < ntiles; ++j) issue(j);

  const int qrow = q0 + 32 * w4 + l32;
  const bool row_ok = qrow < a.Tq;
  const float c = a.scale_log2;
  const uint32_t x_off = X_OFF + (w4 * 2 * 64 + lane) * 16;  // + buffer * XB + half * 1024
  const uint32_t a_off = A_OFF + (w4 * 64 + lane) * 4;       // + buffer * AB

  // Ring bookkeeping (both roles, same barriers).
  auto step_begin = [&](int j) {
    if (j + 2 < ntiles) issue(j + 2);
  };
  auto step_end = [&](int j) {
    if (j + 2 < ntiles)
      __builtin_amdgcn_s_waitcnt((CP & 15) | ((CP >> 4) << 14) | (7 << 4) | (15 << 8));  // vmcnt(CP)
    else
      wait_vmem();
    __syncthreads();
  };
  wait_vmem();
  __syncthreads();

  if (role == 0) {
    u32x4_t qf[C::KS];
#pragma unroll
    for (int t = 0; t < C::KS; ++t)
      qf[t] = row_ok ? gload16(qb + qrow * qrs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
    int nrm[C::KS];
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
      // Byte offsets, opaque to the compiler: it would otherwise factor a
      // common term out of them and add it back on every read.
      nrm[t] = 2 * swz_off<D>(l32, 16 * t + 8 * hh);
      asm volatile("" : "+v"(nrm[t]));
    }
    float m = -INFINITY, lsum = 0.f;
    const int wave_min_row = q0 + 32 * w4;
    const int row_lo = key_lo(qrow, a.win_left);
    const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
    const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
    const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);
    for (int j = 0; j <= ntiles; ++j) {
      step_begin(j);
      if (j < ntiles) {
        // The stage offset as one wave-uniform value: one vector add per read.
        const char* kl = smem + __builtin_amdgcn_readfirstlane((j % C::NST) * 2 * TB);
        u32x4_t ka[C::R];
#pragma unroll
        for (int t = 0; t < C::R; ++t) ka[t] = lds_read16((const uint16_t*)(kl + nrm[t]));
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int t = 0; t < C::KS; ++t) {
          s = mfma_bf16(ka[t % C::R], qf[t], s);
          if (t + C::R < C::KS) ka[t % C::R] = lds_read16((const uint16_t*)(kl + nrm[t + C::R]));
        }
        const int k0 = (j0 + j) * C::BN;
        if ((k0 < wave_all_lo) || (k0 + C::BN - 1 > wave_all_hi)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            s[r] = (key >= row_lo && key <= row_hi) ? s[r] : -INFINITY;
          }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
        mt = half_max(mt);
        // Lazy rescaling as in the single-role forward (reference max moves
        // only when some row would see exponentials above 2^kRescaleLog2).
        const bool grow = (m == -INFINITY) ? (mt != -INFINITY) : ((mt - m) * c > kRescaleLog2);
        const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
        const float mnew = any ? fmaxf(m, mt) : m;
        const float alpha =
            (m == -INFINITY || !any) ? (m == -INFINITY ? 0.f : 1.f) : fast_exp2((m - mnew) * c);
        m = mnew;
        const float nb = (m == -INFINITY) ? 0.f : -m * c;
        float pv[16], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = fast_exp2(__builtin_fmaf(s[r], c, nb));
          ps += pv[r];
        }
        lsum = lsum * alpha + ps;
        const uint32_t xo = x_off + (j & 1) * XB;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          lds_write16((uint16_t*)(smem + xo + u * 1024),
                      u32x4_t{pack_bf16(pv[8 * u + 0], pv[8 * u + 1]), pack_bf16(pv[8 * u + 2], pv[8 * u + 3]),
                              pack_bf16(pv[8 * u + 4], pv[8 * u + 5]), pack_bf16(pv[8 * u + 6], pv[8 * u + 7])});
        *(float*)(smem + a_off + (j & 1) * AB) = alpha;
      }
      step_end(j);
    }
    // 1 / row sum for the O wave, and the LSE.
    const float ltot = half_sum(lsum);
    *(float*)(smem + a_off) = ltot > 0.f ? 1.f / ltot : 0.f;
    if (row_ok && hh == 0)
      a.lse[((long)b * a.Hq + h) * a.Tq + qrow] = ltot > 0.f ? m * a.scale + __logf(ltot) : -INFINITY;
    __syncthreads();
  } else {
    f32x16_t o[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) o[i] = f32x16_t{};
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int trd[C::DB][2];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col);
      trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col);
    }
    for (int j = 0; j <= ntiles; ++j) {
      step_begin(j);
      if (j > 0) {
        const int jp = j - 1;
        const uint32_t xo = x_off + (jp & 1) * XB;
        const u32x4_t pk0 = lds_read16((const uint16_t*)(smem + xo));
        const u32x4_t pk1 = lds_read16((const uint16_t*)(smem + xo + 1024));
        const float alpha = *(const float*)(smem + a_off + (jp & 1) * AB);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
          for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
        }
        const uint16_t* vl = (const uint16_t*)(smem + (jp % C::NST) * 2 * TB + TB);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4_t pk = u == 0 ? pk0 : pk1;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const u32x2_t lo = lds_read_tr(vl + 16 * u * D + trd[db][0]);
            const u32x2_t hi = lds_read_tr(vl + 16 * u * D + trd[db][1]);
            o[db] = mfma_bf16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pk, o[db]);
          }
        }
      }
      step_end(j);
    }
    __syncthreads();
    const float inv = *(const float*)(smem + a_off);
    if (row_ok) {
      uint16_t* ob = (uint16_t*)a.o + ((long)b * a.Tq * a.Hq + h) * D + qrow * qrs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * hh;
          *(u32x2_t*)(ob + d) = u32x2_t{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                        pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        }
    }
  }
}

}  // namespace

void launch_fwd_pair_bf16(const FwdArgs& a, hipStream_t s) {
  const long blocks = (long)a.num_qtiles * a.Hq * a.B;
  if (blocks == 0) return;
  hipLaunchKernelGGL(attn_fwd_pair_kernel<256>, dim3((unsigned)blocks), dim3(FwdPairCfg<256>::THREADS), 0, s, a);
}

}  // namespace attn
