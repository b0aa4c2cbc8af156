// Forward pass of fused exact attention, bf16, gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V and the natural-log LSE with
// an online softmax over KV tiles (probjax pages, "Attention performance":
// the kernels keep only O and the LSE, memory linear in T).
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
// owns 32 rows. Per KV tile of 64 keys:
//   S^T = K Q^T      (32x32x16 MFMA; K from LDS, Q held in registers) so that
//                    every lane holds one query row: lane l has query row l%32
//                    and 16 of the 32 keys of each key block, the other 16 in
//                    lane l^32;
//   softmax          row max over the lane's values plus one half-swap; base-2
//                    exponentials with the scale folded into one FMA; O and
//                    the row sum are rescaled only when a row max grows by
//                    more than 2^8 (wave-uniform decision);
//   O^T += V^T P^T   (32x32x16 MFMA; P is converted from the S accumulator
//                    registers directly, V is read with the LDS transpose read
//                    so its key order matches the registers of P).
// Software pipeline: while the matrix core computes S for tile j + 1, the
// vector unit runs the softmax of tile j; then O += P_j V_j. K and V tiles
// stream into two-stage LDS rings by direct global->LDS copies, K one tile
// ahead of V: during iteration j the copies of K_{j+2} and V_{j+1} are in
// flight while K_{j+1} and V_j are read. Tiles use the swizzled unpadded
// layout of attn_device.hpp (no bank conflicts for row or transpose reads).
// Only the key tiles that some row of the query tile sees are visited (the
// KV length, causal and local window bounds, see key_lo / key_hi); rows of a
// partially visible tile are masked element-wise (the copies of rows past the
// last visible key repeat it).
#include "attn_device.hpp"
#include "attn_internal.h"

#include <type_traits>

namespace attn {
void launch_fwd_pair_bf16(const FwdArgs& a, hipStream_t s);  // head_dim 256, attn_fwd256.hip
namespace {

constexpr float kRescaleLog2 = 8.f;  // rescale O only when a row max grows by > 2^8

template <int D>
struct FwdCfg {
  static constexpr int BM = kFwdBlockM;       // 128 query rows
  static constexpr int BN = 64;               // keys per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;           // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;           // 32-wide blocks of head_dim in O
  static constexpr int TILE = BN * D;         // elements of one K or V tile
};

// Two workgroups per compute unit (head_dim 32, 64 and 128; head_dim 256 runs
// the wave-pair kernel of attn_fwd256.hip).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  // K and V stages; after the tile loop the first two hold the O tile on its way out.
  __shared__ __attribute__((aligned(16))) uint16_t kv_s[4 * C::TILE];
  uint16_t* const k_s0 = kv_s;
  uint16_t* const k_s1 = kv_s + C::TILE;
  uint16_t* const v_s0 = kv_s + 2 * C::TILE;
  uint16_t* const v_s1 = kv_s + 3 * C::TILE;
  static_assert(2 * C::TILE == C::BM * D, "the O tile fills the two K stages");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int bh, rank;
  tile_order(bid, a.num_qtiles, a.B * a.Hq, a.causal, bh, rank, a.Hq / a.Hkv);
  const int qt = a.num_qtiles - 1 - rank;  // rank 0: the last query tile, the most keys when causal
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int kh = h / (a.Hq / a.Hkv);
  const int q0 = qt * C::BM;

  const long qrs = (long)a.Hq * D;
  const long krs = (long)a.Hkv * D;
  const uint16_t* qb = (const uint16_t*)a.q + ((long)b * a.Tq * a.Hq + h) * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  // Keys any row of the tile sees: [key_lo(first row), key_hi(last row)].
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;  // first key tile
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  // Copies of the tile-loop's tile j (key tile j0 + j).
  const TileCopy<D, C::BN, C::THREADS> kvcopy(krs, tid);
  auto issue_k = [&](int j, uint16_t* dst) {
    const int k0 = (j0 + j) * C::BN;
    if (k0 + C::BN <= kv_end)
      kvcopy.copy1(dst, kb, krs, k0);
    else
      dma_tile<D, C::BN, C::THREADS>(dst, kb, krs, k0, kv_end, tid);
  };
  auto issue_v = [&](int j, uint16_t* dst) {
    const int k0 = (j0 + j) * C::BN;
    if (k0 + C::BN <= kv_end)
      kvcopy.copy1(dst, vb, krs, k0);
    else
      dma_tile<D, C::BN, C::THREADS>(dst, vb, krs, k0, kv_end, tid);
  };
  if (ntiles > 0) {
    issue_k(0, k_s0);
    issue_v(0, v_s0);
    if (ntiles > 1) issue_k(1, k_s1);
  }

  const int qrow = q0 + 32 * wave + l32;
  const bool row_ok = qrow < a.Tq;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8hh .. +7].
  u32x4_t qf[C::KS];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    qf[t] = row_ok ? gload16(qb + qrow * qrs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
  }
  // Take Q before the loop: the compiler cannot see the copies, and a first
  // use of Q inside the loop would make it wait for all loads on every pass.
#pragma unroll
  for (int t = 0; t < C::KS; ++t) asm volatile("" ::"v"(qf[t]));

  f32x16_t o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16_t{};
  float m = -INFINITY;   // running max of raw scores S (scale applied in the exponent)
  float lsum = 0.f;      // this lane's share of the softmax denominator

  const float c = a.scale_log2;
  const int wave_min_row = q0 + 32 * wave;
  // Visible keys of this lane's row, and the keys every row of the wave sees.
  const int row_lo = key_lo(qrow, a.win_left);
  const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
  const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
  const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);

  // Swizzled LDS offsets of this lane's reads (row blocks of 16 keep the swizzle).
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int nrm[C::KS], trd[C::DB][2];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) nrm[t] = swz_off<D>(l32, 16 * t + 8 * hh);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    trd[db][0] = swz_off<D>(tr_row, 32 * db + tr_col);
    trd[db][1] = swz_off<D>(tr_row + 8, 32 * db + tr_col);
  }

  // S^T for the two 32-key blocks of a K tile.
  auto sdot = [&](const uint16_t* kl, f32x16_t (&s)[2]) {
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::KS; ++t)
#pragma unroll
      for (int j = 0; j < 2; ++j) s[j] = mfma_bf16(lds_read16(kl + 32 * j * D + nrm[t]), qf[t], s[j]);
  };

  // Softmax of tile j in place (S -> P, unnormalised) and the packed bf16
  // B operands of the PV product. Returns whether O must be rescaled by
  // `alpha` (wave-uniform); the rescale itself is left to the caller so that
  // this stays free of branches.
  auto softmax = [&](auto mask_tag, int j, f32x16_t (&s)[2], u32x4_t (&pf)[4], float& alpha) -> bool {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = (j0 + j) * C::BN;
    if constexpr (MASK) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * x + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = key >= row_lo && key <= row_hi;
          s[x][r] = ok ? s[x][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[x][r]);
    mt = half_max(mt);
    // Lazy rescaling: the reference max m only moves when some row of the
    // wave would otherwise see exponentials above 2^kRescaleLog2 (or had no
    // valid key yet). Numerator and denominator share the reference, so the
    // result is the same; it only bounds P (kept <= 2^8, exact in bf16's range).
    const bool grow = (m == -INFINITY) ? (mt != -INFINITY) : ((mt - m) * c > kRescaleLog2);
    const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
    const float mnew = any ? fmaxf(m, mt) : m;
    alpha = (m == -INFINITY || !any) ? (m == -INFINITY ? 0.f : 1.f) : fast_exp2((m - mnew) * c);
    m = mnew;
    lsum *= alpha;
    const float nb = (m == -INFINITY) ? 0.f : -m * c;
    float ps = 0.f;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[x][r], c, nb));
        s[x][r] = p;
        ps += p;
      }
    lsum += ps;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 8 * u;
        pf[2 * x + u] = u32x4_t{pack_bf16(s[x][r0 + 0], s[x][r0 + 1]), pack_bf16(s[x][r0 + 2], s[x][r0 + 3]),
                                pack_bf16(s[x][r0 + 4], s[x][r0 + 5]), pack_bf16(s[x][r0 + 6], s[x][r0 + 7])};
      }
    return any;
  };

  auto pv = [&](const uint16_t* vl, const u32x4_t (&pf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2_t lo = lds_read_tr(vl + 16 * ks * D + trd[db][0]);
        const u32x2_t hi = lds_read_tr(vl + 16 * ks * D + trd[db][1]);
        o[db] = mfma_bf16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf[ks], o[db]);
      }
  };

  f32x16_t s_cur[2], s_nxt[2];
  if (ntiles > 0) {
    wait_vmem();
    __syncthreads();
    sdot(k_s0, s_cur);
    __syncthreads();  // every wave has read K_0 before K_2 overwrites it
  }

  // Iteration j: copies of K_{j+2} and V_{j+1} start; S_{j+1} from K_{j+1}
  // (on the last tile a stale stage whose result is dropped) runs beside the
  // softmax of tile j; then O += P_j V_j.
  auto step = [&](int j, const uint16_t* kn, uint16_t* kfree, const uint16_t* vc, uint16_t* vfree) {
    if (j + 2 < ntiles) issue_k(j + 2, kfree);
    if (j + 1 < ntiles) issue_v(j + 1, vfree);
    const int k0 = (j0 + j) * C::BN;
    const bool need_mask = (k0 < wave_all_lo) || (k0 + C::BN - 1 > wave_all_hi);
    u32x4_t pf[4];
    float alpha;
    bool any;
    auto body = [&](auto mask_tag) {
      sdot(kn, s_nxt);
      any = softmax(mask_tag, j, s_cur, pf, alpha);
      // Vector instructions per group: 6 at head_dim 128, 8 below (measured;
      // 4, 5, 10 and 12 were slower at 128, and 6 slower at 32 and 64).
      constexpr int VG = D == 128 ? 6 : 8;
#pragma unroll
      for (int i = 0; i < 2 * C::KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, VG, 0);  // then vector ALU work
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // At raised wave priority from head_dim 64 on: with two workgroups per
    // compute unit, the wave running this interleaved phase is served before
    // one running its PV products (at head_dim 32, three waves per SIMD, it
    // measured slower).
    if constexpr (D >= 64) __builtin_amdgcn_s_setprio(1);
    if (need_mask)
      body(std::true_type{});
    else
      body(std::false_type{});
    if constexpr (D >= 64) __builtin_amdgcn_s_setprio(0);
    if (any) {
#pragma unroll
      for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
    }
    pv(vc, pf);
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
    wait_vmem();
    __syncthreads();
  };

  // Stage roles alternate between iterations; unrolled by two so that every
  // LDS address is a constant offset from the lane's base.
  for (int j = 0; j < ntiles; j += 2) {
    step(j, k_s1, k_s0, v_s0, v_s1);
    if (j + 1 >= ntiles) break;
    step(j + 1, k_s0, k_s1, v_s1, v_s0);
  }

  const float ltot = half_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  // O goes to a bf16 tile in LDS (the K stages, whose last reads every wave
  // has passed: the loop ends on a barrier; the swizzled layout of the
  // copies) and from there to memory in whole rows, 16 bytes per lane, rather
  // than 8 bytes to each of 32 rows per instruction.
  const int lrow = 32 * wave + l32;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hh;
      const u32x2_t w = u32x2_t{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
      *(u32x2_t*)(kv_s + swz_off<D>(lrow, d)) = w;
    }
  if (row_ok && hh == 0) {
    const float lse = ltot > 0.f ? m * a.scale + __logf(ltot) : -INFINITY;
    a.lse[((long)b * a.Hq + h) * a.Tq + qrow] = lse;
  }
  __syncthreads();
  using Gm = TileGeom<D, C::BM, C::THREADS>;
  uint16_t* const obase = (uint16_t*)a.o + ((long)b * a.Tq * a.Hq + h) * D;
#pragma unroll
  for (int i = 0; i < Gm::ITERS; ++i) {
    const int r = Gm::row(i, wave, lane);
    if (q0 + r < a.Tq)
      *(u32x4_t*)(obase + Gm::elem(q0 + r, r, lane, qrs)) = lds_read16(kv_s + Gm::block(i, wave) * 512 + lane * 8);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int D, hipStream_t s) {
  const long blocks = (long)a.num_qtiles * a.Hq * a.B;
  if (blocks == 0) return hipSuccess;
  if (D == 32) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else if (D == 256) {
    launch_fwd_pair_bf16(a, s);
  } else if (D == 128) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
