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
// K/V tiles are double-buffered in LDS with a register prefetch of the next
// tile's global loads. Keys at or past min(Tkv, kv_len[b]) and, with causal
// masking, past the query tile are neither loaded nor computed; rows of a
// partially valid tile are masked element-wise and out-of-range K/V rows are
// zero-filled so that no stale value can reach the accumulators.
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr float kRescaleLog2 = 8.f;  // rescale O only when a row max grows by > 2^8

template <int D>
struct FwdCfg {
  static constexpr int BM = kFwdBlockM;       // 128 query rows
  static constexpr int BN = 64;               // keys per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;           // MFMA k-steps over head_dim
  static constexpr int DB = D / 32;           // 32-wide blocks of head_dim in O
  static constexpr int KSTRIDE = D + 8;       // LDS row stride of K (elements)
  static constexpr int VSTRIDE = D + 32;      // LDS row stride of V (elements)
  static constexpr int KTILE = BN * KSTRIDE;
  static constexpr int VTILE = BN * VSTRIDE;
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int CPT = BN * CPR / THREADS;  // chunks per thread per tile
  static_assert(BN * CPR % THREADS == 0, "tile must split evenly over the workgroup");
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::KTILE + C::VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = a.num_qtiles - 1 - (bid % a.num_qtiles);  // longest causal tiles first
  const int bh = bid / a.num_qtiles;
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
  int kv_end = kvlim;
  if (a.causal) kv_end = min(kv_end, q0 + C::BM);
  const int ntiles = (kv_end + C::BN - 1) / C::BN;

  const int qrow = q0 + 32 * wave + l32;
  const bool row_ok = qrow < a.Tq;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8hh .. +7].
  u32x4_t qf[C::KS];
#pragma unroll
  for (int t = 0; t < C::KS; ++t) {
    qf[t] = row_ok ? gload16(qb + qrow * qrs + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
  }

  f32x16_t o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16_t{};
  float m = -INFINITY;   // running max of raw scores S (scale applied in the exponent)
  float lsum = 0.f;      // this lane's share of the softmax denominator

  const float c = a.scale_log2;

  u32x4_t kr[C::CPT], vr[C::CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + C::THREADS * i;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      const int key = k0 + row;
      if (key < kv_end) {
        kr[i] = gload16(kb + key * krs + cc * 8);
        vr[i] = gload16(vb + key * krs + cc * 8);
      } else {
        kr[i] = u32x4_t{0, 0, 0, 0};
        vr[i] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* kl = lds + buf * (C::KTILE + C::VTILE);
    uint16_t* vl = kl + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + C::THREADS * i;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      lds_write16(kl + row * C::KSTRIDE + cc * 8, kr[i]);
      lds_write16(vl + row * C::VSTRIDE + cc * 8, vr[i]);
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  // Transpose-read addressing of V (see attn_device.hpp): lane supplies the
  // chunk of row (4*hh + (lane%16)/4) and columns 16*((lane/16)%2) + 4*(lane%4).
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wave_min_row = q0 + 32 * wave;

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = it * C::BN;
    if (it + 1 < ntiles) gload(k0 + C::BN);
    const uint16_t* kl = lds + (it & 1) * (C::KTILE + C::VTILE);
    const uint16_t* vl = kl + C::KTILE;

    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int t = 0; t < C::KS; ++t) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t kf = lds_read16(kl + (32 * j + l32) * C::KSTRIDE + 16 * t + 8 * hh);
        s[j] = mfma_bf16(kf, qf[t], s[j]);
      }
    }

    const bool need_mask = (k0 + C::BN > kvlim) || (a.causal && k0 + C::BN - 1 > wave_min_row);
    if (need_mask) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = key < kvlim && (!a.causal || key <= qrow);
          s[j][r] = ok ? s[j][r] : -INFINITY;
        }
      }
    }

    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[j][r]);
    mt = half_max(mt);
    // Lazy rescaling: the reference max m only moves when some row of the
    // wave would otherwise see exponentials above 2^kRescaleLog2 (or had no
    // valid key yet). Numerator and denominator share the reference, so the
    // result is the same; it only bounds P (kept <= 2^8, exact in bf16's range).
    const bool grow = (m == -INFINITY) ? (mt != -INFINITY) : ((mt - m) * c > kRescaleLog2);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - mnew) * c);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < C::DB; ++i) o[i] *= alpha;
      m = mnew;
    }
    const float nb = (m == -INFINITY) ? 0.f : -m * c;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[j][r], c, nb));
        s[j][r] = p;
        ps += p;
      }
    lsum += ps;

    // P (bf16) as the B operand of O^T += V^T P^T, one operand per 16 keys.
    u32x4_t pf[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r0 = 8 * u;
        pf[2 * j + u] = u32x4_t{pack_bf16(s[j][r0 + 0], s[j][r0 + 1]), pack_bf16(s[j][r0 + 2], s[j][r0 + 3]),
                                pack_bf16(s[j][r0 + 4], s[j][r0 + 5]), pack_bf16(s[j][r0 + 6], s[j][r0 + 7])};
      }

#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint16_t* vrow = vl + (16 * ks + tr_row) * C::VSTRIDE + tr_col;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2_t lo = lds_read_tr(vrow + 32 * db);
        const u32x2_t hi = lds_read_tr(vrow + 8 * C::VSTRIDE + 32 * db);
        const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        o[db] = mfma_bf16(vf, pf[ks], o[db]);
      }
    }

    if (it + 1 < ntiles) lstore((it + 1) & 1);
    __syncthreads();
  }

  const float ltot = half_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (row_ok) {
    uint16_t* ob = (uint16_t*)a.o + ((long)b * a.Tq * a.Hq + h) * D + qrow * qrs;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        const u32x2_t w = u32x2_t{pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                  pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        *(u32x2_t*)(ob + d) = w;
      }
    if (hh == 0) {
      const float lse = ltot > 0.f ? m * a.scale + __logf(ltot) : -INFINITY;
      a.lse[((long)b * a.Hq + h) * a.Tq + qrow] = lse;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int D, hipStream_t s) {
  const long blocks = (long)a.num_qtiles * a.Hq * a.B;
  if (blocks == 0) return hipSuccess;
  if (D == 128) {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
