// Split-KV decode for few queries over a long KV cache, bf16, gfx950.
//
// probjax pages, "Attention performance", section "Grouped-query attention
// and decoding": with few queries the regular kernel only parallelises over
// batch x heads x query tiles; the split-KV forward instead splits the keys
// across workgroups, packs the query heads of a GQA group into one tile and
// combines the partial results with their log-sum-exp.
//
// Split kernel: one workgroup per (batch, KV head, split, 64 packed rows).
// Packed row p = i * G + g is query i of query head KV_head * G + g. Split s
// covers keys [s * L, min((s + 1) * L, kv_len[b])); splits past the length
// exit at once. Four waves: wave w handles packed rows 32 * (w % 2) .. + 31
// and key block w / 2 of every 64-key tile; the two waves of a row block
// merge their (max, sum, O) through LDS at the end. The partial output is
// written normalised, in fp32, with its natural-log LSE.
//
// Combine kernel: for each output row, the splits are merged in ascending
// order: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s. A row
// with no valid key gets O = 0 and LSE = -inf.
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct DecCfg {
  static constexpr int ROWS = 64;             // packed rows per workgroup
  static constexpr int BN = kDecodeTileN;     // 64 keys per tile
  static constexpr int THREADS = 256;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KSTRIDE = D + 8;
  static constexpr int VSTRIDE = D + 16;
  static constexpr int KTILE = BN * KSTRIDE;
  static constexpr int VTILE = BN * VSTRIDE;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BN * CPR / THREADS;
  static_assert(BN * CPR % THREADS == 0, "tile must split evenly");
  // LDS for the final merge: per row block, O (16 * DB floats per lane) plus max and sum.
  static constexpr int MERGE_FLOATS = 2 * 64 * (16 * DB + 2);
  static_assert(MERGE_FLOATS * 4 <= 2 * (KTILE + VTILE) * 2, "merge area must fit in the staging buffers");
};

template <int D>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(DecodeArgs a) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::KTILE + C::VTILE)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int rb = wave & 1;   // row block
  const int kk = wave >> 1;  // key block within each tile

  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const int nrb = (R + C::ROWS - 1) / C::ROWS;
  int id = blockIdx.x;
  const int rbi = id % nrb;
  id /= nrb;
  const int s = id % a.num_splits;
  id /= a.num_splits;
  const int kh = id % a.Hkv;
  const int b = id / a.Hkv;

  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kbeg = s * a.split_len;
  if (kbeg >= kvlim) return;  // the combine ignores splits past the length
  const int kend = min(kbeg + a.split_len, kvlim);
  const int ntiles = (kend - kbeg + C::BN - 1) / C::BN;

  const long krs = (long)a.Hkv * D;
  const uint16_t* kb = (const uint16_t*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const uint16_t* vb = (const uint16_t*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  const int prow = rbi * C::ROWS + 32 * rb + l32;  // packed row of this lane
  const bool row_ok = prow < R;
  u32x4_t qf[C::KS];
  {
    const int i = row_ok ? prow / G : 0;
    const int g = row_ok ? prow % G : 0;
    const uint16_t* qp = (const uint16_t*)a.q + (((long)b * a.Tq + i) * a.Hq + kh * G + g) * D;
#pragma unroll
    for (int t = 0; t < C::KS; ++t) qf[t] = row_ok ? gload16(qp + 16 * t + 8 * hh) : u32x4_t{0, 0, 0, 0};
  }

  f32x16_t o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;
  const float c = a.scale_log2;

  u32x4_t kr[C::CPT], vr[C::CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int ch = tid + C::THREADS * i;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      const int key = k0 + row;
      if (key < kend) {
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

  gload(kbeg);
  lstore(0);
  __syncthreads();

  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = kbeg + it * C::BN;
    if (it + 1 < ntiles) gload(k0 + C::BN);
    const uint16_t* kl = lds + (it & 1) * (C::KTILE + C::VTILE) + (32 * kk) * C::KSTRIDE;
    const uint16_t* vl = lds + (it & 1) * (C::KTILE + C::VTILE) + C::KTILE + (32 * kk) * C::VSTRIDE;

    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int t = 0; t < C::KS; ++t) sc = mfma_bf16(lds_read16(kl + l32 * C::KSTRIDE + 16 * t + 8 * hh), qf[t], sc);

    const int kblk = k0 + 32 * kk;
    if (kblk + 32 > kend) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kblk + 8 * (r >> 2) + 4 * hh + (r & 3);
        sc[r] = key < kend ? sc[r] : -INFINITY;
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
      const uint16_t* vrow = vl + (16 * u + tr_row) * C::VSTRIDE + tr_col;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const u32x2_t lo = lds_read_tr(vrow + 32 * db);
        const u32x2_t hi = lds_read_tr(vrow + 8 * C::VSTRIDE + 32 * db);
        o[db] = mfma_bf16(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pf, o[db]);
      }
    }

    if (it + 1 < ntiles) lstore((it + 1) & 1);
    __syncthreads();
  }

  // Merge the two key blocks of each row block (waves rb and rb + 2).
  float* mg = reinterpret_cast<float*>(lds) + rb * 64 * (16 * C::DB + 2);
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
    if (row_ok) {
      const long prt = (((long)b * a.Hkv + kh) * a.num_splits + s) * R + prow;
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
// elements per thread, splits merged in ascending order.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;
  const int G = a.Hq / a.Hkv;
  const int R = a.Tq * G;
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gt / TPR;  // ((b * Hkv + kh) * R + p)
  const int part = (int)(gt % TPR);
  if (row >= (long)a.B * a.Hkv * R) return;
  const int p = (int)(row % R);
  const int kh = (int)((row / R) % a.Hkv);
  const int b = (int)(row / ((long)R * a.Hkv));
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int nact = (kvlim + a.split_len - 1) / a.split_len;
  const long base = ((long)b * a.Hkv + kh) * a.num_splits * R + p;

  float lmax = -INFINITY;
  for (int s = 0; s < nact; ++s) lmax = fmaxf(lmax, a.part_lse[base + (long)s * R]);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (lmax != -INFINITY) {
    for (int s = 0; s < nact; ++s) {
      const long pr = base + (long)s * R;
      const float ls = a.part_lse[pr];
      const float w = ls == -INFINITY ? 0.f : __expf(ls - lmax);
      const f32x4_t v = *(const f32x4_t*)(a.part_o + pr * D + 4 * part);
      acc += w * v;
      tot += w;
    }
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
  const long nrb = (R + DecCfg<D>::ROWS - 1) / DecCfg<D>::ROWS;
  const long blocks = (long)a.B * a.Hkv * a.num_splits * nrb;
  hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  const long threads = (long)a.B * a.Hkv * R * (D / 4);
  hipLaunchKernelGGL(attn_decode_combine_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int D, hipStream_t s) {
  if (D == 128)
    launch_decode<128>(a, s);
  else
    launch_decode<64>(a, s);
  return hipGetLastError();
}

}  // namespace attn
