// fp32 path (forward and backward) on the fp32 matrix cores, and the
// backward pre-kernel of both dtypes.
//
// The fp32 path computes in true fp32: v_mfma_f32_32x32x2_f32 multiplies
// fp32 operands and accumulates in fp32 (no reduced-precision matrix format;
// the probjax pages note that TF32-class products cost about three decimal
// digits, "GPU and CPU performance", section "Methodology"). The pages list
// fp32 at head_dim 128 as a weak spot of their Triton kernel ("H100
// (Hopper)", section "Known issues on H100"); here fp32 gets its own tiles
// ("Attention performance", section "Tile selection": one tile table per
// dtype and head_dim).
//
// v_mfma_f32_32x32x2_f32 takes one fp32 value per lane for each operand:
//   A (32 x 2): lane l holds A[l % 32][l / 32]
//   B (2 x 32): lane l holds B[l / 32][l % 32]
//   C/D (32 x 32): register r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32]
//       (the layout of the bf16 product).
// With one contraction element per lane, a "transposed" operand is a plain
// row read: the product that consumes an accumulator as its B operand (P or
// dS) takes register t as k-step t, so lane l's k-index is the accumulator
// row 8*(t/4) + 4*(l/32) + t%4, and its A operand is that row of V, K, Q or
// dO at the lane's output column. Output columns are permuted so that each
// lane reads NB = D/32 consecutive values of one row: row i of output block
// db is head_dim index NB*i + db. Over head_dim the contraction order is
// permuted the same way in both operands: k-step 4g + j of lane half h is
// index 8g + 4h + j, so each lane feeds four k-steps from one 16-byte read.
//
// Masks, tile ranges and the two-pass atomic-free backward follow the bf16
// kernels; every sum runs in a fixed order, so results are bitwise
// reproducible.
//
// The pre-kernel D = rowsum(dO * O) serves both dtypes.
#include "attn_device.hpp"
#include "attn_internal.h"

#include <type_traits>

namespace attn {
namespace {

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// fp32 tiles in LDS: unpadded rows of D floats, logical 16-byte chunk c of
// row r stored at physical chunk c ^ swz4_f(r). Two read patterns occur:
// 16 consecutive rows at one chunk (row operands over head_dim) and one or
// two rows read whole by 32 lanes (the NB-wide reads). With 64 banks of 4
// bytes, a row of D >= 64 floats starts at bank 0, so r & 15 gives 16
// consecutive rows distinct chunks mod 16; at D = 32 two rows share a bank
// line and (r >> 1) & 7 separates the rows of equal parity. Whole-row reads
// see a permutation of the chunks and stay conflict-free (at D = 32 the two
// rows of one read, four apart, share a bank half: a 2-way conflict).
template <int D>
__device__ __forceinline__ int swz4_f(int r) {
  static_assert(D == 32 || D == 64 || D == 128, "fp32 head_dim 32, 64 or 128");
  if constexpr (D >= 64)
    return r & 15;
  else
    return (r >> 1) & 7;
}

template <int D>
__device__ __forceinline__ int swz4_off(int r, int col) {
  return r * D + ((((col >> 2) ^ swz4_f<D>(r))) << 2) + (col & 3);
}

// N consecutive floats from LDS (N = 1, 2 or 4; naturally aligned).
template <int N>
__device__ __forceinline__ void lds_vec(const float* p, float (&v)[N]) {
  if constexpr (N == 4) {
    const f32x4_t x = *(const f32x4_t*)p;
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else if constexpr (N == 2) {
    const f32x2_t x = *(const f32x2_t*)p;
    v[0] = x[0]; v[1] = x[1];
  } else {
    v[0] = *p;
  }
}

// N consecutive floats to global memory.
template <int N>
__device__ __forceinline__ void store_vec(float* p, const float (&v)[N]) {
  if constexpr (N == 4)
    *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]};
  else if constexpr (N == 2)
    *(f32x2_t*)p = f32x2_t{v[0], v[1]};
  else
    *p = v[0];
}

// Asynchronous global -> LDS copy of rows [r0, r0 + ROWS) of an fp32 matrix
// (row stride rs floats) into a swizzled [ROWS, D] tile; each wave copies
// 1 KiB per instruction and realises the swizzle by choosing which logical
// chunk each lane fetches. Rows at or past rlim (>= 1) re-read row rlim - 1.
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void dma_tile_f32(float* tile, const float* g, long rs, int r0, int rlim, int tid) {
  constexpr int CPR = D / 4;     // chunks per row
  constexpr int RPW = 64 / CPR;  // rows per wave instruction
  constexpr int WAVES = THREADS / 64;
  constexpr int ITERS = ROWS / (RPW * WAVES);
  static_assert(ROWS % (RPW * WAVES) == 0, "tile rows must split evenly over the waves");
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int wi = i * WAVES + wave;
    const int r = wi * RPW + lane / CPR;
    const int c = (lane % CPR) ^ swz4_f<D>(r);
    int gr = r0 + r;
    gr = gr < rlim ? gr : rlim - 1;
    dma16(g + gr * rs + c * 4, lds_addr(tile + wi * 256));
  }
}

// dma_tile_f32 for full tiles with the lane offsets fixed at set-up (one
// uniform base pointer per tile). Needs (ROWS - 1) * rs * 4 + 4 * D < 2^32.
template <int D, int ROWS, int THREADS>
struct TileCopyF32 {
  static constexpr int CPR = D / 4;
  static constexpr int RPW = 64 / CPR;
  static constexpr int WAVES = THREADS / 64;
  static constexpr int ITERS = ROWS / (RPW * WAVES);
  static_assert(ROWS % (RPW * WAVES) == 0, "tile rows must split evenly over the waves");
  uint32_t voff[ITERS];
  uint32_t lds_wave;

  __device__ __forceinline__ TileCopyF32(long rs, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int r = (i * WAVES + wave) * RPW + lane / CPR;
      const int c = (lane % CPR) ^ swz4_f<D>(r);
      voff[i] = (uint32_t)((r * rs + c * 4) * 4);
    }
    lds_wave = __builtin_amdgcn_readfirstlane(wave * 1024);
  }

  __device__ __forceinline__ void copy(float* tile, const float* g, long rs, int r0) const {
    const float* base = g + (long)r0 * rs;
    const uint32_t l0 = lds_addr(tile) + lds_wave;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) dma16_s(base, voff[i], l0 + i * WAVES * 1024);
  }
};

// Scheduling fence: the unrolled product loops below read one group ahead of
// the matrix core and fence each group, which bounds the registers that
// hoisted LDS reads would otherwise take (one fp32 MFMA runs 64 cycles, so a
// one-group lead covers the LDS latency).
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

constexpr float kRescaleLog2F32 = 8.f;  // rescale O only when a row max grows by > 2^8

// --------------------------------------------------------------- forward

template <int D>
struct F32FwdCfg {
  static constexpr int BM = kFwdBlockM;       // 128 query rows, 32 per wave
  // Keys per tile: two 32-key blocks up to head_dim 64; one at 128, so that
  // the K/V rings take 64 KiB and two workgroups share a compute unit.
  static constexpr int NX = D > 64 ? 1 : 2;
  static constexpr int BN = 32 * NX;
  static constexpr int THREADS = 256;
  static constexpr int KG = D / 8;            // 16-byte reads per lane over head_dim
  static constexpr int NB = D / 32;           // output blocks over head_dim
  static constexpr int NO = NB > 1 ? NB : 2;  // O^T accumulators (two partial sums at D = 32)
  static constexpr int TILE = BN * D;
};

// One workgroup = 4 waves = 128 query rows of one (batch, head). Per key
// tile (64 keys, 32 at head_dim 128): S^T = K Q^T (lane = query row, Q in registers as the B operand), the
// online softmax in base 2 with lazy rescaling (as the bf16 forward), then
// O^T += V^T P^T with P straight from the S accumulators. K and V stream
// through two-stage LDS rings, K one tile ahead; the next tile's S^T is
// issued before the current tile's softmax so the two overlap.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_f32_kernel(FwdArgs a) {
  using C = F32FwdCfg<D>;
  // K stages 0 and 1, then V stages 0 and 1. Stages are picked at run time:
  // with constant stage addresses the compiler keeps a copy of every lane
  // offset per stage (offsets past 64 KiB do not fit the read's immediate).
  __shared__ __attribute__((aligned(16))) float tiles[4 * C::TILE];
  float* const k_st = tiles;
  float* const v_st = tiles + 2 * C::TILE;

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
  const float* qb = (const float*)a.q + ((long)b * a.Tq * a.Hq + h) * D;
  const float* kb = (const float*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const float* vb = (const float*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  const TileCopyF32<D, C::BN, C::THREADS> kvcopy(krs, tid);
  auto issue = [&](int j, float* dst, const float* src) {
    const int k0 = (j0 + j) * C::BN;
    if (k0 + C::BN <= kv_end)
      kvcopy.copy(dst, src, krs, k0);
    else
      dma_tile_f32<D, C::BN, C::THREADS>(dst, src, krs, k0, kv_end, tid);
  };
  if (ntiles > 0) {
    issue(0, k_st, kb);
    issue(0, v_st, vb);
    if (ntiles > 1) issue(1, k_st + C::TILE, kb);
  }

  const int qrow = q0 + 32 * wave + l32;
  const bool row_ok = qrow < a.Tq;
  // Q as the B operand of S^T = K Q^T: k-step 4g + j is Q[qrow][8g + 4hh + j].
  float qf[D / 2];
#pragma unroll
  for (int g = 0; g < C::KG; ++g) {
    const f32x4_t x = row_ok ? *(const f32x4_t*)(qb + qrow * qrs + 8 * g + 4 * hh) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[4 * g + j] = x[j];
  }
  // Take Q before the loop (the compiler cannot see the tile copies; a
  // first use inside the loop would wait for all loads on every pass).
#pragma unroll
  for (int i = 0; i < D / 2; ++i) asm volatile("" ::"v"(qf[i]));

  f32x16_t o[C::NO];
#pragma unroll
  for (int i = 0; i < C::NO; ++i) o[i] = f32x16_t{};
  float m = -INFINITY;
  float lsum = 0.f;

  const float c = a.scale_log2;
  const int wave_min_row = q0 + 32 * wave;
  const int row_lo = key_lo(qrow, a.win_left);
  const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
  const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
  const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);

  // Lane offsets. Head_dim groups g and g + 8 (head_dim 128) lie 64 elements
  // apart under the same swizzle, and so do rows t and t + 8 of a block
  // (16 rows), so eight of each are kept.
  constexpr int NG = C::KG < 8 ? C::KG : 8;
  int nrm8[NG], vrd8[8];
#pragma unroll
  for (int g = 0; g < NG; ++g) nrm8[g] = swz4_off<D>(l32, 8 * g + 4 * hh);
#pragma unroll
  for (int t = 0; t < 8; ++t) vrd8[t] = swz4_off<D>(8 * (t >> 2) + 4 * hh + (t & 3), C::NB * l32);
  auto nrm = [&](int g) { return nrm8[g & 7] + (g >> 3) * 64; };
  auto vrd = [&](int t) { return vrd8[t & 7] + (t >> 3) * 16 * D; };

  // S^T of the tile's key blocks (with one block the products form one chain;
  // the second workgroup on the SIMD fills its gaps).
  auto sdot = [&](const float* kl, f32x16_t (&s)[C::NX]) {
    f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
    f32x4_t n0 = *(const f32x4_t*)(kl + nrm(0));
    f32x4_t n1 = *(const f32x4_t*)(kl + (C::NX - 1) * 32 * D + nrm(0));
#pragma unroll
    for (int g = 0; g < C::KG; ++g) {
      const f32x4_t k0v = n0, k1v = n1;
      if (g + 1 < C::KG) {
        n0 = *(const f32x4_t*)(kl + nrm(g + 1));
        if constexpr (C::NX == 2) n1 = *(const f32x4_t*)(kl + 32 * D + nrm(g + 1));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (C::NX == 2) {
          acc[0] = mfma_f32(k0v[j], qf[4 * g + j], acc[0]);
          acc[1] = mfma_f32(k1v[j], qf[4 * g + j], acc[1]);
        } else {
          acc[0] = mfma_f32(k0v[j], qf[4 * g + j], acc[0]);
        }
      }
      fence();
    }
    if constexpr (C::NX == 2) {
      s[0] = acc[0];
      s[C::NX - 1] = acc[1];
    } else {
      s[0] = acc[0];
    }
  };

  // S -> P (unnormalised) in place; returns whether O must be rescaled by
  // alpha (wave-uniform).
  auto softmax = [&](auto mask_tag, int j, f32x16_t (&s)[C::NX], float& alpha) -> bool {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = (j0 + j) * C::BN;
    if constexpr (MASK) {
#pragma unroll
      for (int x = 0; x < C::NX; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * x + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = key >= row_lo && key <= row_hi;
          s[x][r] = ok ? s[x][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int x = 0; x < C::NX; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[x][r]);
    mt = half_max(mt);
    const bool grow = (m == -INFINITY) ? (mt != -INFINITY) : ((mt - m) * c > kRescaleLog2F32);
    const bool any = __builtin_amdgcn_ballot_w64(grow) != 0;
    const float mnew = any ? fmaxf(m, mt) : m;
    alpha = (m == -INFINITY || !any) ? (m == -INFINITY ? 0.f : 1.f) : fast_exp2((m - mnew) * c);
    m = mnew;
    lsum *= alpha;
    const float nb = (m == -INFINITY) ? 0.f : -m * c;
    float ps = 0.f;
#pragma unroll
    for (int x = 0; x < C::NX; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[x][r], c, nb));
        s[x][r] = p;
        ps += p;
      }
    lsum += ps;
    return any;
  };

  auto pv = [&](const float* vl, const f32x16_t (&s)[C::NX]) {
    float n[C::NX][C::NB];
#pragma unroll
    for (int x = 0; x < C::NX; ++x) lds_vec<C::NB>(vl + 32 * x * D + vrd(0), n[x]);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float vv[C::NX][C::NB];
#pragma unroll
      for (int x = 0; x < C::NX; ++x)
#pragma unroll
        for (int e = 0; e < C::NB; ++e) vv[x][e] = n[x][e];
      if (t + 1 < 16) {
#pragma unroll
        for (int x = 0; x < C::NX; ++x) lds_vec<C::NB>(vl + 32 * x * D + vrd(t + 1), n[x]);
      }
#pragma unroll
      for (int x = 0; x < C::NX; ++x) {
        if constexpr (C::NB > 1) {
#pragma unroll
          for (int db = 0; db < C::NB; ++db) o[db] = mfma_f32(vv[x][db], s[x][t], o[db]);
        } else {
          o[x] = mfma_f32(vv[x][0], s[x][t], o[x]);
        }
      }
      fence();
    }
  };

  f32x16_t s_cur[C::NX], s_nxt[C::NX];
  if (ntiles > 0) {
    wait_vmem();
    __syncthreads();
    sdot(k_st, s_cur);
    __syncthreads();  // every wave has read K_0 before K_2 overwrites it
  }

  // Iteration j: copies of K_{j+2} and V_{j+1} start; S_{j+1} (on the last
  // tile a stale stage whose result is dropped) beside the softmax of tile
  // j; then O += P_j V_j.
  // Tile j's K and V sit in stage j % 2 of their rings.
  auto step = [&](int j) {
    const int cur = (j & 1) * C::TILE, nxt = C::TILE - cur;
    const float* kn = k_st + nxt;
    float* kfree = k_st + cur;
    const float* vc = v_st + cur;
    float* vfree = v_st + nxt;
    if (j + 2 < ntiles) issue(j + 2, kfree, kb);
    if (j + 1 < ntiles) issue(j + 1, vfree, vb);
    const int k0 = (j0 + j) * C::BN;
    const bool need_mask = (k0 < wave_all_lo) || (k0 + C::BN - 1 > wave_all_hi);
    float alpha;
    bool any;
    sdot(kn, s_nxt);
    if (need_mask)
      any = softmax(std::true_type{}, j, s_cur, alpha);
    else
      any = softmax(std::false_type{}, j, s_cur, alpha);
    if (any) {
#pragma unroll
      for (int i = 0; i < C::NO; ++i) o[i] *= alpha;
    }
    pv(vc, s_cur);
#pragma unroll
    for (int x = 0; x < C::NX; ++x) s_cur[x] = s_nxt[x];
    wait_vmem();
    __syncthreads();
  };

  for (int j = 0; j < ntiles; ++j) step(j);

  const float ltot = half_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (row_ok) {
    float* orow = (float*)a.o + ((long)b * a.Tq * a.Hq + h) * D + qrow * qrs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
      float w[C::NB];
      if constexpr (C::NB > 1) {
#pragma unroll
        for (int db = 0; db < C::NB; ++db) w[db] = o[db][r] * inv;
      } else {
        w[0] = (o[0][r] + o[1][r]) * inv;
      }
      store_vec<C::NB>(orow + C::NB * i, w);
    }
    if (hh == 0) {
      const float lse = ltot > 0.f ? m * a.scale + __logf(ltot) : -INFINITY;
      a.lse[((long)b * a.Hq + h) * a.Tq + qrow] = lse;
    }
  }
}

// -------------------------------------------------------------------- dQ

template <int D>
struct F32DqCfg {
  static constexpr int BM = kBwdBlockM;       // 128 query rows, 32 per wave
  static constexpr int NX = 2;                // 32-key blocks per tile
  static constexpr int BN = 32 * NX;
  static constexpr int THREADS = 256;
  static constexpr int KG = D / 8;
  static constexpr int NB = D / 32;
  static constexpr int NO = NB > 1 ? NB : 2;
  static constexpr int TILE = BN * D;
};

// One workgroup per (batch, head, 128 query rows); Q and dO in registers.
// Per 32-key block: S^T = K Q^T and dP^T = V dO^T (lane = query row),
// dS^T = P (dP - D), dQ^T += K^T dS^T with dS straight from the
// accumulators. Both blocks' products are issued before the first softmax so
// that the vector work overlaps the matrix core. K and V tiles stream through
// a two-stage LDS ring.
// Two workgroups per compute unit up to head_dim 64; at 128 Q, dO and dQ^T
// alone take 192 registers per lane.
template <int D>
__global__ __launch_bounds__(256, D > 64 ? 1 : 2) void attn_dq_f32_kernel(BwdArgs a) {
  using C = F32DqCfg<D>;
  // Stage s holds K at tiles + 2s TILE and V after it; stages are picked at
  // run time (see the forward).
  __shared__ __attribute__((aligned(16))) float tiles[4 * C::TILE];

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
  const float* kb = (const float*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const float* vb = (const float*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;

  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  const int kv_first = key_lo(q0, a.win_left);
  const int kv_end = key_hi(q0 + C::BM - 1, kvlim, a.causal, a.win_right) + 1;
  const int j0 = kv_first / C::BN;
  const int ntiles = kv_end > kv_first ? (kv_end + C::BN - 1) / C::BN - j0 : 0;

  const TileCopyF32<D, C::BN, C::THREADS> kvcopy(krs, tid);
  auto issue = [&](int it, float* ks, float* vs) {
    const int k0 = (j0 + it) * C::BN;
    if (k0 + C::BN <= kv_end) {
      kvcopy.copy(ks, kb, krs, k0);
      kvcopy.copy(vs, vb, krs, k0);
    } else {
      dma_tile_f32<D, C::BN, C::THREADS>(ks, kb, krs, k0, kv_end, tid);
      dma_tile_f32<D, C::BN, C::THREADS>(vs, vb, krs, k0, kv_end, tid);
    }
  };
  if (ntiles > 0) issue(0, tiles, tiles + C::TILE);

  const int qrow = q0 + 32 * wave + l32;
  const bool row_ok = qrow < a.Tq;
  float qf[D / 2], gf[D / 2];
#pragma unroll
  for (int g = 0; g < C::KG; ++g) {
    const long off = qoff + qrow * qrs + 8 * g + 4 * hh;
    const f32x4_t x = row_ok ? *(const f32x4_t*)((const float*)a.q + off) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const f32x4_t y = row_ok ? *(const f32x4_t*)((const float*)a.dout + off) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[4 * g + j] = x[j];
      gf[4 * g + j] = y[j];
    }
  }
  const long stat = ((long)b * a.Hq + h) * a.Tq + qrow;
  // Rows past Tq get P = 0 from an infinite LSE.
  const float lse2 = row_ok ? a.lse2[stat] : INFINITY;
  const float dlt = row_ok ? a.delta[stat] : 0.f;
#pragma unroll
  for (int i = 0; i < D / 2; ++i) asm volatile("" ::"v"(qf[i]), "v"(gf[i]));
  asm volatile("" ::"v"(lse2), "v"(dlt));
  const float c = a.scale_log2;

  f32x16_t acc[C::NO];
#pragma unroll
  for (int i = 0; i < C::NO; ++i) acc[i] = f32x16_t{};

  const int wave_min_row = q0 + 32 * wave;
  const int row_lo = key_lo(qrow, a.win_left);
  const int row_hi = key_hi(qrow, kvlim, a.causal, a.win_right);
  const int wave_all_lo = key_lo(wave_min_row + 31, a.win_left);
  const int wave_all_hi = key_hi(wave_min_row, kvlim, a.causal, a.win_right);
  // Lane offsets, eight of each (see the forward).
  constexpr int NG = C::KG < 8 ? C::KG : 8;
  int nrm8[NG], vrd8[8];
#pragma unroll
  for (int g = 0; g < NG; ++g) nrm8[g] = swz4_off<D>(l32, 8 * g + 4 * hh);
#pragma unroll
  for (int t = 0; t < 8; ++t) vrd8[t] = swz4_off<D>(8 * (t >> 2) + 4 * hh + (t & 3), C::NB * l32);
  auto nrm = [&](int g) { return nrm8[g & 7] + (g >> 3) * 64; };
  auto vrd = [&](int t) { return vrd8[t & 7] + (t >> 3) * 16 * D; };

  auto sdp = [&](const float* kl, const float* vl, int x, f32x16_t& s, f32x16_t& dp) {
    s = f32x16_t{};
    dp = f32x16_t{};
    const float* kx = kl + 32 * x * D;
    const float* vx = vl + 32 * x * D;
    f32x4_t nk = *(const f32x4_t*)(kx + nrm(0));
    f32x4_t nv = *(const f32x4_t*)(vx + nrm(0));
#pragma unroll
    for (int g = 0; g < C::KG; ++g) {
      const f32x4_t kv = nk, vv = nv;
      if (g + 1 < C::KG) {
        nk = *(const f32x4_t*)(kx + nrm(g + 1));
        nv = *(const f32x4_t*)(vx + nrm(g + 1));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = mfma_f32(kv[j], qf[4 * g + j], s);
        dp = mfma_f32(vv[j], gf[4 * g + j], dp);
      }
      fence();
    }
  };
  // S -> dS in place (masked entries select 0 before any product).
  auto softmax = [&](auto mask_tag, int kblk0, f32x16_t& s, const f32x16_t& dp) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
      if constexpr (MASK) {
        const int kk = kblk0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool ok = (kk >= row_lo) & (kk <= row_hi);
        p = ok ? p : 0.f;
      }
      s[r] = p * (dp[r] - dlt);
    }
  };
  auto dq = [&](const float* kl, int x, const f32x16_t& ds) {
    const float* kx = kl + 32 * x * D;
    float n[C::NB];
    lds_vec<C::NB>(kx + vrd(0), n);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float kv[C::NB];
#pragma unroll
      for (int e = 0; e < C::NB; ++e) kv[e] = n[e];
      if (t + 1 < 16) lds_vec<C::NB>(kx + vrd(t + 1), n);
      if constexpr (C::NB > 1) {
#pragma unroll
        for (int db = 0; db < C::NB; ++db) acc[db] = mfma_f32(kv[db], ds[t], acc[db]);
      } else {
        acc[t & 1] = mfma_f32(kv[0], ds[t], acc[t & 1]);
      }
      fence();
    }
  };

  auto compute = [&](int it, const float* kl, const float* vl) {
    const int k0 = (j0 + it) * C::BN;
    const bool mask_tile = (k0 < wave_all_lo) || (k0 + C::BN - 1 > wave_all_hi);
#pragma unroll
    for (int x = 0; x < C::NX; ++x) {
      f32x16_t s, dp;
      sdp(kl, vl, x, s, dp);
      if (mask_tile)
        softmax(std::true_type{}, k0 + 32 * x, s, dp);
      else
        softmax(std::false_type{}, k0 + 32 * x, s, dp);
      dq(kl, x, s);
    }
  };

  // Tile it: wait for its copies, then (once every wave is done with tile
  // it - 1) start the copy of tile it + 1 into the other stage.
  for (int it = 0; it < ntiles; ++it) {
    float* cur = tiles + (it & 1) * 2 * C::TILE;
    float* nxt = tiles + ((it + 1) & 1) * 2 * C::TILE;
    wait_vmem();
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1, nxt, nxt + C::TILE);
    compute(it, cur, cur + C::TILE);
  }

  if (row_ok) {
    float* dqrow = (float*)a.dq + qoff + qrow * qrs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
      float w[C::NB];
      if constexpr (C::NB > 1) {
#pragma unroll
        for (int db = 0; db < C::NB; ++db) w[db] = acc[db][r] * a.scale;
      } else {
        w[0] = (acc[0][r] + acc[1][r]) * a.scale;
      }
      store_vec<C::NB>(dqrow + C::NB * i, w);
    }
  }
}

// ----------------------------------------------------------------- dK/dV

template <int D>
struct F32DkvCfg {
  static constexpr int BN = kBwdBlockN;       // 128 keys, 32 per wave
  static constexpr int BM = 64;               // query rows per tile (two 32-row blocks)
  static constexpr int THREADS = 256;
  static constexpr int KG = D / 8;
  static constexpr int NB = D / 32;
  static constexpr int NO = NB > 1 ? NB : 2;
  static constexpr int TILE = BM * D;
};

// One workgroup per (batch, KV head, 128 keys); each wave holds K and V of
// its 32 keys in registers (B operands). The query rows of the G heads of
// the group are visited in a fixed order in 64-row tiles: per 32-row block
// S = Q K^T and dP = dO V^T (lane = key, registers = query rows),
// P = exp2(c S - LSE log2 e), dS = P (dP - D), dV^T += dO^T P and
// dK^T += Q^T dS with P and dS straight from the accumulators. Q, dO and the
// rows' LSE log2 e and D stream through a two-stage LDS ring.
template <int D>
__global__ __launch_bounds__(256, D > 64 ? 1 : 2) void attn_dkdv_f32_kernel(BwdArgs a) {
  using C = F32DkvCfg<D>;
  constexpr int STAGE = 2 * C::TILE + 2 * C::BM;  // Q, dO, LSE log2 e, D (floats)
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int kt, unit;  // rank 0: the first key tile, the most query rows when causal
  tile_order(bid, a.num_ktiles, a.B * a.Hkv, a.causal, unit, kt);
  const int kh = unit % a.Hkv;
  const int b = unit / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int k0 = kt * C::BN;
  const int wk0 = k0 + 32 * wave;
  const int key = wk0 + l32;

  const long krs = (long)a.Hkv * D;
  const long qrs = (long)a.Hq * D;
  const long kvoff = ((long)b * a.Tkv * a.Hkv + kh) * D;
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);

  f32x16_t dk[C::NO], dv[C::NO];
#pragma unroll
  for (int i = 0; i < C::NO; ++i) {
    dk[i] = f32x16_t{};
    dv[i] = f32x16_t{};
  }

  // Query rows that see some key of the tile: key_hi(i) >= k0 from i_lo on,
  // key_lo(i) <= the last valid key up to i_hi.
  const int kmax = min(k0 + C::BN, kvlim) - 1;
  int i_lo = a.causal ? k0 : 0;
  if (a.win_right >= 0) i_lo = max(i_lo, k0 - a.win_right);
  int i_hi = a.Tq - 1;
  if (a.win_left >= 0) i_hi = min(i_hi, kmax + a.win_left);
  const int qt_begin = i_lo / C::BM;
  const int nq = i_hi >= i_lo ? i_hi / C::BM + 1 - qt_begin : 0;
  const int ntiles = G * nq;

  if (k0 < kvlim && ntiles > 0) {
    const bool key_ok = key < kvlim;
    float kf[D / 2], vf[D / 2];
#pragma unroll
    for (int g = 0; g < C::KG; ++g) {
      const long off = kvoff + (long)key * krs + 8 * g + 4 * hh;
      const f32x4_t x = key_ok ? *(const f32x4_t*)((const float*)a.k + off) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      const f32x4_t y = key_ok ? *(const f32x4_t*)((const float*)a.v + off) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kf[4 * g + j] = x[j];
        vf[4 * g + j] = y[j];
      }
    }

    const TileCopyF32<D, C::BM, C::THREADS> qcopy(qrs, tid);
    // Tile t: head kh * G + t / nq, rows [q0, q0 + 64).
    auto issue = [&](int t, float* st) {
      const int hq = kh * G + t / nq;
      const int q0 = (qt_begin + t % nq) * C::BM;
      const float* qg = (const float*)a.q + ((long)b * a.Tq * a.Hq + hq) * D;
      const float* gg = (const float*)a.dout + ((long)b * a.Tq * a.Hq + hq) * D;
      if (q0 + C::BM <= a.Tq) {
        qcopy.copy(st, qg, qrs, q0);
        qcopy.copy(st + C::TILE, gg, qrs, q0);
      } else {
        dma_tile_f32<D, C::BM, C::THREADS>(st, qg, qrs, q0, a.Tq, tid);
        dma_tile_f32<D, C::BM, C::THREADS>(st + C::TILE, gg, qrs, q0, a.Tq, tid);
      }
      const long s0 = ((long)b * a.Hq + hq) * a.Tq;
      if (wave == 0) dma_row64(st + 2 * C::TILE, a.lse2 + s0, q0, a.Tq, lane);
      if (wave == 1) dma_row64(st + 2 * C::TILE + C::BM, a.delta + s0, q0, a.Tq, lane);
    };
    issue(0, smem);
#pragma unroll
    for (int i = 0; i < D / 2; ++i) asm volatile("" ::"v"(kf[i]), "v"(vf[i]));

    const float c = a.scale_log2;
    // Lane offsets, eight of each (see the forward).
    constexpr int NG = C::KG < 8 ? C::KG : 8;
    int nrm8[NG], vrd8[8];
#pragma unroll
    for (int g = 0; g < NG; ++g) nrm8[g] = swz4_off<D>(l32, 8 * g + 4 * hh);
#pragma unroll
    for (int t = 0; t < 8; ++t) vrd8[t] = swz4_off<D>(8 * (t >> 2) + 4 * hh + (t & 3), C::NB * l32);
    auto nrm = [&](int g) { return nrm8[g & 7] + (g >> 3) * 64; };
    auto vrd = [&](int t) { return vrd8[t & 7] + (t >> 3) * 16 * D; };

    auto sp = [&](const float* ql, const float* gl, int x, f32x16_t& s, f32x16_t& dp) {
      s = f32x16_t{};
      dp = f32x16_t{};
      const float* qx = ql + 32 * x * D;
      const float* gx = gl + 32 * x * D;
      f32x4_t nq = *(const f32x4_t*)(qx + nrm(0));
      f32x4_t ng = *(const f32x4_t*)(gx + nrm(0));
#pragma unroll
      for (int g = 0; g < C::KG; ++g) {
        const f32x4_t qv = nq, gv = ng;
        if (g + 1 < C::KG) {
          nq = *(const f32x4_t*)(qx + nrm(g + 1));
          ng = *(const f32x4_t*)(gx + nrm(g + 1));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s = mfma_f32(qv[j], kf[4 * g + j], s);
          dp = mfma_f32(gv[j], vf[4 * g + j], dp);
        }
        fence();
      }
    };
    // S -> P and dP -> dS in place for block x of the tile at row q0.
    auto softmax = [&](auto mask_tag, const float* stl, int q0, int x, f32x16_t& s, f32x16_t& dp) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4_t ls = *(const f32x4_t*)(stl + 32 * x + 8 * u + 4 * hh);
        const f32x4_t dl = *(const f32x4_t*)(stl + C::BM + 32 * x + 8 * u + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * u + e;
          float p = fast_exp2(__builtin_fmaf(s[r], c, -ls[e]));
          if constexpr (MASK) {
            const int q = q0 + 32 * x + 8 * u + 4 * hh + e;
            const bool ok = (q < a.Tq) & (key >= key_lo(q, a.win_left)) &
                            (key <= key_hi(q, kvlim, a.causal, a.win_right));
            p = ok ? p : 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - dl[e]);
        }
      }
    };
    auto dkdv = [&](const float* ql, const float* gl, int x, const f32x16_t& p, const f32x16_t& ds) {
      const float* qx = ql + 32 * x * D;
      const float* gx = gl + 32 * x * D;
      float ng[C::NB], nq[C::NB];
      lds_vec<C::NB>(gx + vrd(0), ng);
      lds_vec<C::NB>(qx + vrd(0), nq);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float gv[C::NB], qv[C::NB];
#pragma unroll
        for (int e = 0; e < C::NB; ++e) {
          gv[e] = ng[e];
          qv[e] = nq[e];
        }
        if (t + 1 < 16) {
          lds_vec<C::NB>(gx + vrd(t + 1), ng);
          lds_vec<C::NB>(qx + vrd(t + 1), nq);
        }
        if constexpr (C::NB > 1) {
#pragma unroll
          for (int db = 0; db < C::NB; ++db) {
            dv[db] = mfma_f32(gv[db], p[t], dv[db]);
            dk[db] = mfma_f32(qv[db], ds[t], dk[db]);
          }
        } else {
          dv[t & 1] = mfma_f32(gv[0], p[t], dv[t & 1]);
          dk[t & 1] = mfma_f32(qv[0], ds[t], dk[t & 1]);
        }
        fence();
      }
    };

    auto compute = [&](int t, const float* st) {
      const int q0 = (qt_begin + t % nq) * C::BM;
      const float* ql = st;
      const float* gl = st + C::TILE;
      const float* stl = st + 2 * C::TILE;
      // Every (row, key) pair of the tile and the wave visible: no mask.
      const bool full = (q0 + C::BM <= a.Tq) && key_lo(q0 + C::BM - 1, a.win_left) <= wk0 &&
                        key_hi(q0, kvlim, a.causal, a.win_right) >= wk0 + 31;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        f32x16_t s, dp;
        sp(ql, gl, x, s, dp);
        if (full)
          softmax(std::false_type{}, stl, q0, x, s, dp);
        else
          softmax(std::true_type{}, stl, q0, x, s, dp);
        dkdv(ql, gl, x, s, dp);
      }
    };

    for (int t = 0; t < ntiles; ++t) {
      float* cur = smem + (t & 1) * STAGE;
      float* nxt = smem + ((t + 1) & 1) * STAGE;
      wait_vmem();
      __syncthreads();  // tile t landed; every wave is done with tile t - 1
      if (t + 1 < ntiles) issue(t + 1, nxt);
      compute(t, cur);
    }
  }

  // dK^T / dV^T: register r of block db is head_dim index NB * i + db of
  // row i = 8(r/4) + 4hh + r%4, for the lane's key.
  if (key < a.Tkv) {
    float* dkrow = (float*)a.dk + kvoff + (long)key * krs;
    float* dvrow = (float*)a.dv + kvoff + (long)key * krs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
      float wk[C::NB], wv[C::NB];
      if constexpr (C::NB > 1) {
#pragma unroll
        for (int db = 0; db < C::NB; ++db) {
          wk[db] = dk[db][r] * a.scale;
          wv[db] = dv[db][r];
        }
      } else {
        wk[0] = (dk[0][r] + dk[1][r]) * a.scale;
        wv[0] = dv[0][r] + dv[1][r];
      }
      store_vec<C::NB>(dkrow + C::NB * i, wk);
      store_vec<C::NB>(dvrow + C::NB * i, wv);
    }
  }
}

// D[b, h, i] = sum_d dO[b, i, h, d] * O[b, i, h, d] in fp32 and the other
// per-row statistics of write_row_stats (head_dim 32 and 256, and fp32).
// Each thread reduces 8 contiguous elements; D/8 threads share a row.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void attn_delta_kernel(BwdArgs a, long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
  // The work counters of the dK/dV pass start at zero.
  if (blockIdx.x == 0 && threadIdx.x < kBwdQueueWords && a.queue != nullptr) a.queue[threadIdx.x] = 0u;
  const long row = gt / TPR;   // row index in [B, Tq, Hq] order
  const int part = (int)(gt % TPR);
  float acc = 0.f;
  if (row < rows) {
    const long off = row * D + part * 8;
    if (BF16) {
      const u32x4_t x = gload16((const uint16_t*)a.o + off);
      const u32x4_t y = gload16((const uint16_t*)a.dout + off);
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += bf16_lo(x[w]) * bf16_lo(y[w]) + bf16_hi(x[w]) * bf16_hi(y[w]);
    } else {
      const f32x4_t* xp = (const f32x4_t*)((const float*)a.o + off);
      const f32x4_t* yp = (const f32x4_t*)((const float*)a.dout + off);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const f32x4_t x = xp[w], y = yp[w];
        acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    const int h = (int)(row % a.Hq);
    const int i = (int)((row / a.Hq) % a.Tq);
    const int b = (int)(row / ((long)a.Hq * a.Tq));
    const long st = ((long)b * a.Hq + h) * a.Tq + i;
    write_row_stats(a, st, acc, a.lse[st]);
  }
}

// The same statistics at bf16 head_dim 64 and 128, with D formed as the dQ
// kernel forms it (row_dot_half: two threads per row, each one chain over its
// half of the row), so that the dQ pass that computes them itself
// (attn_bwd_dq_and_preprocess) writes the same bits.
template <int D>
__global__ __launch_bounds__(256) void attn_delta_rows_kernel(BwdArgs a, long rows) {
  constexpr int KS = D / 16;
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
  // The work counters of the dK/dV pass start at zero.
  if (blockIdx.x == 0 && threadIdx.x < kBwdQueueWords && a.queue != nullptr) a.queue[threadIdx.x] = 0u;
  const long row = gt >> 1;  // row index in [B, Tq, Hq] order
  const int hh = (int)(gt & 1);
  float p = 0.f;
  if (row < rows) {
    const uint16_t* o = (const uint16_t*)a.o + row * D + 8 * hh;
    const uint16_t* g = (const uint16_t*)a.dout + row * D + 8 * hh;
    u32x4_t of[KS], gf[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      of[t] = gload16(o + 16 * t);
      gf[t] = gload16(g + 16 * t);
    }
    p = row_dot_half<KS>(of, gf);
  }
  const float dsum = p + __shfl_xor(p, 1, 64);
  if (row < rows && hh == 0) {
    const int h = (int)(row % a.Hq);
    const int i = (int)((row / a.Hq) % a.Tq);
    const int b = (int)(row / ((long)a.Hq * a.Tq));
    const long st = ((long)b * a.Hq + h) * a.Tq + i;
    write_row_stats(a, st, dsum, a.lse[st]);
  }
}

template <int D>
void launch_delta(const BwdArgs& a, bool bf16, hipStream_t s) {
  const long rows = (long)a.B * a.Tq * a.Hq;
  if (bf16 && (D == 64 || D == 128)) {
    const long threads = rows * 2;
    const unsigned blocks = threads > 0 ? (unsigned)((threads + 255) / 256) : 1u;
    hipLaunchKernelGGL((attn_delta_rows_kernel<D == 64 ? 64 : 128>), dim3(blocks), dim3(256), 0, s, a, rows);
    return;
  }
  const long threads = rows * (D / 8);
  const unsigned blocks = threads > 0 ? (unsigned)((threads + 255) / 256) : 1u;  // one block zeroes the counters
  if (bf16)
    hipLaunchKernelGGL((attn_delta_kernel<D, true>), dim3(blocks), dim3(256), 0, s, a, rows);
  else
    hipLaunchKernelGGL((attn_delta_kernel<D, false>), dim3(blocks), dim3(256), 0, s, a, rows);
}

}  // namespace

void launch_delta_any(const BwdArgs& a, int D, bool bf16, hipStream_t s) {
  if ((long)a.B * a.Tq * a.Hq == 0 && a.queue == nullptr) return;
  if (D == 128)
    launch_delta<128>(a, bf16, s);
  else if (D == 256)
    launch_delta<256>(a, bf16, s);
  else if (D == 64)
    launch_delta<64>(a, bf16, s);
  else
    launch_delta<32>(a, bf16, s);
}

hipError_t launch_fwd_fp32(const FwdArgs& a, int D, hipStream_t s) {
  const long blocks = (long)a.num_qtiles * a.Hq * a.B;
  if (blocks == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (D == 64)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pass_fp32(const BwdArgs& a, int D, int pass, hipStream_t s) {
  if (pass == kBwdPre) {
    launch_delta_any(a, D, false, s);
  } else if (pass == kBwdDkdv) {
    const long blocks = (long)a.num_ktiles * a.Hkv * a.B;
    if (blocks > 0) {
      if (D == 128)
        hipLaunchKernelGGL(attn_dkdv_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
      else if (D == 64)
        hipLaunchKernelGGL(attn_dkdv_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(attn_dkdv_f32_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    }
  } else {
    const long blocks = (long)((a.Tq + kBwdBlockM - 1) / kBwdBlockM) * a.Hq * a.B;
    if (blocks > 0) {
      if (D == 128)
        hipLaunchKernelGGL(attn_dq_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
      else if (D == 64)
        hipLaunchKernelGGL(attn_dq_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(attn_dq_f32_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace attn
