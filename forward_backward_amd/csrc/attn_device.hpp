// Device helpers for the gfx950 (CDNA4) attention kernels.
//
// Lane layouts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16): lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]
//   B operand (16 x 32): lane l holds B[8*(l/32) .. +7][l % 32]
//   C/D (32 x 32, 16 fp32 per lane): register r of lane l is
//       C[8*(r/4) + 4*(l/32) + (r%4)][l % 32]
// The contraction index of an MFMA may be permuted freely as long as both
// operands agree; the kernels use that to feed the fp32 accumulator of one
// product straight into the next product as its B operand.
//
// ds_read_b64_tr_b16 (the LDS transpose read): within each group of 16
// lanes, lane j returns 4 elements; element e is element (j % 4) of the
// 8-byte chunk addressed by lane 4*e + j/4 of the same group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// D += A * B on bf16 operands held as raw 32-bit words.
__device__ __forceinline__ f32x16_t mfma_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Two fp32 values to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Transposed 4 x bf16 LDS read (see the header comment); `p` points into LDS.
__device__ __forceinline__ u32x2_t lds_read_tr(const uint16_t* p) {
  s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

#ifdef ATTN_DEBUG
// Debug build: this code object's table of valid byte ranges and its counters
// (accesses outside every range, the first such address). The host fills the
// table before each call's launches and reads the counters through the
// functions registered below (see attn_internal.h).
namespace dbg {
static __device__ DbgRange ranges[kDbgRanges];
static __device__ int nranges;
static __device__ unsigned long long counts[2];
__device__ __forceinline__ void check(const void* p, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(p);
  if (!dbg_in_ranges(a, bytes, ranges, nranges)) {
    atomicAdd(&counts[0], 1ull);
    atomicCAS(&counts[1], 0ull, a);
  }
}
static hipError_t set(const DbgRange* r, int n) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(ranges), r, sizeof(DbgRange) * n, 0, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(nranges), &n, sizeof(int), 0, hipMemcpyHostToDevice);
  return e;
}
static hipError_t take(unsigned long long* count, unsigned long long* first) {
  unsigned long long c[2] = {0, 0};
  hipError_t e = hipMemcpyFromSymbol(c, HIP_SYMBOL(counts), sizeof(c), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *count += c[0];
  if (*first == 0) *first = c[1];
  const unsigned long long z[2] = {0, 0};
  return hipMemcpyToSymbol(HIP_SYMBOL(counts), z, sizeof(z), 0, hipMemcpyHostToDevice);
}
static const int registered = dbg_register(&set, &take);
}  // namespace dbg
#define ATTN_DBG_CHECK(p, bytes) ::attn::dbg::check((p), (bytes))
#else
#define ATTN_DBG_CHECK(p, bytes) ((void)0)
#endif

__device__ __forceinline__ u32x4_t lds_read16(const uint16_t* p) { return *(const u32x4_t*)(p); }
__device__ __forceinline__ void lds_write16(uint16_t* p, u32x4_t v) { *(u32x4_t*)(p) = v; }
__device__ __forceinline__ u32x4_t gload16(const uint16_t* p) {
  ATTN_DBG_CHECK(p, 16);
  return *(const u32x4_t*)(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum with the lane 32 positions away (v_permlane32_swap).
__device__ __forceinline__ float half_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Partial of D = rowsum(dO * O) over one lane's half of a bf16 row: the
// 16-byte chunks t = 0 .. KS - 1 at elements 16 t + 8 hh .. + 7 (the layout of
// the dQ kernel's Q/dO fragments), in one fixed chain of fused multiply-adds.
// D is the sum of the two halves' partials. The dQ kernel and the head_dim
// 64/128 pre-kernel both form D this way, so they agree bit for bit.
template <int KS>
__device__ __forceinline__ float row_dot_half(const u32x4_t (&o)[KS], const u32x4_t (&g)[KS]) {
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(bf16_lo(o[t][w]), bf16_lo(g[t][w]), acc);
      acc = __builtin_fmaf(bf16_hi(o[t][w]), bf16_hi(g[t][w]), acc);
    }
  return acc;
}

// Three bf16 terms whose sum is x to fp32 precision (each term is the
// round-to-nearest-even bf16 of what the previous ones left; every
// difference is exact in fp32).
__device__ __forceinline__ u32x2_t split_bf16x3(float x) {
  const float h = bf16_lo(pack_bf16(x, 0.f));
  const float r1 = x - h;
  const float m = bf16_lo(pack_bf16(r1, 0.f));
  const float r2 = r1 - m;
  return u32x2_t{pack_bf16(h, m), pack_bf16(r2, 0.f)};
}

// The backward's per-row statistics of row `st` ([B, Hq, Tq] index) from its
// D = rowsum(dO * O) and LSE: D, the base-2 LSE (LSE * log2(e)) that the tile
// kernels load, and the row terms the dK/dV kernel adds to S and dP with one
// extra matrix k-step: -LSE/scale (so that scale * log2(e) * (S - LSE/scale)
// is the base-2 exponent of P) and -D, each as three bf16 terms. Rows without
// a finite LSE (no valid key) get 0 terms; no kernel forms P for them.
__device__ __forceinline__ void write_row_stats(const BwdArgs& a, long st, float dsum, float lse) {
  a.delta[st] = dsum;
  a.lse2[st] = lse * 1.4426950408889634f;
  const float x = __builtin_isfinite(lse) ? -lse / a.scale : 0.f;
  const u32x2_t xs = split_bf16x3(x), ys = split_bf16x3(-dsum);
  *(u32x4_t*)(a.rowstat + st * 8) = u32x4_t{xs[0], xs[1], ys[0], ys[1]};
}

// LDS bank model used for layouts (measured with the bank-conflict counter):
// 64 banks of 4 bytes; a 128-bit read serves 16 lanes per cycle, the 64-bit
// transpose read 32 lanes per cycle.
//
// Tiles read both row-wise (16-byte chunks, 16 consecutive rows per cycle)
// and with the transpose read (4 consecutive rows x 64 bytes per cycle) use
// an unpadded row stride of D elements and store logical 16-byte chunk c of
// row r at physical chunk c ^ swz_f(r). swz_f takes 16 (D=128) or 8 (D=64,
// two rows per bank line) distinct values over consecutive rows, and gives
// the 4 rows of a transpose read disjoint groups of 4 chunks. At D=32 four
// rows share a bank line: rows of equal r % 4 get distinct chunks through
// (r >> 2) & 3, and a transpose read's 4 consecutive rows never collide.
// At D=256 a row spans two bank lines and the D=128 pattern applies to the
// low four bits of the chunk index.
template <int D>
__host__ __device__ __forceinline__ int swz_f(int r) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head_dim 32, 64, 128 or 256");
  if constexpr (D >= 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else if constexpr (D == 64) {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  } else {
    return (r >> 2) & 3;
  }
}

// Element offset of logical (row, col) in a swizzled tile; col % 4 == 0.
template <int D>
__host__ __device__ __forceinline__ int swz_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz_f<D>(r))) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((const lds_void_t*)p));
}

// global_load_lds_dword{,x4}: lane i's 4 or 16 bytes land at LDS address
// m0 + (4 or 16) * i. Issued as inline assembly so that the compiler does not
// treat the copy as an LDS store that later LDS reads of *other* buffers
// must wait for; the kernels order the copy themselves: the destination is
// read only after s_waitcnt vmcnt(0) (wait_vmem) and a workgroup barrier.
// Loads complete in order, so the compiler's own vmcnt waits for other loads
// stay correct (they can only wait longer).
// M0 is saved and restored around the copy (the compiler neither knows nor
// expects it to change); the LDS address must be wave-uniform and is moved
// into a scalar register first.
//
// NT = true marks the copy non-temporal (the nt cache policy): for data read
// exactly once, such as a decode's KV cache, which then does not compete for
// the L2 with other streams.
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  ATTN_DBG_CHECK(g, 16);
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(base)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(base)
        : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  ATTN_DBG_CHECK(g, 4);
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(base)
      : "memory");
}

// Geometry of the copy of a swizzled [ROWS, D] bf16 tile by THREADS threads:
// each wave copies 1 KiB blocks, one 16-byte chunk per lane, lane i of a
// block landing at LDS byte 16 i of it. Copy i of wave w fills block
// i * WAVES + w; a lane fetches the logical chunk that the swizzle puts at its
// physical place. Shared by the copy paths below and by a host-compiled
// bounds model in the tests.
template <int D, int ROWS, int THREADS>
struct TileGeom {
  static constexpr int RPW = 1024 / (2 * D);  // rows per block
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int WAVES = THREADS / 64;
  static constexpr int ITERS = ROWS / (RPW * WAVES);
  static_assert(ROWS % (RPW * WAVES) == 0, "tile rows must split evenly over the waves");
  __host__ __device__ static int block(int i, int wave) { return i * WAVES + wave; }
  __host__ __device__ static int row(int i, int wave, int lane) { return block(i, wave) * RPW + lane / CPR; }
  __host__ __device__ static int chunk(int r, int lane) { return (lane % CPR) ^ swz_f<D>(r); }
  // Element offset of the lane's chunk in row `gr` of a matrix with row stride rs.
  __host__ __device__ static long elem(long gr, int r, int lane, long rs) { return gr * rs + chunk(r, lane) * 8; }
  // Byte offset of the lane's chunk from the tile's first row (32 bits: the
  // API bounds heads * head_dim, so (ROWS - 1) * rs * 2 + 2 * D < 2^32).
  __host__ __device__ static uint32_t voff(int i, int wave, int lane, long rs) {
    const int r = row(i, wave, lane);
    return static_cast<uint32_t>(elem(r, r, lane, rs) * 2);
  }
  // Row a lane of a partial tile reads: rows at or past rlim (>= 1) re-read rlim - 1.
  __host__ __device__ static int clamp_row(int r0, int r, int rlim) {
    const int gr = r0 + r;
    return gr < rlim ? gr : rlim - 1;
  }
};

// A 64-bit address from its two 32-bit halves, each taken as unsigned (the
// halves come back from readfirstlane as signed ints; a signed widening of the
// low half would spread its bit 31 over the high half).
__host__ __device__ __forceinline__ uint64_t join_halves(uint32_t lo, uint32_t hi) {
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Asynchronous global -> LDS copy of rows [r0, r0 + ROWS) of a bf16 matrix
// with row stride `rs` elements into a swizzled [ROWS, D] LDS tile, by the
// THREADS threads of the workgroup: each wave copies 1 KiB per instruction,
// and the swizzle is realised by choosing which logical chunk each lane
// fetches. Rows at or past `rlim` (>= 1) re-read row rlim - 1: the caller
// masks their contribution, and nothing outside the valid rows is read.
// VISIBLE = true issues the copy through the compiler builtin instead, so the
// compiler orders later LDS reads after it itself (it cannot tell stages of
// one array apart and waits before transpose reads in particular).
template <int D, int ROWS, int THREADS, bool VISIBLE = false, bool NT = false>
__device__ __forceinline__ void dma_tile(uint16_t* tile, const uint16_t* g, long rs, int r0, int rlim, int tid) {
  using Gm = TileGeom<D, ROWS, THREADS>;
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < Gm::ITERS; ++i) {
    const int r = Gm::row(i, wave, lane);
    const uint16_t* src = g + Gm::elem(Gm::clamp_row(r0, r, rlim), r, lane, rs);
    uint16_t* dst = tile + Gm::block(i, wave) * 512;
    if constexpr (VISIBLE) {
      ATTN_DBG_CHECK(src, 16);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)dst, 16, 0, 0);
    }
    else
      dma16<NT>(src, lds_addr(dst));
  }
}

// Copy with a wave-uniform 64-bit base (scalar registers) and a per-lane
// 32-bit byte offset: the address arithmetic is one scalar add per tile.
// The base is made explicitly wave-uniform (both halves through
// readfirstlane) so that it always lands in scalar registers. readfirstlane
// returns a signed int: each half is taken back as uint32_t before widening,
// or a low half with bit 31 set would sign-extend over the high half.
template <bool NT = false>
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const void* sbase = reinterpret_cast<const void*>(join_halves(lo, hi));
  ATTN_DBG_CHECK(static_cast<const char*>(sbase) + voff, 16);
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}

// Batched dma16_s: the ITERS copies of one tile (lane byte offsets voff[i],
// LDS destinations lds + i * STEP) from base_a and, with TWO, the same copies
// of a second tile from base_b to lds + AB + i * STEP, in one inline-asm
// block, so that M0 is saved and restored once per batch and each further
// destination is one scalar add of an immediate. lds must be wave-uniform.
#define ATTN_DMA_AT(v, b) "s_nop 0\n\tglobal_load_lds_dwordx4 %[" v "], %[" b "]" ATTN_DMA_POL "\n\t"
#define ATTN_DMA_STEP(d) "s_add_u32 m0, m0, %[" d "]\n\t"
#define ATTN_DMA_POL ""
#define ATTN_DMA_NT false
#define DMA16_BATCH_NAME dma16_batch_plain
template <int ITERS, int STEP, bool TWO, int AB = 0>
__device__ __forceinline__ void DMA16_BATCH_NAME(const void* base_a, const void* base_b, const uint32_t (&voff)[ITERS],
                                            uint32_t lds) {
  if constexpr (ITERS != 2 && ITERS != 4) {
    // Other counts (head_dim 32 and 256 tiles of some kernels): one copy at a time.
#pragma unroll
    for (int i = 0; i < ITERS; ++i) dma16_s<ATTN_DMA_NT>(base_a, voff[i], lds + i * STEP);
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) dma16_s<ATTN_DMA_NT>(base_b, voff[i], lds + AB + i * STEP);
    }
    return;
  }
  auto uniform = [](const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32)));
    return reinterpret_cast<const void*>(join_halves(lo, hi));
  };
  const void* sa = uniform(base_a);
#ifdef ATTN_DEBUG
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    ATTN_DBG_CHECK(static_cast<const char*>(sa) + voff[i], 16);
    if constexpr (TWO) ATTN_DBG_CHECK(static_cast<const char*>(uniform(base_b)) + voff[i], 16);
  }
#endif
  const uint32_t l0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
  uint32_t saved;
  if constexpr (ITERS == 2 && !TWO) {
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [a] "s"(sa), [l0] "s"(l0), [st] "n"(STEP)
                 : "memory");
  } else if constexpr (ITERS == 2 && TWO) {
    const void* sb = uniform(base_b);
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("ab") ATTN_DMA_AT("v0", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "b") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [a] "s"(sa), [b] "s"(sb), [l0] "s"(l0), [st] "n"(STEP),
                   [ab] "n"(AB - STEP)
                 : "memory");
  } else if constexpr (ITERS == 4 && !TWO) {
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "a") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]), [a] "s"(sa),
                   [l0] "s"(l0), [st] "n"(STEP)
                 : "memory");
  } else if constexpr (ITERS == 4 && TWO) {
    const void* sb = uniform(base_b);
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "a") ATTN_DMA_STEP("ab") ATTN_DMA_AT("v0", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "b") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "b") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]), [a] "s"(sa),
                   [b] "s"(sb), [l0] "s"(l0), [st] "n"(STEP), [ab] "n"(AB - 3 * STEP)
                 : "memory");
  }
}
#undef DMA16_BATCH_NAME
#undef ATTN_DMA_NT
#undef ATTN_DMA_POL
#define ATTN_DMA_POL " nt"
#define ATTN_DMA_NT true
#define DMA16_BATCH_NAME dma16_batch_nt
template <int ITERS, int STEP, bool TWO, int AB = 0>
__device__ __forceinline__ void DMA16_BATCH_NAME(const void* base_a, const void* base_b, const uint32_t (&voff)[ITERS],
                                            uint32_t lds) {
  if constexpr (ITERS != 2 && ITERS != 4) {
    // Other counts (head_dim 32 and 256 tiles of some kernels): one copy at a time.
#pragma unroll
    for (int i = 0; i < ITERS; ++i) dma16_s<ATTN_DMA_NT>(base_a, voff[i], lds + i * STEP);
    if constexpr (TWO) {
#pragma unroll
      for (int i = 0; i < ITERS; ++i) dma16_s<ATTN_DMA_NT>(base_b, voff[i], lds + AB + i * STEP);
    }
    return;
  }
  auto uniform = [](const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32)));
    return reinterpret_cast<const void*>(join_halves(lo, hi));
  };
  const void* sa = uniform(base_a);
#ifdef ATTN_DEBUG
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    ATTN_DBG_CHECK(static_cast<const char*>(sa) + voff[i], 16);
    if constexpr (TWO) ATTN_DBG_CHECK(static_cast<const char*>(uniform(base_b)) + voff[i], 16);
  }
#endif
  const uint32_t l0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
  uint32_t saved;
  if constexpr (ITERS == 2 && !TWO) {
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [a] "s"(sa), [l0] "s"(l0), [st] "n"(STEP)
                 : "memory");
  } else if constexpr (ITERS == 2 && TWO) {
    const void* sb = uniform(base_b);
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("ab") ATTN_DMA_AT("v0", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "b") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [a] "s"(sa), [b] "s"(sb), [l0] "s"(l0), [st] "n"(STEP),
                   [ab] "n"(AB - STEP)
                 : "memory");
  } else if constexpr (ITERS == 4 && !TWO) {
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "a") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]), [a] "s"(sa),
                   [l0] "s"(l0), [st] "n"(STEP)
                 : "memory");
  } else if constexpr (ITERS == 4 && TWO) {
    const void* sb = uniform(base_b);
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[l0]\n\t" ATTN_DMA_AT("v0", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "a") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "a") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "a") ATTN_DMA_STEP("ab") ATTN_DMA_AT("v0", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v1", "b") ATTN_DMA_STEP("st") ATTN_DMA_AT("v2", "b") ATTN_DMA_STEP("st")
                 ATTN_DMA_AT("v3", "b") "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [v0] "v"(voff[0]), [v1] "v"(voff[1]), [v2] "v"(voff[2]), [v3] "v"(voff[3]), [a] "s"(sa),
                   [b] "s"(sb), [l0] "s"(l0), [st] "n"(STEP), [ab] "n"(AB - 3 * STEP)
                 : "memory");
  }
}
#undef DMA16_BATCH_NAME
#undef ATTN_DMA_NT
#undef ATTN_DMA_POL
// The batch with the default cache policy, or (NT) non-temporal as for dma16.
template <int ITERS, int STEP, bool TWO, int AB = 0, bool NT = false>
__device__ __forceinline__ void dma16_batch(const void* base_a, const void* base_b, const uint32_t (&voff)[ITERS],
                                            uint32_t lds) {
  if constexpr (NT)
    dma16_batch_nt<ITERS, STEP, TWO, AB>(base_a, base_b, voff, lds);
  else
    dma16_batch_plain<ITERS, STEP, TWO, AB>(base_a, base_b, voff, lds);
}
#undef ATTN_DMA_AT
#undef ATTN_DMA_STEP

// Precomputed form of dma_tile for full tiles (every row valid): the lane
// offsets (row * rs + swizzled chunk) are fixed at set-up, so each tile costs
// one uniform base pointer. Needs (ROWS - 1) * rs * 2 + 2 * D < 2^32 bytes.
template <int D, int ROWS, int THREADS>
struct TileCopy {
  using Gm = TileGeom<D, ROWS, THREADS>;
  static constexpr int RPW = Gm::RPW;
  static constexpr int CPR = Gm::CPR;
  static constexpr int WAVES = Gm::WAVES;
  static constexpr int ITERS = Gm::ITERS;
  uint32_t voff[ITERS];  // byte offset of this lane's chunk from the tile's first row
  uint32_t lds_wave;     // byte offset of this wave's first 1 KiB block in the tile (uniform)

  __device__ __forceinline__ TileCopy(long rs, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) voff[i] = Gm::voff(i, wave, lane, rs);
    lds_wave = __builtin_amdgcn_readfirstlane(wave * 1024);
  }

  // Rows [r0, r0 + ROWS) of g (row stride rs elements), all valid; g and r0
  // wave-uniform.
  __device__ __forceinline__ void copy(uint16_t* tile, const uint16_t* g, long rs, int r0) const {
    const uint16_t* base = g + (long)r0 * rs;
    const uint32_t l0 = lds_addr(tile) + lds_wave;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) dma16_s(base, voff[i], l0 + i * WAVES * 1024);
  }

  // Rows [r0, r0 + ROWS) of two matrices with the same row stride into two
  // tiles `ab_bytes` apart in LDS (tile_b = tile_a + AB bytes), one batch.
  template <int AB, bool NT = false>
  __device__ __forceinline__ void copy2(uint16_t* tile_a, const uint16_t* ga, const uint16_t* gb, long rs,
                                        int r0) const {
    const long off = (long)r0 * rs;
    dma16_batch<ITERS, WAVES * 1024, true, AB, NT>(ga + off, gb + off, voff, lds_addr(tile_a) + lds_wave);
  }
  // One tile, one batch.
  __device__ __forceinline__ void copy1(uint16_t* tile, const uint16_t* g, long rs, int r0) const {
    dma16_batch<ITERS, WAVES * 1024, false>(g + (long)r0 * rs, nullptr, voff, lds_addr(tile) + lds_wave);
  }

  // Same through the compiler builtin (see dma_tile's VISIBLE).
  __device__ __forceinline__ void copy_visible(uint16_t* tile, const uint16_t* g, long rs, int r0) const {
    const char* base = (const char*)(g + (long)r0 * rs);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      ATTN_DBG_CHECK(base + voff[i], 16);
      __builtin_amdgcn_global_load_lds((const void*)(base + voff[i]),
                                       (lds_void_t*)((char*)tile + lds_wave + i * WAVES * 1024), 16, 0, 0);
    }
  }
};

// Asynchronous copy of 64 consecutive floats (indices clamped to < lim, lim >= 1)
// into LDS by one wave.
__device__ __forceinline__ void dma_row64(float* dst, const float* g, int i0, int lim, int lane) {
  int i = i0 + lane;
  i = i < lim ? i : lim - 1;
  dma4(g + i, lds_addr(dst));
}

// Wait for this wave's outstanding global loads (including LDS DMA).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N), the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip; map the
// hardware id to a logical id so that each XCD gets a contiguous range of
// logical ids (neighbouring tiles of one head then share that XCD's L2).
// Index of the XCD (accelerator complex die) the calling wave runs on.
__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}

__host__ __device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcds = 8;
  const int q = n / kXcds, r = n % kXcds;
  const int x = bid % kXcds;
  const int start = x * q + (x < r ? x : r);
  return start + bid / kXcds;
}

// Order of a grid's tiles over the remapped workgroup ids: `nunits` units
// (a batch and head, say) of `ntiles` tiles each; returns the unit and the
// tile rank t (t = 0 is the unit's most expensive tile). Without causal
// masking every tile costs the same, and a unit's tiles stay adjacent so that
// the XCD running them shares the unit's K/V rows in its L2. With causal
// masking the costs fall linearly with t; issued unit by unit, a tile count
// per unit unequal to the number of workgroups resident on an XCD leaves long
// tiles for last (up to 1.5 times the balanced time in a list-scheduling
// model). So the units are cut into groups, one per XCD when their number is
// a multiple of 8, and each group issues its tiles rank by rank (longest
// first) across its units.
//
// Either way each XCD receives a contiguous share of the unit ids, and units
// can differ in cost (KV lengths per batch): the last batch's units would all
// land on the last XCDs. So the ids are dealt out to the XCDs in turn: with
// `together` consecutive units kept as one (the query heads of one KV head,
// which share its K/V rows in L2) and their number S a multiple of 8, the i-th
// super-unit of XCD x's share becomes super-unit x + 8 i.
__host__ __device__ __forceinline__ void tile_order(int bid, int ntiles, int nunits, bool longest_first, int& unit,
                                                    int& t, int together = 1) {
  if (!longest_first) {
    unit = bid / ntiles;
    t = bid % ntiles;
  } else {
    const int gsz = nunits >= 8 ? nunits / 8 : 1;     // units per group
    const int g = bid / (gsz * ntiles);
    const int gs = min(gsz, nunits - g * gsz);        // units in this group (the last may be short)
    const int p = bid - g * gsz * ntiles;
    t = p / gs;
    unit = g * gsz + p % gs;
  }
  const int nsu = together > 0 && nunits % together == 0 ? nunits / together : 0;
  if (nsu >= 8 && nsu % 8 == 0) {
    const int per = nsu / 8;                  // super-units per XCD
    const int su = unit / together;
    unit = ((su % per) * 8 + su / per) * together + unit % together;
  }
}

__host__ __device__ __forceinline__ int clamp_len(const int32_t* kv_lens, int b, int tkv) {
  if (kv_lens == nullptr) return tkv;
  int n = kv_lens[b];
  return n < 0 ? 0 : (n > tkv ? tkv : n);
}

// The keys query row i sees are key_lo(i) <= j <= key_hi(i): the AND of the
// KV length (j < kvlim), the causal mask (j <= i) and the local window
// (i - left <= j <= i + right; -1 = no bound on that side). Both bounds are
// non-decreasing in i, so a tile of rows [r0, r1] touches keys
// [key_lo(r0), key_hi(r1)] and every key of [key_lo(r1), key_hi(r0)].
__host__ __device__ __forceinline__ int key_lo(int i, int left) { return left < 0 ? 0 : max(i - left, 0); }
__host__ __device__ __forceinline__ int key_hi(int i, int kvlim, int causal, int right) {
  int hi = kvlim - 1;
  if (causal) hi = min(hi, i);
  if (right >= 0) hi = min(hi, i + right);
  return hi;
}

}  // namespace attn
