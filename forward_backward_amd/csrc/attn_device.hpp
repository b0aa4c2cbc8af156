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

__device__ __forceinline__ u32x4_t lds_read16(const uint16_t* p) { return *(const u32x4_t*)(p); }
__device__ __forceinline__ void lds_write16(uint16_t* p, u32x4_t v) { *(u32x4_t*)(p) = v; }
__device__ __forceinline__ u32x4_t gload16(const uint16_t* p) { return *(const u32x4_t*)(p); }

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

// Workgroups are dispatched round-robin over the 8 XCDs of the chip; map the
// hardware id to a logical id so that each XCD gets a contiguous range of
// logical ids (neighbouring tiles of one head then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcds = 8;
  const int q = n / kXcds, r = n % kXcds;
  const int x = bid % kXcds;
  const int start = x * q + (x < r ? x : r);
  return start + bid / kXcds;
}

__device__ __forceinline__ int clamp_len(const int32_t* kv_lens, int b, int tkv) {
  if (kv_lens == nullptr) return tkv;
  int n = kv_lens[b];
  return n < 0 ? 0 : (n > tkv ? tkv : n);
}

}  // namespace attn
