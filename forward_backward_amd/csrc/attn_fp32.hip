// fp32 attention path (forward and backward) and the backward pre-kernel.
//
// The fp32 path is true fp32 arithmetic on the vector ALUs (no reduced
// precision matrix format; the probjax pages note that TF32-class matmuls
// cost about three decimal digits, "GPU and CPU performance", section
// "Methodology"). It is a correctness path for small problems: one wave per
// row, lanes over head_dim, dot products by wave reductions. It follows the
// same masking rules (KV length, causal, local window) and the same two-pass,
// atomic-free backward as the bf16 kernels, so it is deterministic too.
//
// The pre-kernel D = rowsum(dO * O) serves both dtypes.
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// One wave per (batch, head, query row); lane holds head_dim elements lane
// and lane + 64 (D = 128).
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_fp32_kernel(FwdArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const long row_id = blockIdx.x;  // (b * Hq + h) * Tq + i
  const int i = (int)(row_id % a.Tq);
  const int h = (int)((row_id / a.Tq) % a.Hq);
  const int b = (int)(row_id / ((long)a.Tq * a.Hq));
  const int kh = h / (a.Hq / a.Hkv);
  const float* qp = (const float*)a.q + (((long)b * a.Tq + i) * a.Hq + h) * D;
  const float* kp = (const float*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const float* vp = (const float*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const long krs = (long)a.Hkv * D;
  const int kv_begin = key_lo(i, a.win_left);
  const int kv_end = key_hi(i, clamp_len(a.kv_lens, b, a.Tkv), a.causal, a.win_right) + 1;

  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = qp[lane + 64 * e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;
  for (int j = kv_begin; j < kv_end; ++j) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part += q[e] * kp[j * krs + lane + 64 * e];
    const float s = wave_sum(part);
    const float mnew = fmaxf(m, s);
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2((m - mnew) * c);
    const float p = fast_exp2((s - mnew) * c);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + p * vp[j * krs + lane + 64 * e];
    m = mnew;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = (float*)a.o + (((long)b * a.Tq + i) * a.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) op[lane + 64 * e] = acc[e] * inv;
  if (lane == 0) a.lse[((long)b * a.Hq + h) * a.Tq + i] = l > 0.f ? m * a.scale + __logf(l) : -INFINITY;
}

// dQ: one wave per (batch, head, query row), keys in ascending order.
template <int D>
__global__ __launch_bounds__(64) void attn_dq_fp32_kernel(BwdArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const long row_id = blockIdx.x;
  const int i = (int)(row_id % a.Tq);
  const int h = (int)((row_id / a.Tq) % a.Hq);
  const int b = (int)(row_id / ((long)a.Tq * a.Hq));
  const int kh = h / (a.Hq / a.Hkv);
  const long qoff = (((long)b * a.Tq + i) * a.Hq + h) * D;
  const float* kp = (const float*)a.k + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const float* vp = (const float*)a.v + ((long)b * a.Tkv * a.Hkv + kh) * D;
  const long krs = (long)a.Hkv * D;
  const int kv_begin = key_lo(i, a.win_left);
  const int kv_end = key_hi(i, clamp_len(a.kv_lens, b, a.Tkv), a.causal, a.win_right) + 1;
  const long stat = ((long)b * a.Hq + h) * a.Tq + i;
  const float lse2 = a.lse[stat] * 1.4426950408889634f;
  const float dlt = a.delta[stat];
  const float c = a.scale_log2;

  float q[E], g[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ((const float*)a.q)[qoff + lane + 64 * e];
    g[e] = ((const float*)a.dout)[qoff + lane + 64 * e];
    acc[e] = 0.f;
  }
  for (int j = kv_begin; j < kv_end; ++j) {
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ps += q[e] * kp[j * krs + lane + 64 * e];
      pd += g[e] * vp[j * krs + lane + 64 * e];
    }
    const float s = wave_sum(ps);
    const float dp = wave_sum(pd);
    const float p = fast_exp2(s * c - lse2);
    const float ds = p * (dp - dlt);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ds * kp[j * krs + lane + 64 * e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) ((float*)a.dq)[qoff + lane + 64 * e] = acc[e] * a.scale;
}

// dK, dV: one wave per (batch, KV head, key row); query heads of the group
// in ascending order, then query rows in ascending order.
template <int D>
__global__ __launch_bounds__(64) void attn_dkdv_fp32_kernel(BwdArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const long row_id = blockIdx.x;  // (b * Hkv + kh) * Tkv + j
  const int j = (int)(row_id % a.Tkv);
  const int kh = (int)((row_id / a.Tkv) % a.Hkv);
  const int b = (int)(row_id / ((long)a.Tkv * a.Hkv));
  const int G = a.Hq / a.Hkv;
  const long koff = (((long)b * a.Tkv + j) * a.Hkv + kh) * D;
  const int kvlim = clamp_len(a.kv_lens, b, a.Tkv);
  float k[E], v[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = ((const float*)a.k)[koff + lane + 64 * e];
    v[e] = ((const float*)a.v)[koff + lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const float c = a.scale_log2;
  if (j < kvlim) {
    const long qrs = (long)a.Hq * D;
    for (int g = 0; g < G; ++g) {
      const int h = kh * G + g;
      const float* qp = (const float*)a.q + ((long)b * a.Tq * a.Hq + h) * D;
      const float* gp = (const float*)a.dout + ((long)b * a.Tq * a.Hq + h) * D;
      const long stat0 = ((long)b * a.Hq + h) * a.Tq;
      // Rows that see key j: key_hi(i) >= j from i_lo on, key_lo(i) <= j up to i_hi.
      int i_lo = a.causal ? j : 0;
      if (a.win_right >= 0) i_lo = max(i_lo, j - a.win_right);
      int i_hi = a.Tq - 1;
      if (a.win_left >= 0) i_hi = min(i_hi, j + a.win_left);
      for (int i = i_lo; i <= i_hi; ++i) {
        float ps = 0.f, pd = 0.f, qv[E], gv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          qv[e] = qp[i * qrs + lane + 64 * e];
          gv[e] = gp[i * qrs + lane + 64 * e];
          ps += qv[e] * k[e];
          pd += gv[e] * v[e];
        }
        const float s = wave_sum(ps);
        const float dp = wave_sum(pd);
        const float p = fast_exp2(s * c - a.lse[stat0 + i] * 1.4426950408889634f);
        const float ds = p * (dp - a.delta[stat0 + i]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dv[e] += p * gv[e];
          dk[e] += ds * qv[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ((float*)a.dk)[koff + lane + 64 * e] = dk[e] * a.scale;
    ((float*)a.dv)[koff + lane + 64 * e] = dv[e];
  }
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

// D[b, h, i] = sum_d dO[b, i, h, d] * O[b, i, h, d] in fp32, the base-2 LSE
// (LSE * log2(e)) that the tile kernels load straight into LDS, and the row
// terms the dK/dV kernel adds to S and dP with one extra matrix k-step:
// -LSE/scale (so that scale * log2(e) * (S - LSE/scale) is the base-2
// exponent of P) and -D, each as three bf16 terms. Rows without a finite LSE
// (no valid key) get 0; no kernel forms P for them.
// Each thread reduces 8 contiguous elements; D/8 threads share a row.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void attn_delta_kernel(BwdArgs a, long rows) {
  constexpr int TPR = D / 8;  // threads per row
  const long gt = (long)blockIdx.x * 256 + threadIdx.x;
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
    a.delta[st] = acc;
    const float lse = a.lse[st];
    a.lse2[st] = lse * 1.4426950408889634f;
    const float x = __builtin_isfinite(lse) ? -lse / a.scale : 0.f;
    const u32x2_t xs = split_bf16x3(x), ys = split_bf16x3(-acc);
    *(u32x4_t*)(a.rowstat + st * 8) = u32x4_t{xs[0], xs[1], ys[0], ys[1]};
  }
}

template <int D>
void launch_delta(const BwdArgs& a, bool bf16, hipStream_t s) {
  const long rows = (long)a.B * a.Tq * a.Hq;
  const long threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL((attn_delta_kernel<D, true>), dim3(blocks), dim3(256), 0, s, a, rows);
  else
    hipLaunchKernelGGL((attn_delta_kernel<D, false>), dim3(blocks), dim3(256), 0, s, a, rows);
}

}  // namespace

void launch_delta_any(const BwdArgs& a, int D, bool bf16, hipStream_t s) {
  if ((long)a.B * a.Tq * a.Hq == 0) return;
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
  const long rows = (long)a.B * a.Hq * a.Tq;
  if (rows == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_fp32_kernel<128>, dim3((unsigned)rows), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_fp32_kernel<64>, dim3((unsigned)rows), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pass_fp32(const BwdArgs& a, int D, int pass, hipStream_t s) {
  if (pass == kBwdPre) {
    launch_delta_any(a, D, false, s);
  } else if (pass == kBwdDkdv) {
    const long krows = (long)a.B * a.Hkv * a.Tkv;
    if (krows > 0) {
      if (D == 128)
        hipLaunchKernelGGL(attn_dkdv_fp32_kernel<128>, dim3((unsigned)krows), dim3(64), 0, s, a);
      else
        hipLaunchKernelGGL(attn_dkdv_fp32_kernel<64>, dim3((unsigned)krows), dim3(64), 0, s, a);
    }
  } else {
    const long qrows = (long)a.B * a.Hq * a.Tq;
    if (qrows > 0) {
      if (D == 128)
        hipLaunchKernelGGL(attn_dq_fp32_kernel<128>, dim3((unsigned)qrows), dim3(64), 0, s, a);
      else
        hipLaunchKernelGGL(attn_dq_fp32_kernel<64>, dim3((unsigned)qrows), dim3(64), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace attn
