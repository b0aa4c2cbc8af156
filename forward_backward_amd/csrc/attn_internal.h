// Internal host/device interface between the C ABI (attn_api.cpp) and the
// HIP kernels. Not installed; callers use include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Arguments of the forward kernels (bf16 tiles or the fp32 path).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // [B, Hq, Tq], natural log
  const int32_t* kv_lens;  // device [B] or nullptr
  int B, Tq, Tkv, Hq, Hkv;
  float scale;             // softmax scale
  float scale_log2;        // scale * log2(e): the kernels work in base 2
  int causal;
  int win_left, win_right; // local window bounds, -1 = none (see key_lo / key_hi)
  int num_qtiles;
};

// Arguments of the backward kernels.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;            // workspace: D = rowsum(dO * O), [B, Hq, Tq]
  float* lse2;             // workspace: LSE * log2(e), [B, Hq, Tq]
  uint16_t* rowstat;       // workspace: [B, Hq, Tq][8] bf16, -LSE/scale and -D, each split into three
                           // bf16 terms: (x_hi, x_mid, x_lo, 0, y_hi, y_mid, y_lo, 0)
  const int32_t* kv_lens;
  int B, Tq, Tkv, Hq, Hkv;
  float scale;
  float scale_log2;
  int causal;
  int win_left, win_right; // local window bounds, -1 = none (see key_lo / key_hi)
  int num_ktiles;          // KV tiles of the dK/dV kernel
  int kv_split;            // dK/dV workgroups per KV tile, each over heads_per_split query heads of the group
  int heads_per_split;
  float* dkv_part;         // workspace when kv_split > 1: fp32 partial dK then dV, [kv_split][B, Tkv, Hkv, D] each
  unsigned* queue;         // workspace: kBwdQueueWords work counters, zero between passes
  int dq_stats;            // dQ pass (bf16 head_dim 64/128): form D from O and dO itself, write the
                           // pre-kernel's statistics and zero the counters (attn_bwd_dq_and_preprocess)
};

// Arguments of the split-KV decode kernels.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // optional [B, Hq, Tq]
  float* part_o;           // workspace [slots, kDecodeRows, D] fp32
  float* part_lse;         // workspace [slots, kDecodeRows] fp32 (natural log)
  const int32_t* kv_lens;
  int B, Tq, Tkv, Hq, Hkv;
  float scale;
  float scale_log2;
  int budget;              // P: key ranges are sized as if P workgroups shared all key tiles
  int num_rblocks;         // packed row blocks per (batch, KV head)
  int num_slots;           // P + B * Hkv * num_rblocks (upper bound on the key ranges)
  int direct;              // P == 1: one range per segment, written as the output itself (no combine)
};

// Launchers (each returns the hipGetLastError() after its launches).
hipError_t launch_fwd_bf16(const FwdArgs& a, int D, hipStream_t s);
hipError_t launch_fwd_fp32(const FwdArgs& a, int D, hipStream_t s);
// Backward passes: 0 = D pre-kernel, 1 = dK/dV, 2 = dQ.
enum BwdPass { kBwdPre = 0, kBwdDkdv = 1, kBwdDq = 2 };
hipError_t launch_bwd_pass_bf16(const BwdArgs& a, int D, int pass, hipStream_t s);
hipError_t launch_bwd_pass_fp32(const BwdArgs& a, int D, int pass, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, int D, hipStream_t s);
// Device address of the decode's static scratch on the current device (the
// array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES in attn_decode.hip), looked up
// once per device.
hipError_t decode_scratch(void** ptr);

// Tile sizes the host needs for grids and workspaces.
constexpr int kFwdBlockM = 128;   // query rows per forward workgroup
constexpr int kBwdBlockM = 128;   // query rows per dQ workgroup
constexpr int kBwdBlockN = 128;   // keys per dK/dV workgroup
constexpr int kBwdQueueWords = 64;   // counters of the persistent dK/dV kernel (256 bytes of workspace)
constexpr int kBwdFillTarget = 256;  // dK/dV workgroups below which a group's query heads are split (one per CU)
constexpr int kDecodeTileN = 64;  // keys per decode iteration
constexpr int kDecodeRows = 64;   // packed query rows per decode workgroup
constexpr int kDecodeSlots = 256; // decode workgroups resident at once (one per compute unit)

// Address checks of the debug build (compiled with -DATTN_DEBUG into
// libattn_debug.so): before a call's launches the host registers the byte
// ranges of the call's buffers, and every global load and global->LDS copy
// of the kernels checks the bytes it reads against them, counting the
// accesses that fall outside (no trap: the kernels run on). Each code object
// (source file) holds its own table and counters; each registers a setter
// and a reader with the host side at load time.
struct DbgRange {
  unsigned long long lo, hi;  // bytes [lo, hi)
};
constexpr int kDbgRanges = 16;
__host__ __device__ inline bool dbg_in_ranges(unsigned long long addr, unsigned bytes, const DbgRange* r, int n) {
  for (int i = 0; i < n; ++i)
    if (addr >= r[i].lo && addr <= r[i].hi && bytes <= r[i].hi - addr) return true;
  return false;
}
using DbgSetFn = hipError_t (*)(const DbgRange* ranges, int n);
using DbgTakeFn = hipError_t (*)(unsigned long long* count, unsigned long long* first);
int dbg_register(DbgSetFn set, DbgTakeFn take);
// One wave checking the 16-byte accesses at base + 16 * lane (64 lanes) without reading them.
hipError_t launch_debug_selftest(const void* base, hipStream_t s);

}  // namespace attn
