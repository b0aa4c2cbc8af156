// C ABI of the attention library: validation, workspace queries, launches.
//
// Validation runs on the host before any HIP call, so every argument error
// is reported without touching a device (and can be exercised on a host
// without a GPU). The library allocates nothing and never synchronises.
#include "../../include/attn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "attn_internal.h"

namespace attn {
void launch_delta_any(const BwdArgs& a, int D, bool bf16, hipStream_t s);
}

namespace {

thread_local char g_last_error[256] = "";

__attribute__((format(printf, 2, 3))) attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

attn_status_t ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Element counts of the tensor families; a tensor with no elements may be NULL.
struct Sizes {
  long q, kv, stat;  // Q/O/dO/dQ, K/V/dK/dV, LSE
};
Sizes sizes_of(const attn_params_t* p) {
  return Sizes{(long)p->B * p->Tq * p->Hq * p->D, (long)p->B * p->Tkv * p->Hkv * p->D, (long)p->B * p->Hq * p->Tq};
}
// A tensor pointer is acceptable when the tensor is empty, or non-NULL and 16-byte aligned.
attn_status_t check_ptr(const void* ptr, long count, bool need_align) {
  if (count == 0) return ATTN_OK;
  if (ptr == nullptr) return ATTN_ERR_INVALID;
  if (need_align && !aligned16(ptr)) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

constexpr long kMaxGrid = 2147483647L;
constexpr float kLog2e = 1.4426950408889634f;

size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

}  // namespace

namespace attn {
// Setters and readers of the debug build's per-code-object address tables
// (see attn_internal.h); a release build registers none.
namespace {
struct DbgRegistry {
  DbgSetFn set[32];
  DbgTakeFn take[32];
  int n = 0;
};
DbgRegistry& dbg_registry() {
  static DbgRegistry r;
  return r;
}
}  // namespace
int dbg_register(DbgSetFn set, DbgTakeFn take) {
  DbgRegistry& r = dbg_registry();
  if (r.n < 32) {
    r.set[r.n] = set;
    r.take[r.n] = take;
    ++r.n;
  }
  return r.n;
}
}  // namespace attn

namespace {
// Debug build: register the byte ranges of a call's buffers with every code
// object before its launches (nothing in a release build). The tables are
// written synchronously once the stream's earlier work is done, so debug
// calls run one at a time and cannot be captured into a graph.
struct Buf {
  const void* p;
  size_t bytes;
};
attn_status_t dbg_prepare(std::initializer_list<Buf> bufs, void* stream) {
#ifdef ATTN_DEBUG
  attn::DbgRange r[attn::kDbgRanges];
  int n = 0;
  for (const Buf& b : bufs)
    if (b.p != nullptr && b.bytes > 0 && n < attn::kDbgRanges) {
      const unsigned long long lo = reinterpret_cast<unsigned long long>(b.p);
      r[n++] = attn::DbgRange{lo, lo + b.bytes};
    }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return fail(ATTN_ERR_UNSUPPORTED, "the debug build cannot be captured into a graph");
  if (hipStreamSynchronize(s) != hipSuccess) return fail(ATTN_ERR_HIP, "stream synchronisation failed");
  const attn::DbgRegistry& reg = attn::dbg_registry();
  for (int i = 0; i < reg.n; ++i)
    if (reg.set[i](r, n) != hipSuccess) return fail(ATTN_ERR_HIP, "debug address table upload failed");
#else
  (void)bufs;
  (void)stream;
#endif
  return ATTN_OK;
}
}  // namespace

extern "C" {

attn_status_t attn_debug_take(unsigned long long* out) {
#ifdef ATTN_DEBUG
  if (out == nullptr) return fail(ATTN_ERR_INVALID, "out must hold two values");
  if (hipDeviceSynchronize() != hipSuccess) return fail(ATTN_ERR_HIP, "device synchronisation failed");
  unsigned long long count = 0, first = 0;
  const attn::DbgRegistry& reg = attn::dbg_registry();
  for (int i = 0; i < reg.n; ++i)
    if (reg.take[i](&count, &first) != hipSuccess) return fail(ATTN_ERR_HIP, "debug counter read failed");
  out[0] = count;
  out[1] = first;
  return ok();
#else
  (void)out;
  return fail(ATTN_ERR_UNSUPPORTED, "address checks are compiled into libattn_debug.so only");
#endif
}

attn_status_t attn_debug_selftest(void* stream) {
#ifdef ATTN_DEBUG
  // A made-up address range: the self-test kernel only compares addresses.
  const void* base = reinterpret_cast<const void*>(static_cast<uintptr_t>(1) << 40);
  const attn_status_t st = dbg_prepare({{base, 32 * 16}}, stream);
  if (st != ATTN_OK) return st;
  if (attn::launch_debug_selftest(base, static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(ATTN_ERR_HIP, "self-test launch failed");
  return ok();
#else
  (void)stream;
  return fail(ATTN_ERR_UNSUPPORTED, "address checks are compiled into libattn_debug.so only");
#endif
}

attn_status_t attn_validate(const attn_params_t* p, int32_t op) {
  if (p == nullptr) return fail(ATTN_ERR_INVALID, "params is NULL");
  if (op != ATTN_OP_FWD && op != ATTN_OP_BWD && op != ATTN_OP_DECODE)
    return fail(ATTN_ERR_INVALID, "unknown op %d", op);
  if (p->B < 0 || p->Tq < 0 || p->Tkv < 0)
    return fail(ATTN_ERR_INVALID, "B, Tq and Tkv must be >= 0");
  if (p->Hq < 1 || p->Hkv < 1) return fail(ATTN_ERR_INVALID, "Hq and Hkv must be >= 1");
  if (p->Hq % p->Hkv != 0) return fail(ATTN_ERR_INVALID, "Hq (%d) is not a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID, "unknown dtype %d", p->dtype);
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_ERR_INVALID, "causal must be 0 or 1, got %d", p->causal);
  if (!(std::isfinite(p->scale) && p->scale > 0.f)) return fail(ATTN_ERR_INVALID, "scale must be finite and > 0");
  if (p->causal && p->Tq != p->Tkv)
    return fail(ATTN_ERR_INVALID, "causal masking needs Tq == Tkv (got %d and %d)", p->Tq, p->Tkv);
  if (op == ATTN_OP_DECODE && p->causal) return fail(ATTN_ERR_INVALID, "decode is non-causal");
  const bool window = (p->window_left >= 0 && p->window_left < p->Tkv) ||
                      (p->window_right >= 0 && p->window_right < p->Tkv);
  if (window && p->Tq != p->Tkv)
    return fail(ATTN_ERR_INVALID, "window masks need Tq == Tkv (got %d and %d)", p->Tq, p->Tkv);
  if (window && op == ATTN_OP_DECODE) return fail(ATTN_ERR_INVALID, "decode takes no window mask");
  if (p->D != 32 && p->D != 64 && p->D != 128 && p->D != 256)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d (supported: 32, 64, 128, 256)", p->D);
  if (p->D == 256 && p->dtype == ATTN_FP32)
    return fail(ATTN_ERR_UNSUPPORTED, "the fp32 path takes head_dim 32, 64 or 128");
  if (op == ATTN_OP_DECODE && p->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode is bf16 only");
  // Tile copies address a tile's rows with 32-bit byte offsets.
  if ((long)p->Hq * p->D > (1L << 22) || (long)p->Hkv * p->D > (1L << 22))
    return fail(ATTN_ERR_UNSUPPORTED, "heads * head_dim above 2^22 (Hq = %d, Hkv = %d)", p->Hq, p->Hkv);
  const long qrows = (long)p->B * p->Hq * p->Tq;
  const long krows = (long)p->B * p->Hkv * p->Tkv;
  if (qrows >= kMaxGrid || krows >= kMaxGrid) return fail(ATTN_ERR_UNSUPPORTED, "problem too large for one launch");
  return ok();
}

// A window bound as the kernels take it: -1 (no bound) for negative values and
// for bounds that reach past every key.
static int window_bound(int32_t w, int32_t tkv) { return (w < 0 || w >= tkv) ? -1 : w; }

// fp32 [B, Hq, Tq] row statistics per array.
static size_t bwd_stat_bytes(const attn_params_t* p) {
  return round_up((size_t)(p->B > 0 ? p->B : 0) * (p->Hq > 0 ? p->Hq : 0) * (p->Tq > 0 ? p->Tq : 0) * sizeof(float),
                  256);
}

// Query-head split of the bf16 dK/dV pass. One workgroup per (batch, KV
// head, 128 keys) sums the gradients of all G query heads of the group; when
// that leaves compute units idle (fewer than kBwdFillTarget workgroups), the G
// heads are divided over S workgroups per KV tile that write fp32 partial
// sums, and a reduction adds the S partials in a fixed order. A pure function
// of the shape, so reruns are bitwise identical.
static int bwd_kv_split(const attn_params_t* p, int* heads_per_split) {
  const int G = (p->Hkv > 0 && p->Hq >= p->Hkv) ? p->Hq / p->Hkv : 1;
  *heads_per_split = G;
  if (p->dtype != ATTN_BF16 || G <= 1 || p->B <= 0 || p->Tkv <= 0) return 1;
  const long base = (long)p->B * p->Hkv * ((p->Tkv + attn::kBwdBlockN - 1) / attn::kBwdBlockN);
  if (base >= attn::kBwdFillTarget) return 1;
  const long want = (attn::kBwdFillTarget + base - 1) / base;
  const int s = (int)(want < G ? want : G);
  const int hps = (G + s - 1) / s;
  *heads_per_split = hps;
  return (G + hps - 1) / hps;
}

static size_t bwd_part_bytes(const attn_params_t* p) {
  int hps;
  const int s = bwd_kv_split(p, &hps);
  if (s <= 1) return 0;
  return round_up(2 * (size_t)s * p->B * p->Tkv * p->Hkv * p->D * sizeof(float), 256);
}

// Work counters of the dK/dV pass, after the row statistics and partials.
static constexpr size_t kQueueBytes = attn::kBwdQueueWords * sizeof(unsigned);

size_t attn_bwd_workspace_size(const attn_params_t* p) {
  if (p == nullptr) return 0;
  return 6 * bwd_stat_bytes(p) + bwd_part_bytes(p) + kQueueBytes;
}

attn_status_t attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v, void* o, float* lse,
                       void* stream) {
  attn_status_t st = attn_validate(p, ATTN_OP_FWD);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k, n.kv, true) || check_ptr(v, n.kv, true) || check_ptr(o, n.q, true) ||
      check_ptr(lse, n.stat, false))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  attn::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.kv_lens = p->kv_lens;
  a.B = p->B; a.Tq = p->Tq; a.Tkv = p->Tkv; a.Hq = p->Hq; a.Hkv = p->Hkv;
  a.scale = p->scale; a.scale_log2 = p->scale * kLog2e; a.causal = p->causal;
  a.win_left = window_bound(p->window_left, p->Tkv); a.win_right = window_bound(p->window_right, p->Tkv);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  a.num_qtiles = (p->Tq + attn::kFwdBlockM - 1) / attn::kFwdBlockM;
  if ((long)a.num_qtiles * a.Hq * a.B >= kMaxGrid) return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
  const size_t es = p->dtype == ATTN_BF16 ? 2 : 4;
  st = dbg_prepare({{q, n.q * es}, {k, n.kv * es}, {v, n.kv * es}, {o, n.q * es}, {lse, n.stat * sizeof(float)},
                    {p->kv_lens, p->B * sizeof(int32_t)}},
                   stream);
  if (st != ATTN_OK) return st;
  if (p->dtype == ATTN_BF16)
    e = attn::launch_fwd_bf16(a, p->D, s);
  else
    e = attn::launch_fwd_fp32(a, p->D, s);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "launch failed (hip error %d)", (int)e);
  return ok();
}

}  // extern "C"

namespace {

// Shared checks and argument setup of the backward entry points; each entry
// point then checks and fills the tensors its passes touch.
attn_status_t bwd_setup(const attn_params_t* p, attn::BwdArgs& a, const void* ws, size_t ws_bytes) {
  attn_status_t st = attn_validate(p, ATTN_OP_BWD);
  if (st != ATTN_OK) return st;
  const size_t need = attn_bwd_workspace_size(p);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace too small (%zu bytes needed, %zu given)", need, ws_bytes);
  std::memset(&a, 0, sizeof(a));
  a.delta = static_cast<float*>(const_cast<void*>(ws));
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(ws)) + bwd_stat_bytes(p));
  a.rowstat = reinterpret_cast<uint16_t*>(static_cast<char*>(const_cast<void*>(ws)) + 2 * bwd_stat_bytes(p));
  a.kv_split = bwd_kv_split(p, &a.heads_per_split);
  a.dkv_part = a.kv_split > 1
                   ? reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(ws)) + 6 * bwd_stat_bytes(p))
                   : nullptr;
  a.queue = reinterpret_cast<unsigned*>(static_cast<char*>(const_cast<void*>(ws)) + 6 * bwd_stat_bytes(p) +
                                        bwd_part_bytes(p));
  a.kv_lens = p->kv_lens;
  a.B = p->B; a.Tq = p->Tq; a.Tkv = p->Tkv; a.Hq = p->Hq; a.Hkv = p->Hkv;
  a.scale = p->scale; a.scale_log2 = p->scale * kLog2e; a.causal = p->causal;
  a.win_left = window_bound(p->window_left, p->Tkv); a.win_right = window_bound(p->window_right, p->Tkv);
  a.num_ktiles = (p->Tkv + attn::kBwdBlockN - 1) / attn::kBwdBlockN;
  return ATTN_OK;
}

attn_status_t run_pass(const attn_params_t* p, const attn::BwdArgs& a, int pass, void* stream) {
  const Sizes n = sizes_of(p);
  const size_t es = p->dtype == ATTN_BF16 ? 2 : 4;
  const attn_status_t st =
      dbg_prepare({{a.q, n.q * es}, {a.k, n.kv * es}, {a.v, n.kv * es}, {a.o, n.q * es}, {a.dout, n.q * es},
                   {a.dq, n.q * es}, {a.dk, n.kv * es}, {a.dv, n.kv * es}, {a.lse, n.stat * sizeof(float)},
                   {a.delta, attn_bwd_workspace_size(p)}, {p->kv_lens, p->B * sizeof(int32_t)}},
                  stream);
  if (st != ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = p->dtype == ATTN_BF16 ? attn::launch_bwd_pass_bf16(a, p->D, pass, s)
                                       : attn::launch_bwd_pass_fp32(a, p->D, pass, s);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "launch failed (hip error %d)", (int)e);
  return ok();
}

}  // namespace

extern "C" {

attn_status_t attn_bwd_preprocess(const attn_params_t* p, const void* o, const float* lse, const void* dout,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  attn::BwdArgs a;
  attn_status_t st = bwd_setup(p, a, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(o, n.q, true) || check_ptr(lse, n.stat, false) || check_ptr(dout, n.q, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  a.o = o; a.lse = lse; a.dout = dout;
  return run_pass(p, a, attn::kBwdPre, stream);
}

attn_status_t attn_bwd_dkdv(const attn_params_t* p, const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            void* stream) {
  attn::BwdArgs a;
  attn_status_t st = bwd_setup(p, a, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k, n.kv, true) || check_ptr(v, n.kv, true) ||
      check_ptr(lse, n.stat, false) || check_ptr(dout, n.q, true) || check_ptr(dk, n.kv, true) ||
      check_ptr(dv, n.kv, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  a.q = q; a.k = k; a.v = v; a.lse = lse; a.dout = dout; a.dk = dk; a.dv = dv;
  return run_pass(p, a, attn::kBwdDkdv, stream);
}

attn_status_t attn_bwd_dq(const attn_params_t* p, const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dq, const void* workspace, size_t workspace_bytes, void* stream) {
  attn::BwdArgs a;
  attn_status_t st = bwd_setup(p, a, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k, n.kv, true) || check_ptr(v, n.kv, true) ||
      check_ptr(lse, n.stat, false) || check_ptr(dout, n.q, true) || check_ptr(dq, n.q, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  a.q = q; a.k = k; a.v = v; a.lse = lse; a.dout = dout; a.dq = dq;
  return run_pass(p, a, attn::kBwdDq, stream);
}

// dQ together with the preprocess outputs: one launch where the dQ kernel
// forms D itself (bf16 head_dim 64 and 128), else the pre-kernel and then dQ.
// Without query rows the dQ grid is empty, and the pre-kernel (which always
// launches) still zeroes the dK/dV pass's work counters.
static attn_status_t dq_and_preprocess(const attn_params_t* p, attn::BwdArgs& a, void* stream) {
  if (p->dtype == ATTN_BF16 && (p->D == 64 || p->D == 128) && (long)p->B * p->Hq * p->Tq > 0) {
    a.dq_stats = 1;
    const attn_status_t st = run_pass(p, a, attn::kBwdDq, stream);
    a.dq_stats = 0;
    return st;
  }
  const attn_status_t st = run_pass(p, a, attn::kBwdPre, stream);
  return st != ATTN_OK ? st : run_pass(p, a, attn::kBwdDq, stream);
}

attn_status_t attn_bwd_dq_and_preprocess(const attn_params_t* p, const void* q, const void* k, const void* v,
                                         const void* o, const float* lse, const void* dout, void* dq,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  attn::BwdArgs a;
  attn_status_t st = bwd_setup(p, a, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k, n.kv, true) || check_ptr(v, n.kv, true) || check_ptr(o, n.q, true) ||
      check_ptr(lse, n.stat, false) || check_ptr(dout, n.q, true) || check_ptr(dq, n.q, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout; a.dq = dq;
  return dq_and_preprocess(p, a, stream);
}

attn_status_t attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, void* stream) {
  attn::BwdArgs a;
  attn_status_t st = bwd_setup(p, a, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k, n.kv, true) || check_ptr(v, n.kv, true) || check_ptr(o, n.q, true) ||
      check_ptr(lse, n.stat, false) || check_ptr(dout, n.q, true) || check_ptr(dq, n.q, true) ||
      check_ptr(dk, n.kv, true) || check_ptr(dv, n.kv, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  st = dq_and_preprocess(p, a, stream);
  return st != ATTN_OK ? st : run_pass(p, a, attn::kBwdDkdv, stream);
}

// Packed query rows (Tq * G) of one (batch, KV head) in blocks of the decode tile.
static long decode_row_blocks(const attn_params_t* p) {
  const long rows = (long)(p->Tq > 0 ? p->Tq : 0) * (p->Hkv > 0 && p->Hq >= p->Hkv ? p->Hq / p->Hkv : 0);
  return (rows + attn::kDecodeRows - 1) / attn::kDecodeRows;
}

static long decode_segments(const attn_params_t* p) {
  return (long)(p->B > 0 ? p->B : 0) * (p->Hkv > 0 ? p->Hkv : 0) * decode_row_blocks(p);
}

int32_t attn_decode_num_splits(const attn_params_t* p) {
  if (p == nullptr) return 1;
  // One workgroup per compute unit at D = 128 (its LDS ring takes 128 KiB),
  // two at D = 64 or 32; the budget leaves room for the up to one extra range per
  // segment that rounding adds, so that all ranges run in one wave.
  const long resident = (long)attn::kDecodeSlots * (p->D <= 64 ? 2 : 1);
  const long budget = resident - decode_segments(p);
  return budget < 1 ? 1 : (int32_t)budget;
}

size_t attn_decode_workspace_size(const attn_params_t* p, int32_t num_splits) {
  if (p == nullptr || p->Hkv < 1 || p->Hq < p->Hkv || p->D < 1) return 0;
  if (num_splits <= 0) num_splits = attn_decode_num_splits(p);
  const long segs = decode_segments(p);
  if (segs == 0) return 0;
  const size_t rows = (size_t)(num_splits + segs) * attn::kDecodeRows;
  return round_up(rows * (size_t)p->D * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

}  // extern "C"

namespace {

// Checks of a decode call that need no device (arguments, split budget);
// fills `num_splits` (0 = automatic resolved) and the workspace size needed.
attn_status_t decode_check(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache,
                           const void* o, int32_t& num_splits, size_t& need) {
  attn_status_t st = attn_validate(p, ATTN_OP_DECODE);
  if (st != ATTN_OK) return st;
  const Sizes n = sizes_of(p);
  if (check_ptr(q, n.q, true) || check_ptr(k_cache, n.kv, true) || check_ptr(v_cache, n.kv, true) ||
      check_ptr(o, n.q, true))
    return fail(ATTN_ERR_INVALID, "tensor pointers must be non-NULL and 16-byte aligned (except empty tensors)");
  if (num_splits < 0) return fail(ATTN_ERR_INVALID, "num_splits must be >= 0 (0 = automatic)");
  if (num_splits == 0) num_splits = attn_decode_num_splits(p);
  if ((long)num_splits + decode_segments(p) >= kMaxGrid) return fail(ATTN_ERR_UNSUPPORTED, "too many splits");
  // The kernels count the key tiles of all segments in 32 bits.
  if ((double)decode_segments(p) * (double)((p->Tkv + attn::kDecodeTileN - 1) / attn::kDecodeTileN) >= 2147483648.0)
    return fail(ATTN_ERR_UNSUPPORTED, "decode problem too large (key tiles of all segments must stay below 2^31)");
  need = attn_decode_workspace_size(p, num_splits);
  return ATTN_OK;
}

// Launches of a checked decode call with its workspace.
attn_status_t decode_run(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache, void* o,
                         float* lse, int32_t num_splits, void* workspace, void* stream) {
  const long segs = decode_segments(p);
  attn::DecodeArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse; a.kv_lens = p->kv_lens;
  const size_t rows = (size_t)(num_splits + segs) * attn::kDecodeRows;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(rows * p->D * sizeof(float), 256));
  a.B = p->B; a.Tq = p->Tq; a.Tkv = p->Tkv; a.Hq = p->Hq; a.Hkv = p->Hkv;
  a.scale = p->scale; a.scale_log2 = p->scale * kLog2e;
  a.budget = num_splits;
  a.num_rblocks = (int)decode_row_blocks(p);
  a.num_slots = (int)(num_splits + segs);
  a.direct = num_splits == 1;
  const Sizes n = sizes_of(p);
  const attn_status_t st =
      dbg_prepare({{q, n.q * size_t{2}}, {k_cache, n.kv * size_t{2}}, {v_cache, n.kv * size_t{2}}, {o, n.q * size_t{2}},
                   {lse, n.stat * sizeof(float)}, {workspace, attn_decode_workspace_size(p, num_splits)},
                   {p->kv_lens, p->B * sizeof(int32_t)}},
                  stream);
  if (st != ATTN_OK) return st;
  hipError_t e = attn::launch_decode_bf16(a, p->D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "launch failed (hip error %d)", (int)e);
  return ok();
}

}  // namespace

extern "C" {

attn_status_t attn_decode(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache, void* o,
                          float* lse, int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  size_t need = 0;
  attn_status_t st = decode_check(p, q, k_cache, v_cache, o, num_splits, need);
  if (st != ATTN_OK) return st;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "workspace too small (%zu bytes needed, %zu given)", need, workspace_bytes);
  return decode_run(p, q, k_cache, v_cache, o, lse, num_splits, workspace, stream);
}

attn_status_t attn_decode_noalloc(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache,
                                  void* o, float* lse, int32_t num_splits, void* stream) {
  size_t need = 0;
  attn_status_t st = decode_check(p, q, k_cache, v_cache, o, num_splits, need);
  if (st != ATTN_OK) return st;
  if (need > ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_ERR_WORKSPACE, "needs %zu bytes of scratch; the library's static scratch holds %zu",
                need, (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = attn::decode_scratch(&scratch);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "static scratch unavailable (hip error %d)", (int)e);
  }
  return decode_run(p, q, k_cache, v_cache, o, lse, num_splits, scratch, stream);
}

const char* attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
