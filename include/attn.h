/*
 * attn.h - C ABI of the fused exact attention library for AMD MI355X (gfx950).
 *
 * Operation (probjax benchmark pages, "Attention performance", introduction
 * and section "Memory"): for tensors laid out [batch, seq, heads, head_dim],
 *     O = softmax(scale * Q K^T + mask) V,
 * keeping O and the log-sum-exp of each row for the backward pass, and the
 * gradients of a scalar loss with respect to Q, K and V given dO.
 *
 * Masks:
 *   - causal, equal-length form: key j is visible to query i iff j <= i
 *     ("Attention performance", section "When to use which");
 *   - per-batch KV length (the pages' KVLenMask): keys j >= kv_lens[b] are
 *     skipped; a query row with no valid key returns zeros
 *     ("H100 (Hopper)", section "Mosaic GPU");
 *   - local window (one of the position-only masks the pages' fused kernel
 *     takes, "Attention performance", section on the default attention
 *     function): key j is visible to query i iff
 *     i - window_left <= j <= i + window_right; a negative bound (or one of
 *     at least Tkv) means no bound on that side; equal lengths only, like
 *     the causal form;
 *   - the masks combine by AND;
 *   - grouped-query attention: query head h reads KV head h / (Hq / Hkv),
 *     without repeating K or V ("Attention performance", section
 *     "Grouped-query attention and decoding").
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     in [B, T, H, D] order (row stride H*D elements) and 16-byte aligned.
 *     Q, dO, O, dQ: [B, Tq, Hq, D]; K, V, dK, dV: [B, Tkv, Hkv, D].
 *     Tensors are bf16 or fp32 as given by attn_params_t.dtype (fp32 is
 *     computed in fp32 throughout, on the fp32 matrix cores). A tensor
 *     with no elements (B, Tq or Tkv = 0) may be passed as NULL; any other
 *     NULL or misaligned tensor pointer -> ATTN_ERR_INVALID.
 *   - LSE is fp32 [B, Hq, Tq], natural logarithm, -inf on rows with no
 *     valid key (where O is 0).
 *   - kv_lens, when not NULL, is a DEVICE int32 [B]; each value is clamped
 *     to [0, Tkv] by the kernels (the host cannot read it without a sync).
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous on it. The library never allocates, frees or
 *     synchronises (the address-checking debug build at the end of this
 *     header does synchronise) and is safe to call from several threads; its
 *     only state is, per device, the address of attn_decode_noalloc's static
 *     scratch and the compute-unit count that sizes the persistent dK/dV
 *     grid.
 *   - Argument errors are reported before anything is launched: the call
 *     returns a status and attn_last_error() (thread-local) describes it.
 *     The pages' own rule is to reject what cannot be computed exactly
 *     ("H100 (Hopper)", section "Device-specific defaults").
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_BF16 = 0, ATTN_FP32 = 1 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, bad sizes, Hq % Hkv != 0, causal or window with Tq != Tkv,
                               causal or window in decode, bad scale */
  ATTN_ERR_UNSUPPORTED = 2, /* head_dim or dtype the library has no kernel for: D outside {32, 64, 128, 256},
                               fp32 with D = 256, fp32 decode; or a problem too large for one launch */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_size query */
  ATTN_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} attn_status_t;

typedef enum { ATTN_OP_FWD = 0, ATTN_OP_BWD = 1, ATTN_OP_DECODE = 2 } attn_op_t;

typedef struct {
  int32_t B;      /* batch, >= 0 */
  int32_t Tq;     /* query length, >= 0 */
  int32_t Tkv;    /* key/value length (KV cache capacity for decode), >= 0 */
  int32_t Hq;     /* query heads, >= 1 */
  int32_t Hkv;    /* key/value heads, >= 1, divides Hq */
  int32_t D;      /* head_dim: 32, 64, 128 or 256 (bf16); 32, 64 or 128 (fp32) */
  int32_t dtype;  /* attn_dtype_t of Q, K, V, O, dO, dQ, dK, dV */
  float scale;    /* softmax scale, finite and > 0 (e.g. 1/sqrt(D)) */
  int32_t causal; /* 0 or 1; 1 requires Tq == Tkv */
  const int32_t* kv_lens; /* device int32[B] or NULL (= Tkv for every batch) */
  int32_t window_left;    /* local window: keys down to i - window_left; < 0 = no bound */
  int32_t window_right;   /* local window: keys up to i + window_right; < 0 = no bound */
} attn_params_t;

/* Host-only check of `p` for operation `op` (attn_op_t). Touches no device
 * and no HIP runtime; returns ATTN_OK or the status the call would return. */
attn_status_t attn_validate(const attn_params_t* p, int32_t op);

/* Forward (online softmax over KV tiles).
 * q [B,Tq,Hq,D], k/v [B,Tkv,Hkv,D] in; o [B,Tq,Hq,D], lse fp32 [B,Hq,Tq] out.
 * Only KV tiles below min(Tkv, kv_lens[b]) and, with causal, below the
 * query tile's last row are read. */
attn_status_t attn_fwd(const attn_params_t* p, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* stream);

/* Bytes of device workspace attn_bwd (and each of its passes) needs, for the
 * row statistics of the split backward ("Attention performance", section
 * "When to use which"): per query row (B * Hq * Tq rows)
 * 24 bytes, each region rounded up to 256 bytes: D = rowsum(dO * O) and
 * LSE * log2(e) (fp32 each), and 16 bytes of bf16 terms of -LSE/scale and -D
 * that the dK/dV pass adds to its products. With GQA (Hq > Hkv, bf16) and
 * fewer than 256 dK/dV workgroups (B * Hkv * ceil(Tkv / 128)), the query
 * heads of a group are split over S workgroups per 128 keys (the smallest S
 * that reaches 256, at most Hq / Hkv) and the workspace adds two fp32
 * [S, B, Tkv, Hkv, D] arrays of partial dK and dV, summed in split order by
 * a reduction pass; S depends only on the shape, so results stay bitwise
 * reproducible. The last 256 bytes hold the work counters of the head_dim 128
 * dK/dV pass (persistent workgroups taking 128-key tiles from a queue): the
 * preprocess (or attn_bwd_dq_and_preprocess) sets them to zero and the dK/dV
 * pass leaves them at zero. */
size_t attn_bwd_workspace_size(const attn_params_t* p);

/* Backward: the gradients of a scalar loss with respect to Q, K and V given
 * dO ("Attention performance", introduction). The pages' split backward is
 * the scheme used here: a pass over key tiles for dK and dV and a separate
 * pass over query tiles for dQ, which needs no atomic accumulation and so
 * gives bitwise reproducible gradients ("Attention performance", section
 * "When to use which"; "H100 (Hopper)", section "Why", where it is the
 * robust choice). P is recomputed from the forward's `lse`, the residuals
 * being O and LSE only ("Attention performance", section "Memory").
 * D = rowsum(dO * O) is formed first (by the dQ kernel itself at bf16
 * head_dim 64 and 128, which then runs first; by a pre-kernel otherwise) and
 * kept in the workspace; one kernel forms dK and dV per KV tile (summing the
 * G query heads of a group in a fixed order); one kernel forms dQ per query
 * tile. attn_bwd runs attn_bwd_dq_and_preprocess, then attn_bwd_dkdv.
 * q, k, v, o, lse as produced/consumed by attn_fwd; dout = dO like q.
 * dq like q; dk, dv like k. Keys at or past kv_lens[b] get dK = dV = 0.
 * Reruns on the same inputs are bitwise identical. */
attn_status_t attn_bwd(const attn_params_t* p, const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The passes of attn_bwd as separate calls (the split backward of
 * "Attention performance", section "When to use which").
 * attn_bwd_preprocess writes D = rowsum(dO * O) and LSE * log2(e) into the
 * workspace (and zeroes its work counters); attn_bwd_dkdv and attn_bwd_dq
 * read them and are independent of each other, so a caller may run them on
 * two streams once the preprocess has completed. attn_bwd_dq_and_preprocess
 * does what attn_bwd_preprocess and then attn_bwd_dq do, in one launch at
 * bf16 head_dim 64 and 128 (the dQ kernel forms D from O and dO itself), and
 * writes the same workspace bits, so attn_bwd_dkdv may follow it; attn_bwd is
 * that call and then attn_bwd_dkdv. Every order gives the same gradients bit
 * for bit. attn_bwd_dkdv also counts its work in the workspace's counters and
 * returns them to zero, so the same workspace serves the next pass or a
 * replay of a captured graph; two attn_bwd_dkdv calls must not run at the
 * same time on one workspace, nor one with a preprocess on that workspace.
 * Arguments mean what they mean for attn_bwd. */
attn_status_t attn_bwd_preprocess(const attn_params_t* p, const void* o, const float* lse, const void* dout,
                                  void* workspace, size_t workspace_bytes, void* stream);
attn_status_t attn_bwd_dkdv(const attn_params_t* p, const void* q, const void* k, const void* v, const float* lse,
                            const void* dout, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                            void* stream);
attn_status_t attn_bwd_dq(const attn_params_t* p, const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dq, const void* workspace, size_t workspace_bytes, void* stream);
attn_status_t attn_bwd_dq_and_preprocess(const attn_params_t* p, const void* q, const void* k, const void* v,
                                         const void* o, const float* lse, const void* dout, void* dq,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Split budget of the split-KV decode ("Attention performance", section
 * "Grouped-query attention and decoding", where the keys are split because
 * few queries leave the chip idle) when num_splits = 0: sized so that every key
 * range of the call runs at once on the chip (a pure function of the shape,
 * so reruns are bitwise identical). */
int32_t attn_decode_num_splits(const attn_params_t* p);

/* Bytes of device workspace attn_decode needs, for the partial results of
 * the split-KV decode ("Attention performance", section "Grouped-query
 * attention and decoding"), for the split budget
 * `num_splits` (0 = auto): fp32 partial outputs and partial LSEs for at most
 * num_splits + B * Hkv * ceil(Tq * Hq / Hkv / 64) key ranges of 64 packed
 * rows each. */
size_t attn_decode_workspace_size(const attn_params_t* p, int32_t num_splits);

/* Split-KV decode ("Attention performance", section "Grouped-query attention
 * and decoding"): few queries over a long KV cache. The Tq queries of the G
 * query heads of a KV head are packed into tiles of 64 rows (row i * G + g),
 * the keys are split across workgroups, and the partial results are
 * combined by their LSE in a fixed order. The split is balanced over the
 * actual lengths: with U the 64-key tiles of all (batch, KV head, row tile)
 * segments and P = num_splits (the split budget; 0 = automatic), a segment
 * with n tiles is cut into min(n, ceil(n * P / U)) near-equal key ranges, so
 * no range exceeds ceil(U / P) tiles. The schedule is computed on the device
 * from kv_lens; results depend on it only through rounding and are bitwise
 * reproducible for the same inputs and budget. With a budget of 1 (the
 * automatic budget once B * Hkv * ceil(Tq * Hq / Hkv / 64) reaches 255) every
 * segment is one range and the split kernel writes O and the LSE itself,
 * without the combine (the same bits the combine makes of one range).
 * Non-causal (p->causal must be 0); bf16 only.
 * q [B,Tq,Hq,D]; k_cache/v_cache [B,Tkv,Hkv,D] (Tkv = capacity); keys at or
 * past kv_lens[b] are never read. kv_lens = valid length per batch (NULL =
 * Tkv). o [B,Tq,Hq,D] bf16; lse fp32 [B,Hq,Tq] or NULL. A row with no valid
 * key gets O = 0 and LSE = -inf. num_splits < 0 -> ATTN_ERR_INVALID; a
 * workspace smaller than attn_decode_workspace_size -> ATTN_ERR_WORKSPACE;
 * B * Hkv * ceil(Tq * Hq / Hkv / 64) * ceil(Tkv / 64) >= 2^31 (the kernels
 * count key tiles in 32 bits) -> ATTN_ERR_UNSUPPORTED. */
attn_status_t attn_decode(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache,
                          void* o, float* lse, int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of device memory behind attn_decode_noalloc on each device. */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments and results as attn_decode (the same
 * kernels, bit for bit); the partial results live in a static device array of
 * ATTN_DECODE_NOALLOC_SCRATCH_BYTES per device, held until the process ends.
 * A call whose workspace (attn_decode_workspace_size for its split budget)
 * exceeds that returns ATTN_ERR_WORKSPACE before touching the device. The
 * call allocates and frees nothing; its first call on a device looks up the
 * array's device address. Every call on one device shares the array:
 * calls that overlap on one device (several streams or threads) race. */
attn_status_t attn_decode_noalloc(const attn_params_t* p, const void* q, const void* k_cache, const void* v_cache,
                                  void* o, float* lse, int32_t num_splits, void* stream);

/* Static description of a status code. */
const char* attn_status_string(attn_status_t status);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char* attn_last_error(void);

/* Address checks of the debug build, for callers hunting a memory error, not
 * for production use. libattn_debug.so (built from the same sources with
 * -DATTN_DEBUG) registers the byte ranges of each call's buffers before its
 * launches (tensors at their sizes from the parameters, the workspace at the
 * size the call needs) and has every global load and global->LDS copy of the
 * kernels check the bytes it reads against them. An access outside every
 * range is counted and the kernel runs on. Debug calls synchronise their
 * stream before launching and cannot be captured into a graph
 * (ATTN_ERR_UNSUPPORTED).
 * attn_debug_take synchronises the device and writes to out[0] the number of
 * lane accesses found outside the ranges since its previous call and to
 * out[1] the first such address (0 if none), then resets both. out must hold
 * two values (caller-owned host memory). A release build (libattn.so)
 * returns ATTN_ERR_UNSUPPORTED and leaves out untouched. */
attn_status_t attn_debug_take(unsigned long long* out);

/* Positive control of the debug build's checks: registers a made-up 512-byte
 * range and launches one wave on `stream` whose 64 lanes check the 16-byte
 * accesses at 16-byte steps from its start without reading any memory, so
 * that the next attn_debug_take counts exactly 32 accesses outside it. A
 * release build returns ATTN_ERR_UNSUPPORTED and launches nothing. */
attn_status_t attn_debug_selftest(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
