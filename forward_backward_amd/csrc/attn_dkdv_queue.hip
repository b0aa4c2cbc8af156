// dK/dV of fused exact attention at head_dim 128, bf16, gfx950: persistent
// workgroups taking their work from a queue.
//
// The work of an item (batch, KV head, split of the group's query heads, 128
// keys) is that of the wave-pair kernel in attn_bwd.hip, in the same order of
// sums, so the gradients are bitwise the same whichever workgroup takes the
// item (two-pass backward: probjax pages, "Attention performance", section
// "When to use which"). Per 32-key block a pair of waves splits the work:
//   S wave:  K rows (B operand) and dV^T; per 32-row block S = Q K^T,
//            P = exp2(c S'), P (bf16) to LDS for its partner, dV^T += dO^T P
//   dP wave: V rows and dK^T; dP = dO V^T, P from LDS, dS = P dP',
//            dK^T += Q^T dS
// over 64-row query tiles that stream through a three-stage LDS ring.
//
// What differs is the scheduling. One workgroup per compute unit runs item
// after item, and its pipeline continues from one item into the next. The
// copy walker streams the next item's first Q/dO tiles while the current
// item's last tiles are computed. The next item's K/V rows are copied into
// LDS while the finished item's dK/dV are stored. With one item per
// workgroup, each workgroup paid about 6 us of start-up (first copies, K/V
// rows, the first row products), 2.5 us of stores and a 3 us gap before the
// next workgroup started on its compute unit. That is a quarter of the time
// of a short (local-window) item.
//
// The queue: one counter per XCD over that XCD's share of the item ids, in
// the order of the one-item-per-workgroup grid (xcd_remap, tile_order: the
// items of a head stay on one XCD, causal items longest first). A workgroup
// takes from its own XCD's counter and, once that is exhausted, from the
// others'. The XCDs of a chip do not run at the same speed (9% apart in the
// clock counter of one run), so a static share would leave the fast ones idle
// at the end. An item is taken two steps before the previous one ends (just
// in time for the walker to copy its first tiles); taking it a whole item
// ahead held work back from idle workgroups. Thread 0 takes the items and
// hands them over through LDS. The counters live in the backward workspace:
// the pre-kernel zeroes them, and the last workgroup to finish zeroes them
// again, so repeated passes and graph replays find them at zero.
#include "attn_device.hpp"
#include "attn_internal.h"

#include <atomic>

namespace attn {
namespace {

constexpr int QD = 128;                     // head_dim
constexpr int QNP = 4;                      // wave pairs, 32 keys each
constexpr int QBN = 32 * QNP;               // keys per item
constexpr int QBM = 64;                     // query rows per tile (two 32-row blocks)
constexpr int QNST = 3;                     // ring stages
constexpr int QTHREADS = 128 * QNP;         // QNP S waves, then QNP dP waves
constexpr int QKS = QD / 16;                // MFMA k-steps over head_dim
constexpr int QDB = QD / 32;                // 32-column blocks of dK / dV
constexpr int QR = 4;                       // depth of the fragment read-ahead
constexpr int QTILE = QBM * QD;             // elements of one Q or dO tile
constexpr int TB = QTILE * 2;               // bytes of one tile
constexpr int BB = 32 * QD * 2;             // bytes of one 32-row block
constexpr int R_OFF = 0;                    // row terms: 16 bytes per query row
constexpr int Q_OFF = QNST * QBM * 16;      // Q stages
constexpr int G_OFF = Q_OFF + QNST * TB;    // dO stages
constexpr int XN = 4;                       // hand-over slots
constexpr int X_OFF = G_OFF + QNST * TB;    // P hand-over: [XN][QNP waves][2 halves][64 lanes] x 16 B
constexpr int XB = QNP * 2 * 1024;          // bytes of one hand-over slot
constexpr int SMEM = X_OFF + XN * XB;
static_assert(QBN == kBwdBlockN, "an item is one 128-key tile");
static_assert(XN * XB == QBN * QD * 2, "the hand-over slots hold an item's K rows");
static_assert(kBwdQueueWords >= 9, "eight queues and the count of finished workgroups");

// One item and the query tiles it visits (all wave-uniform).
struct Item {
  int b, kh, split, k0, kvlim, qt_begin, nq, nh, h_lo;
};

__global__ __launch_bounds__(QTHREADS) void attn_dkdv_queue_kernel(BwdArgs a, int n_items) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  // The taker thread's queue state and the items it took, shared through LDS
  // so that none of it stays in registers through the step loops: the current
  // item in items_s[cs], the next one in items_s[cs ^ 1].
  __shared__ Item items_s[2];
  __shared__ unsigned q_gone;   // queues found exhausted
  __shared__ int q_pend_valid;  // an index of the own queue is on its way
  uint16_t* const q_st = (uint16_t*)(smem + Q_OFF);
  uint16_t* const g_st = (uint16_t*)(smem + G_OFF);
  uint16_t* const r_st = (uint16_t*)(smem + R_OFF);
  uint16_t* const k_lds = (uint16_t*)(smem + X_OFF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave / QNP;  // 0: S, P, dV; 1: dP, dS, dK
  const int w4 = wave % QNP;    // key block of the pair
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const long krs = (long)a.Hkv * QD;
  const long qrs = (long)a.Hq * QD;
  const float c = a.scale_log2;

  // ---- queue (thread 0) ----
  unsigned* const ctr = a.queue;
  const int xq = (int)(xcc_id() & 7);
  const int qn = n_items / 8, qr = n_items % 8;
  auto qstart = [&](int x) { return x * qn + (x < qr ? x : qr); };
  // The queue is served by the first lane of the first dP wave: the S waves
  // issue most of the instructions and stay free of it.
  constexpr int kTaker = QTHREADS / 2;
  unsigned pend = 0;  // index of the own queue taken ahead of its use (taker)
  if (tid == kTaker) {
    q_gone = 0;
    q_pend_valid = 0;
  }
  // take_begin sends the atomic for the own queue; take_end uses its result
  // (two steps later, so the round trip is hidden) or, once the own queue is
  // exhausted, takes from the others. Taker thread only.
  auto take_begin = [&]() {
    if (!((q_gone >> xq) & 1u)) {
      pend = atomicAdd(ctr + xq, 1u);
      q_pend_valid = 1;
    }
  };
  auto take_end = [&]() -> int {
    if (!q_pend_valid) take_begin();
    unsigned gone = q_gone;
    int r = -1;
    if (q_pend_valid) {
      q_pend_valid = 0;
      if (pend < (unsigned)(qstart(xq + 1) - qstart(xq))) r = qstart(xq) + (int)pend;
      else gone |= 1u << xq;
    }
    for (int d = 1; d < 8 && r < 0; ++d) {
      const int x = (xq + d) & 7;
      if ((gone >> x) & 1u) continue;
      const unsigned i = atomicAdd(ctr + x, 1u);
      if (i < (unsigned)(qstart(x + 1) - qstart(x))) r = qstart(x) + (int)i;
      else gone |= 1u << x;
    }
    q_gone = gone;
    return r;
  };

  // ---- items ----
  auto make_item = [&](int id, Item& it) {
    int kt, rest;
    tile_order(id, a.num_ktiles, a.kv_split * a.B * a.Hkv, a.causal, rest, kt);
    it.kh = rest % a.Hkv;
    rest /= a.Hkv;
    it.b = rest % a.B;
    it.split = rest / a.B;
    it.h_lo = it.split * a.heads_per_split;
    it.nh = min(a.heads_per_split, G - it.h_lo);
    it.k0 = kt * QBN;
    it.kvlim = __builtin_amdgcn_readfirstlane(clamp_len(a.kv_lens, it.b, a.Tkv));
    const int kmax = min(it.k0 + QBN, it.kvlim) - 1;
    int i_lo = a.causal ? it.k0 : 0;
    if (a.win_right >= 0) i_lo = max(i_lo, it.k0 - a.win_right);
    int i_hi = a.Tq - 1;
    if (a.win_left >= 0) i_hi = min(i_hi, kmax + a.win_left);
    it.qt_begin = i_lo / QBM;
    it.nq = i_hi >= i_lo && it.k0 < it.kvlim ? i_hi / QBM + 1 - it.qt_begin : 0;
    // Every field is one value for the whole wave. Without saying so (the KV
    // length comes through a vector load here) the compiler kept the copy
    // walker's state per lane and ran the step loops under exec masks.
    for (int* f : {&it.b, &it.kh, &it.split, &it.k0, &it.qt_begin, &it.nq, &it.nh, &it.h_lo})
      *f = __builtin_amdgcn_readfirstlane(*f);
  };

  f32x16_t acc[QDB];  // dV^T (S wave) or dK^T (dP wave)
#pragma unroll
  for (int i = 0; i < QDB; ++i) acc[i] = f32x16_t{};

  // Store of an item's sums (zeros when `zero`): lane = key, register r of
  // block db = head_dim 32 db + 8 (r / 4) + 4 hh + r % 4; the S wave holds dV,
  // the dP wave dK.
  auto store = [&](const Item& it, bool zero) {
    const int key = it.k0 + 32 * w4 + l32;
    if (key >= a.Tkv) return;
    const bool is_dk = role == 1;
    const long kvoff = ((long)it.b * a.Tkv * a.Hkv + it.kh) * QD;
    if (a.kv_split > 1) {
      const long part = (long)a.B * a.Tkv * krs;
      float* dst = a.dkv_part + (is_dk ? it.split : a.kv_split + it.split) * part + kvoff + key * krs;
#pragma unroll
      for (int db = 0; db < QDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_t v = zero ? f32x4_t{0.f, 0.f, 0.f, 0.f}
                                 : f32x4_t{acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
          *(f32x4_t*)(dst + 32 * db + 8 * g + 4 * hh) = v;
        }
      return;
    }
    const float f = is_dk ? a.scale : 1.f;
    uint16_t* dst = (uint16_t*)(is_dk ? a.dk : a.dv) + kvoff + key * krs;
#pragma unroll
    for (int db = 0; db < QDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t v = zero ? u32x2_t{0u, 0u}
                               : u32x2_t{pack_bf16(acc[db][4 * g] * f, acc[db][4 * g + 1] * f),
                                         pack_bf16(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f)};
        *(u32x2_t*)(dst + 32 * db + 8 * g + 4 * hh) = v;
      }
  };
  // An item the taker published in LDS, read where it is needed.
  auto read_item = [&](int slot) {
    const Item& src = items_s[slot];
    Item it;
    it.b = __builtin_amdgcn_readfirstlane(src.b);
    it.kh = __builtin_amdgcn_readfirstlane(src.kh);
    it.split = __builtin_amdgcn_readfirstlane(src.split);
    it.k0 = __builtin_amdgcn_readfirstlane(src.k0);
    it.kvlim = __builtin_amdgcn_readfirstlane(src.kvlim);
    it.qt_begin = __builtin_amdgcn_readfirstlane(src.qt_begin);
    it.nq = __builtin_amdgcn_readfirstlane(src.nq);
    it.nh = __builtin_amdgcn_readfirstlane(src.nh);
    it.h_lo = __builtin_amdgcn_readfirstlane(src.h_lo);
    return it;
  };
  // The taker takes the next item with tiles and publishes it in `slot` (nq <
  // 0: none left); items without tiles (past the KV length, or no query row
  // sees their keys) get zeros on the way. Every wave calls it at the same
  // point.
  auto next_item = [&](int slot) -> bool {
    for (;;) {
      __syncthreads();  // every wave is done with what the slot held
      if (tid == kTaker) {
        const int id = take_end();
        Item it;
        it.nq = -1;
        if (id >= 0) make_item(id, it);
        items_s[slot] = it;
      }
      __syncthreads();
      const int nq = __builtin_amdgcn_readfirstlane(items_s[slot].nq);
      if (nq != 0) return nq > 0;
      store(read_item(slot), true);
    }
  };

  int cs = 0;  // LDS slot of the current item
  if (next_item(cs)) {
    Item cur = read_item(cs);
    // Lane byte offsets: the row operand is Q (S wave) or dO (dP wave), the
    // transposed operand the other one.
    const int tr_row = 4 * hh + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const uint32_t row_base = role == 0 ? Q_OFF : G_OFF;
    const uint32_t tr_base = role == 0 ? G_OFF : Q_OFF;
    uint32_t row_off[QKS], tr_off[QDB][2];
#pragma unroll
    for (int t = 0; t < QKS; ++t) row_off[t] = row_base + 2 * swz_off<QD>(l32, 16 * t + 8 * hh);
#pragma unroll
    for (int db = 0; db < QDB; ++db) {
      tr_off[db][0] = tr_base + 2 * swz_off<QD>(tr_row, 32 * db + tr_col);
      tr_off[db][1] = tr_base + 2 * swz_off<QD>(tr_row + 8, 32 * db + tr_col);
    }
    const uint32_t x_off = X_OFF + (w4 * 2 * 64 + lane) * 16;  // + slot * XB + half * 1024

    // ---- tile copies ----
    // Tile t of an item is query tile qt_begin + t % nq of head h_lo + t / nq.
    // Inside an item's step loop the walker (iss_*) advances by one tile per
    // step without divisions; an item's first two tiles are copied by
    // issue_item_tile during the previous item's last two steps.
    const TileCopy<QD, QBM, QTHREADS> qcopy(qrs, tid);
    auto issue_tile = [&](const uint16_t* qh, const uint16_t* gh, const uint16_t* rh, int q0, int st) {
      uint16_t* qs = q_st + st * QTILE;
      if (q0 + QBM <= a.Tq) {
        qcopy.template copy2<G_OFF - Q_OFF>(qs, qh, gh, qrs, q0);
      } else {
        dma_tile<QD, QBM, QTHREADS>(qs, qh, qrs, q0, a.Tq, tid);
        dma_tile<QD, QBM, QTHREADS>(g_st + st * QTILE, gh, qrs, q0, a.Tq, tid);
      }
      if (wave == 0 && lane < QBM) {
        const int i = min(q0 + lane, a.Tq - 1);
        dma16(rh + (long)i * 8, lds_addr(r_st + st * QBM * 8));
      }
    };
    auto head_ptrs = [&](const Item& it, int h, const uint16_t*& qh, const uint16_t*& gh, const uint16_t*& rh) {
      const long hb = (long)it.b * a.Tq * a.Hq + it.kh * G + it.h_lo + h;
      qh = (const uint16_t*)a.q + hb * QD;
      gh = (const uint16_t*)a.dout + hb * QD;
      rh = a.rowstat + (((long)it.b * a.Hq + it.kh * G + it.h_lo + h) * a.Tq) * 8;
    };
    auto issue_item_tile = [&](const Item& it, int t, int st) {
      const uint16_t *qh, *gh, *rh;
      head_ptrs(it, t / it.nq, qh, gh, rh);
      issue_tile(qh, gh, rh, (it.qt_begin + t % it.nq) * QBM, st);
    };
    int iss_q = 0, iss_st = 0;
    const uint16_t *iss_qh, *iss_gh, *iss_rh;
    // Walker at tile t of `it`, whose copy goes to stage st.
    auto walk_from = [&](const Item& it, int t, int st) {
      head_ptrs(it, t / it.nq, iss_qh, iss_gh, iss_rh);
      iss_q = t % it.nq;
      iss_st = st;
    };
    auto issue_next = [&](int nq, int qt_begin) {
      issue_tile(iss_qh, iss_gh, iss_rh, (qt_begin + iss_q) * QBM, iss_st);
      iss_st = iss_st + 1 == QNST ? 0 : iss_st + 1;
      if (++iss_q == nq) {
        iss_q = 0;
        iss_qh += QD;
        iss_gh += QD;
        iss_rh += (long)a.Tq * 8;
      }
    };
    bool nxt_ready = false;  // the item after `cur` is taken (and published in LDS)
    auto resolve = [&]() { nxt_ready = next_item(cs ^ 1); };
    // The taker publishes the next item itself, before the barrier of a step
    // (every wave reads it after that barrier); take_begin went out two steps
    // earlier. An item without tiles still goes the way of next_item.
    auto publish = [&]() {
      const int id = take_end();
      Item it;
      it.nq = -1;
      if (id >= 0) make_item(id, it);
      items_s[cs ^ 1] = it;
    };
    auto collect = [&]() {
      const int nq = __builtin_amdgcn_readfirstlane(items_s[cs ^ 1].nq);
      if (nq == 0) {
        store(read_item(cs ^ 1), true);
        resolve();
      } else {
        nxt_ready = nq > 0;
      }
    };
    // K (S waves) and V (dP waves) rows of the first item into LDS: K into the
    // hand-over slots, V into the stage of the item's third tile (keys 0..63
    // in its Q part, 64..127 in its dO part); both areas are free until the
    // first row products.
    auto copy_kv = [&](const Item& it, int st) {
      const long kvoff = ((long)it.b * a.Tkv * a.Hkv + it.kh) * QD;
      const uint16_t* kg = (const uint16_t*)a.k + kvoff;
      const uint16_t* vg = (const uint16_t*)a.v + kvoff;
      dma_tile<QD, 64, QTHREADS>(k_lds, kg, krs, it.k0, it.kvlim, tid);
      dma_tile<QD, 64, QTHREADS>(k_lds + 64 * QD, kg, krs, it.k0 + 64, it.kvlim, tid);
      dma_tile<QD, 64, QTHREADS>(q_st + st * QTILE, vg, krs, it.k0, it.kvlim, tid);
      dma_tile<QD, 64, QTHREADS>(g_st + st * QTILE, vg, krs, it.k0 + 64, it.kvlim, tid);
    };
    u32x4_t frag[QKS];  // K (S wave) or V (dP wave) rows of the lane's key: B operands
    // A later item's rows straight from memory (in the current item's last
    // step, once its own rows are no longer read).
    auto load_frag = [&](const Item& it) {
      const int key = it.k0 + 32 * w4 + l32;
      const uint16_t* src = (const uint16_t*)(role == 0 ? a.k : a.v) + ((long)it.b * a.Tkv * a.Hkv + it.kh) * QD +
                            (long)key * krs + 8 * hh;
      const bool key_ok = key < it.kvlim;
#pragma unroll
      for (int t = 0; t < QKS; ++t) frag[t] = key_ok ? gload16(src + 16 * t) : u32x4_t{0, 0, 0, 0};
    };
    auto read_frag = [&](const Item& it, int st) {
      const int r = 32 * w4 + l32;  // row of the lane's key in the 128-key tile
      const bool key_ok = it.k0 + r < it.kvlim;
      const uint16_t* kv = role == 0 ? k_lds + (r >> 6) * 64 * QD : (r < 64 ? q_st : g_st) + st * QTILE;
#pragma unroll
      for (int t = 0; t < QKS; ++t)
        frag[t] = key_ok ? lds_read16(kv + swz_off<QD>(r & 63, 16 * t + 8 * hh)) : u32x4_t{0, 0, 0, 0};
    };

    // Row terms as one extra k-step: the S wave selects -LSE/scale, the dP wave -D.
    const unsigned one2 = 0x3F803F80u, one1 = 0x00003F80u;
    const u32x4_t sel = hh != 0 ? u32x4_t{0, 0, 0, 0}
                        : role == 0 ? u32x4_t{one2, one1, 0, 0} : u32x4_t{0, 0, one2, one1};
    // Row product of block `half` of the tile in stage `st`: S (S wave) or dP
    // (dP wave), row terms included.
    auto row_product_at = [&](int st, int half) {
      const uint32_t bo = (uint32_t)__builtin_amdgcn_readfirstlane(st * TB + half * BB);
      const u32x4_t terms = lds_read16((const uint16_t*)(smem + R_OFF + (st * QBM + 32 * half + l32) * 16));
      u32x4_t ra[QR];
#pragma unroll
      for (int m = 0; m < QR; ++m) ra[m] = lds_read16((const uint16_t*)(smem + row_off[m] + bo));
      f32x16_t r = f32x16_t{};
#pragma unroll
      for (int m = 0; m < QKS; ++m) {
        r = mfma_bf16(ra[m % QR], frag[m], r);
        if (m + QR < QKS) ra[m % QR] = lds_read16((const uint16_t*)(smem + row_off[m + QR] + bo));
      }
      return mfma_bf16(terms, sel, r);
    };
    // Transposed product of block `half` of the tile in stage `st`:
    // acc += (dO or Q)^T x packed B operand.
    auto tr_product_at = [&](int st, int half, const u32x4_t (&pk)[2]) {
      const uint32_t bo = (uint32_t)__builtin_amdgcn_readfirstlane(st * TB + half * BB);
      u32x2_t tra[QR][2];
      auto rd = [&](int m, int slot) {
        const int u = m / QDB, db = m % QDB;
        tra[slot][0] = lds_read_tr((const uint16_t*)(smem + tr_off[db][0] + bo + 16 * u * QD * 2));
        tra[slot][1] = lds_read_tr((const uint16_t*)(smem + tr_off[db][1] + bo + 16 * u * QD * 2));
      };
#pragma unroll
      for (int m = 0; m < QR; ++m) rd(m, m);
#pragma unroll
      for (int m = 0; m < QKS; ++m) {
        const int u = m / QDB, db = m % QDB, slot = m % QR;
        acc[db] = mfma_bf16(u32x4_t{tra[slot][0][0], tra[slot][0][1], tra[slot][1][0], tra[slot][1][1]}, pk[u],
                            acc[db]);
        if (m + QR < QKS) rd(m + QR, slot);
      }
    };
    auto pack8 = [](const float* v) {
      return u32x4_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    };

    // First item: its first two tiles (a one-tile item needs the next item's
    // first tile as its second) and its K/V rows.
    int st0 = 0;  // stage of the current item's first tile
    issue_item_tile(cur, 0, 0);
    if (cur.nh * cur.nq >= 2) {
      issue_item_tile(cur, 1, 1);
    } else {
      resolve();
      if (nxt_ready) issue_item_tile(read_item(cs ^ 1), 0, 1);
    }
    copy_kv(cur, 2);
    wait_vmem();
    __syncthreads();
    read_frag(cur, 2);
    __syncthreads();

    for (;;) {
      const int nq = cur.nq, ntiles = cur.nh * cur.nq, qt_begin = cur.qt_begin, kvlim = cur.kvlim;
      // Steps 0 .. ntiles - 3 copy the item's own tiles 2 .. ntiles - 1; step
      // ntiles - 2 copies the next item's first tile and step ntiles - 1 its
      // second, so the next item is taken before step ntiles - 2.
      const int nmain = ntiles >= 2 ? ntiles - 2 : 0;
      const bool need_next = !nxt_ready;
      const bool early = need_next && nmain >= 1;  // the next item is published before a step's barrier
      walk_from(cur, 2, st0 + 2 >= QNST ? st0 + 2 - QNST : st0 + 2);
      // Copies of the last two steps: the next item's tiles 0 and 1.
      auto issue_peeled = [&](int t) {
        if (!nxt_ready) return;
        const Item nx = read_item(cs ^ 1);
        if (t < nx.nh * nx.nq) issue_item_tile(nx, t, iss_st);
        iss_st = iss_st + 1 == QNST ? 0 : iss_st + 1;
      };
      const int key = cur.k0 + 32 * w4 + l32;
      const int wave_min_key = cur.k0 + 32 * w4;
      const int wave_max_key = wave_min_key + 31;
      auto mask_q0 = [&](int q0) {
        return (wave_min_key < key_lo(q0 + QBM - 1, a.win_left)) ||
               (wave_max_key > key_hi(q0, kvlim, a.causal, a.win_right)) || (q0 + QBM > a.Tq);
      };
      if (role == 0) {
        u32x4_t pk[2];
        // P of block blk of the tile at query row qt0 (masked when msk).
        auto softmax_at = [&](int blk, const f32x16_t& s, bool msk, int qt0) {
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(s[r] * c);
          if (msk) {
            const int q0 = qt0 + 32 * (blk % 2);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ql = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
              const bool ok = (key >= key_lo(ql, a.win_left)) & (key <= key_hi(ql, kvlim, a.causal, a.win_right)) &
                              (ql < a.Tq);
              pv[r] = ok ? pv[r] : 0.f;
            }
          }
          pk[0] = pack8(pv);
          pk[1] = pack8(pv + 8);
          const uint32_t xo = x_off + (blk % XN) * XB;
          lds_write16((uint16_t*)(smem + xo), pk[0]);
          lds_write16((uint16_t*)(smem + xo + 1024), pk[1]);
        };
        u32x4_t pa[2], pb[2];
        int sm_q = 0;
        int sq0 = qt_begin * QBM;
        bool msk = mask_q0(sq0);
        auto sm_advance = [&](int t_next) {
          if (++sm_q == nq) sm_q = 0;
          sq0 = (qt_begin + sm_q) * QBM;
          msk = t_next < ntiles && mask_q0(sq0);
        };
        softmax_at(0, row_product_at(st0, 0), msk, sq0);
        pa[0] = pk[0];
        pa[1] = pk[1];
        softmax_at(1, row_product_at(st0, 1), msk, sq0);
        pb[0] = pk[0];
        pb[1] = pk[1];
        sm_advance(1);
        __syncthreads();
        int st_j = st0, st_n = st0 + 1 == QNST ? 0 : st0 + 1;  // stages of tiles j and j + 1
        // Step j: the transposed products of tile j's blocks 2j and 2j + 1
        // (their P from the previous step) and the row products and softmax
        // of tile j + 1's blocks, one block after the other, then one barrier.
        auto step = [&](int j) {
          // The S wave issues its row product at raised priority: its
          // softmax, and through P the partner's next step, wait on it.
          __builtin_amdgcn_s_setprio(1);
          f32x16_t s = row_product_at(st_n, 0);
          __builtin_amdgcn_s_setprio(0);
          tr_product_at(st_j, 0, pa);
          softmax_at(2 * j + 2, s, msk, sq0);
          pa[0] = pk[0];
          pa[1] = pk[1];
          __builtin_amdgcn_sched_barrier(0);  // one block's state live at a time
          s = row_product_at(st_n, 1);
          tr_product_at(st_j, 1, pb);
          softmax_at(2 * j + 3, s, msk, sq0);
          pb[0] = pk[0];
          pb[1] = pk[1];
          sm_advance(j + 2);
          st_j = st_n;
          st_n = st_n + 1 == QNST ? 0 : st_n + 1;
          wait_vmem();  // the tile issued above is read from the next step on
          __syncthreads();
        };
        for (int j = 0; j < nmain; ++j) {
          issue_next(nq, qt_begin);
          step(j);
        }
        if (early) collect();
        else if (need_next) resolve();
        if (ntiles >= 2) {
          issue_peeled(0);
          step(ntiles - 2);
        }
        // Last step: the transposed products only (no tile follows in this
        // item); the next item's K rows load meanwhile.
        issue_peeled(ntiles >= 2 ? 1 : 1);
        if (nxt_ready) load_frag(read_item(cs ^ 1));
        tr_product_at(st_j, 0, pa);
        tr_product_at(st_j, 1, pb);
        st_j = st_n;
        wait_vmem();
        __syncthreads();
        st0 = st_j;
      } else {
        auto ds_of = [&](int blk, const f32x16_t& dp, u32x4_t (&pk)[2]) {
          const uint32_t xo = x_off + (blk % XN) * XB;
          const u32x4_t p0 = lds_read16((const uint16_t*)(smem + xo));
          const u32x4_t p1 = lds_read16((const uint16_t*)(smem + xo + 1024));
          float dsv[16];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            dsv[2 * w] = bf16_lo(p0[w]) * dp[2 * w];
            dsv[2 * w + 1] = bf16_hi(p0[w]) * dp[2 * w + 1];
            dsv[8 + 2 * w] = bf16_lo(p1[w]) * dp[8 + 2 * w];
            dsv[8 + 2 * w + 1] = bf16_hi(p1[w]) * dp[8 + 2 * w + 1];
          }
          pk[0] = pack8(dsv);
          pk[1] = pack8(dsv + 8);
        };
        __syncthreads();
        int st_j = st0;
        // Step j: tile j's blocks one after the other, dP' and dS formed in
        // the step (P from the previous step).
        auto step = [&](int j) {
          u32x4_t pk[2];
          const f32x16_t dp0 = row_product_at(st_j, 0);
          const f32x16_t dp1 = row_product_at(st_j, 1);
          ds_of(2 * j, dp0, pk);
          tr_product_at(st_j, 0, pk);
          ds_of(2 * j + 1, dp1, pk);
          tr_product_at(st_j, 1, pk);
          st_j = st_j + 1 == QNST ? 0 : st_j + 1;
          wait_vmem();  // the tile issued above is read from the next step on
          __syncthreads();
        };
        // The taker sends the queue's atomic two steps before it publishes the
        // next item, and publishes it before the barrier of the last main
        // step; all between runs of the same loop (no test inside it).
        const int npub = early ? nmain - 1 : nmain;
        const int nbefore = early ? (npub >= 2 ? npub - 2 : 0) : (need_next && nmain >= 2 ? nmain - 2 : 0);
        for (int j = 0; j < nbefore; ++j) {
          issue_next(nq, qt_begin);
          step(j);
        }
        if (need_next && tid == kTaker) take_begin();
        for (int j = nbefore; j < npub; ++j) {
          issue_next(nq, qt_begin);
          step(j);
        }
        if (early && tid == kTaker) publish();
        for (int j = npub; j < nmain; ++j) {
          issue_next(nq, qt_begin);
          step(j);
        }
        if (early) collect();
        else if (need_next) resolve();
        if (ntiles >= 2) {
          issue_peeled(0);
          step(ntiles - 2);
        }
        {  // last step: the next item's V rows load once this item's are read
          issue_peeled(1);
          u32x4_t pk[2];
          const f32x16_t dp0 = row_product_at(st_j, 0);
          const f32x16_t dp1 = row_product_at(st_j, 1);
          if (nxt_ready) load_frag(read_item(cs ^ 1));
          ds_of(2 * ntiles - 2, dp0, pk);
          tr_product_at(st_j, 0, pk);
          ds_of(2 * ntiles - 1, dp1, pk);
          tr_product_at(st_j, 1, pk);
          st_j = st_j + 1 == QNST ? 0 : st_j + 1;
          wait_vmem();
          __syncthreads();
        }
        st0 = st_j;
      }
      // Item done (every wave has passed its last barrier; the next item's
      // K/V rows are in registers): store this item's sums.
      store(read_item(cs), false);
#pragma unroll
      for (int i = 0; i < QDB; ++i) acc[i] = f32x16_t{};
      if (!nxt_ready) break;
      cs ^= 1;
      cur = read_item(cs);
      nxt_ready = false;
      // A one-tile item's second tile is the following item's first: take
      // that item now and copy its first tile.
      if (cur.nh * cur.nq == 1) {
        resolve();
        if (nxt_ready) {
          issue_item_tile(read_item(cs ^ 1), 0, st0 + 1 == QNST ? 0 : st0 + 1);
          wait_vmem();
          __syncthreads();
        }
      }
    }
  }

  // Done: the taker counts the workgroup out; the last one zeroes the counters.
  if (tid == kTaker) {
    const unsigned done = atomicAdd(ctr + 8, 1u);
    if (done + 1 == gridDim.x) {
#pragma unroll
      for (int x = 0; x < 9; ++x) atomicExch(ctr + x, 0u);
    }
  }
}

// Compute units of the current device: the persistent grid, one workgroup each.
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

void launch_dkdv_queue(const BwdArgs& a, hipStream_t s) {
  const long items = (long)a.kv_split * a.num_ktiles * a.Hkv * a.B;
  if (items <= 0) return;
  const int cu = compute_units();
  const int grid = items < cu ? (int)items : cu;
  hipLaunchKernelGGL(attn_dkdv_queue_kernel, dim3((unsigned)grid), dim3(QTHREADS), 0, s, a, (int)items);
}

}  // namespace attn
