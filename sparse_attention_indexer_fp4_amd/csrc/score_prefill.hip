// Prefill scorer: row groups of a prefill step against the paged FP4 key cache.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), commit message: the FP4 prefill
// variant scores the chunk's query rows straight out of the paged cache; ROCm/ATOM #2125
// section 3: the row-group kernel finds a group's page table as group b -> block_tables[b],
// and padding rows, folded into the last request's group, read no key. Each valid row r
// at position p sees keys [0, p] (causal, inclusive).
//
// Design for gfx950. Work items are (tile, page) pairs where a tile is up to 16 rows of one
// request's group; the step's schedule (schedule.hip) has already turned every item into its
// physical page and gives each unit a start record. A unit is one workgroup of 16 waves, one
// per row of the tile, and one unit runs per CU (four waves per SIMD, all of one unit, so no
// unit's waves are starved by another's). The unit takes a contiguous range of items; all its
// waves walk the same items, so one key page feeds 16 rows x n_heads query heads of MFMA work.
//   - Pages go through a ring of P slots in LDS filled by direct global-to-LDS loads: four
//     waves copy one 1 KiB key tile each and a fifth the 256-byte scale block, lane i fetching
//     exactly the 16 bytes that lane i of every wave later reads as its MFMA operand (the
//     decode scorer's operand layout), so the LDS reads are linear.
//   - Items go in groups of B: per group the loader waves wait until their copies have
//     landed (vmcnt counting in issue order), the unit meets at one barrier, the slots of the
//     previous group are refilled P-B items ahead, and every wave scores its row for the whole
//     group from LDS without further synchronisation.
//   - Each wave holds its row's query operands, scales and weights in registers; they are
//     reloaded only when the items cross into the next tile (at most a few times per unit).
//   - The unit's first items come from its start record (one scalar load), so the first page
//     copies are in flight after a single round trip; the pages of its later items come from
//     the schedule's item table by scalar loads issued one group ahead.
// Logits past a row's length fall outside the range-checked store. A unit handles at most 64
// heads (4 MFMA M-tiles); more heads are scored in further passes over the same schedule that
// add their partial sums with range-checked atomic adds (one add per logit, so the result does
// not depend on timing).
#include "score_common.h"

// pages in the LDS ring of a unit, and items between the unit's barriers (divides the ring)
#ifndef IFP4_PREFILL_RING
#define IFP4_PREFILL_RING 8
#endif
#ifndef IFP4_PREFILL_GROUP
#define IFP4_PREFILL_GROUP 4
#endif

namespace ifp4 {

constexpr int kPrefillMaxRing = 8;
constexpr int kPrefillWaves = kPrefillTileRows;  // one wave per tile row
constexpr int kPrefillPassHeads16 = 4;           // M-tiles of 16 heads per pass

// One LDS array per ring slot: with every slot access indexed by a constant the compiler
// can tell the slots apart and adds no waits of its own between a slot's reads and the
// direct loads in flight into other slots.
#define IFP4_SLOT(I)                                                   \
  __shared__ __attribute__((aligned(16))) uint4 pf_keys##I[kPage * 4]; \
  __shared__ uint32_t pf_scales##I[kPage];
IFP4_SLOT(0) IFP4_SLOT(1) IFP4_SLOT(2) IFP4_SLOT(3) IFP4_SLOT(4) IFP4_SLOT(5) IFP4_SLOT(6) IFP4_SLOT(7)
#undef IFP4_SLOT

template <int S>
__device__ __forceinline__ uint4 *slot_keys() {
  static_assert(S >= 0 && S < kPrefillMaxRing, "ring slot");
  if constexpr (S == 0) return pf_keys0;
  else if constexpr (S == 1) return pf_keys1;
  else if constexpr (S == 2) return pf_keys2;
  else if constexpr (S == 3) return pf_keys3;
  else if constexpr (S == 4) return pf_keys4;
  else if constexpr (S == 5) return pf_keys5;
  else if constexpr (S == 6) return pf_keys6;
  else return pf_keys7;
}
template <int S>
__device__ __forceinline__ uint32_t *slot_scales() {
  if constexpr (S == 0) return pf_scales0;
  else if constexpr (S == 1) return pf_scales1;
  else if constexpr (S == 2) return pf_scales2;
  else if constexpr (S == 3) return pf_scales3;
  else if constexpr (S == 4) return pf_scales4;
  else if constexpr (S == 5) return pf_scales5;
  else if constexpr (S == 6) return pf_scales6;
  else return pf_scales7;
}

typedef __attribute__((address_space(3))) void lds_void;

// A tile as the scorer tracks it (wave-uniform): its record from the schedule.
struct TileState {
  int t, row0, nvalid, pos0, pages, item0;
};

template <int NH16, bool ADD, int P, int B>
__global__ __launch_bounds__(kPrefillWaves * 64) void score_prefill_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    int head0, const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages, int64_t bt_ld,
    int n_req, int n_rows_padded, int n_units, const int32_t *__restrict__ sched_g, int32_t *__restrict__ err,
    float *__restrict__ logits, int64_t ld) {
  static_assert(P <= kPrefillMaxRing && B >= 1 && P % B == 0 && P / B >= 2, "ring and groups");
  const PrefillSchedLayout L(n_req, n_rows_padded, n_units, bt_ld);
  const const_ptr<int32_t> sched = as_const(sched_g);
  const int u = blockIdx.x;
  // One scalar round: the header and this unit's start record (in bounds whatever they hold:
  // the host checked the buffer's size for these sizes). Nothing is used before the header
  // shows a schedule built for this step's sizes and this pool; a stale or zeroed buffer is
  // flagged once, by unit 0, and nothing is scored.
  const const_ptr<int32_t> rec = sched + L.urec + (int64_t)kUnitRecWords * u;
  int rv[kUnitRecWords];
#pragma unroll
  for (int j = 0; j < kUnitRecWords; j++) rv[j] = rec[j];
  if (sched[0] != kPrefillMagic || sched[2] != n_req || sched[3] != n_rows_padded || sched[4] != n_units ||
      sched[7] != kPrefillTileRows || sched[8] != (int32_t)bt_ld ||
      sched[9] != (int32_t)min(n_pages, (int64_t)INT32_MAX)) {
    if (u == 0 && threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
    return;
  }
  const int n_tiles = min(sched[5], (int)L.max_tiles);
  const int items = min(sched[6], (int)(L.max_tiles * bt_ld));
  const int it0 = max(rv[0], 0), it1 = min(rv[1], items);
  if (it0 >= it1 || n_tiles <= 0) return;  // empty unit (uniform over the workgroup): nothing else is touched
  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);  // this wave's row inside a tile
  const int n_my = it1 - it0;
  const bool loader = wv < 5;  // waves 0-3 copy key tiles, wave 4 the scale block

  // the current tile (from the start record), and this wave's row in it
  TileState T;
  T.t = min(max(rv[2], 0), n_tiles - 1);
  T.row0 = rv[4];
  T.nvalid = rv[6];
  T.pos0 = rv[7];
  T.pages = rv[9];
  T.item0 = rv[10];
  // Physical pages of the unit's items: the first (G-1)B from the start record, the others by
  // scalar loads from the schedule's item table one group before their copies are issued
  // (scalar loads wait on their own counter, not behind the copies in flight).
  constexpr int G = P / B;
  static_assert((G - 1) * B <= kUnitRecPhys, "the start record holds the prologue's pages");
  const const_ptr<int32_t> item_phys = sched + L.item_phys + it0;
  int nphys[B];
  auto prefetch = [&](int i) {  // pages of items i .. i+B-1 (clamped to the unit's last item)
    static_for<B>([&](auto bb) { nphys[decltype(bb)::value] = item_phys[min(i + (int)decltype(bb)::value, n_my - 1)]; });
  };

  // the first item of each ring group's slots, and one bit per slot: its item is scored
  int gbase[G];
  uint32_t live_bits = 0;
  // copy item i (past the unit's last item: that one again) with physical page `phys` into
  // ring slot S; the loader waves issue one direct load each (a page that cannot be read is
  // replaced by page 0, which exists, and is not scored)
  auto issue = [&](auto ss, int i, int phys) {
    constexpr int S = decltype(ss)::value;
    if constexpr (S % B == 0) gbase[S / B] = i;
    const bool live = i < n_my && phys >= 0;
    live_bits = live ? (live_bits | (1u << S)) : (live_bits & ~(1u << S));
    const int64_t pg = phys >= 0 ? phys : 0;
    if (wv < 4) {
      const uint8_t *src = kvp + pg * kPageBytes + 1024 * wv + 64 * (lane & 15) + 16 * (lane >> 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(slot_keys<S>() + 64 * wv), 16, 0, 0);
    } else if (wv == 4) {
      const uint8_t *src = kvs + pg * kPageScaleBytes + 4 * lane;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)slot_scales<S>(), 4, 0, 0);
    }
  };
  // a store that writes nothing (empty range): keeps every wave at one store per item
  auto idle_store = [&]() { buffer_store_f32(0.f, buffer_view(logits, 0u), 0u); };

  // This wave's query row (operands, scales, weights of this pass's heads) in registers.
  RowRegs<NH16, 1> R;
  int row = 0, len = 0;
  auto load_row = [&](bool wait) __attribute__((always_inline)) {
    row = T.row0 + wv;
    len = wv < T.nvalid ? T.pos0 + wv + 1 : 0;
    if (len > 0) {
      // the pass's heads [head0, head0 + 16 NH16) of row `row`
      const uint8_t *q = qp + (int64_t)head0 * kKeyBytes;
      const uint8_t *s = qs + (int64_t)head0 * kGroups;
      const float *ww = w + head0;
      if (wait) load_rows<NH16, 1, true>(R, q, s, ww, row, 1, n_heads, lane);
      else load_rows<NH16, 1, false>(R, q, s, ww, row, 1, n_heads, lane);
    }
  };
  auto next_tile = [&]() __attribute__((always_inline)) {
    // tiles of no page hold no item, so the next item's tile is found by walking forward
    T.t = min(T.t + 1, n_tiles - 1);
    const const_ptr<int32_t> rt = sched + L.tiles + (int64_t)kTileRecWords * T.t;
    T.row0 = rt[0];
    T.nvalid = rt[2];
    T.pos0 = rt[3];
    T.pages = rt[5];
    T.item0 = rt[6];
  };

  auto item_of = [&](auto ss) { return min(gbase[decltype(ss)::value / B] + decltype(ss)::value % B, n_my - 1); };
  auto score = [&](auto ss) __attribute__((always_inline)) {
    constexpr int S = decltype(ss)::value;
    const int p = it0 + item_of(ss) - T.item0;  // the item's page within its tile
    if (!((live_bits >> S) & 1u) || len <= p * kPage) {
      idle_store();
      return;
    }
    PageRegs pg;
#pragma unroll
    for (int t = 0; t < 4; t++) pg.k[t] = slot_keys<S>()[64 * t + lane];
    pg.s = slot_scales<S>()[lane];
    const float v = page_logit<NH16, 1, 0, (NH16 <= 3)>(pg, R, lane);  // one accumulator set at 64 heads (registers)
    const __amdgpu_buffer_rsrc_t dst = buffer_view(logits + (int64_t)row * ld, 4u * (uint32_t)len);
    const uint32_t off = 4u * (uint32_t)(p * kPage + lane);
    if constexpr (ADD) __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, dst, (int)off, 0, 0);
    else buffer_store_f32(v, dst, off);
  };
  // score the B items of group GG; a group that reaches into the next tile(s) moves there
  // item by item (loading the new row waits for every copy in flight: rare, a few times per
  // unit at most)
  auto score_group = [&](auto gg) __attribute__((always_inline)) {
    constexpr int GG = decltype(gg)::value;
    const int last = it0 + item_of(std::integral_constant<int, GG * B + B - 1>{});  // the group's items ascend
    if (last < T.item0 + T.pages) {
      static_for<B>([&](auto bb) { score(std::integral_constant<int, GG * B + decltype(bb)::value>{}); });
    } else {
      static_for<B>([&](auto bb) {
        constexpr int S = GG * B + decltype(bb)::value;
        bool moved = false;
        while (it0 + item_of(std::integral_constant<int, S>{}) >= T.item0 + T.pages && T.t < n_tiles - 1) {
          next_tile();
          moved = true;
        }
        if (moved) load_row(true);
        score(std::integral_constant<int, S>{});
      });
    }
  };

  // Items go in groups of B; the ring holds G = P / B groups. At the start of group k the
  // loader waves wait until the group's copies have landed, the unit meets once, the slots
  // of group k-1 are refilled with group k+G-1, and every wave scores its row for the B
  // items of group k without further synchronisation.
  // Prologue: groups 0 .. G-2 (pages from the start record), each followed by B idle stores
  // so that a loader wave issues the same sequence (B loads, then B stores) before every group.
  static_for<G - 1>([&](auto gg) {
    constexpr int GG = decltype(gg)::value;
    static_for<B>([&](auto bb) {
      constexpr int I = GG * B + decltype(bb)::value;
      issue(std::integral_constant<int, I>{}, I, I < n_my ? rv[12 + I] : -1);
    });
    if (loader) static_for<B>([&](auto) { idle_store(); });
  });
  prefetch((G - 1) * B);
  // the row's query, in flight with the first copies; its wait (vmcnt 0) also covers them,
  // and leaves no load the compiler would still have to wait for later
  load_row(true);
  for (int i0 = 0; i0 < n_my; i0 += P) {
    static_for<G>([&](auto gg) {
      constexpr int GG = decltype(gg)::value;
      // After the last load of this group a loader wave issued the stores of the G-1 groups
      // before it and the loads of the G-2 groups after it, B each, and memory operations
      // complete in issue order: at most B(2G-3) outstanding means the group is in LDS.
      if (loader) __builtin_amdgcn_s_waitcnt(0x0F70 | (B * (2 * G - 3)));
      __builtin_amdgcn_s_barrier();  // the group landed; the previous group's slots are free
      asm volatile("" ::: "memory");
      constexpr int GR = (GG + G - 1) % G;  // slots of the previous group
      const int ir = i0 + (GG + G - 1) * B;  // the refill's first item
      static_for<B>([&](auto bb) {
        constexpr int BB = decltype(bb)::value;
        issue(std::integral_constant<int, GR * B + BB>{}, ir + BB, nphys[BB]);
      });
      prefetch(ir + B);
      score_group(gg);
    });
  }
}

template <int NH16, bool ADD>
static void launch_prefill_pass(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                                int n_heads, int head0, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages,
                                int64_t bt_ld, int n_req, int n_rows_padded, int32_t *sched, float *logits,
                                int64_t ld) {
  constexpr int P = IFP4_PREFILL_RING, B = IFP4_PREFILL_GROUP;
  hipLaunchKernelGGL((score_prefill_kernel<NH16, ADD, P, B>), dim3(n_units), dim3(kPrefillWaves * 64), 0, st, qp, qs,
                     w, n_heads, head0, kvp, kvs, n_pages, bt_ld, n_req, n_rows_padded, n_units, sched, sched + 1,
                     logits, ld);
}

template <bool ADD>
static void launch_prefill(int nh16, hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs,
                           const float *w, int n_heads, int head0, const uint8_t *kvp, const uint8_t *kvs,
                           int64_t n_pages, int64_t bt_ld, int n_req, int n_rows_padded, int32_t *sched,
                           float *logits, int64_t ld) {
  switch (nh16) {
#define IFP4_CASE(X) \
  case X: launch_prefill_pass<X, ADD>(st, n_units, qp, qs, w, n_heads, head0, kvp, kvs, n_pages, bt_ld, n_req, n_rows_padded, sched, logits, ld); break;
    IFP4_CASE(1) IFP4_CASE(2) IFP4_CASE(3) IFP4_CASE(4)
#undef IFP4_CASE
  }
}

}  // namespace ifp4

using namespace ifp4;

extern "C" int indexer_fp4_score_prefill(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                                         int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                                         int64_t n_pages, int64_t bt_ld, int32_t n_req, void *sched,
                                         int64_t sched_bytes, int32_t n_units, int32_t n_rows_padded, float *logits,
                                         int64_t logits_ld, void *stream) {
  clear_error();
  if (n_heads <= 0 || n_heads % INDEXER_FP4_HEAD_MULT != 0 || n_heads > INDEXER_FP4_MAX_HEADS)
    return fail(INDEXER_FP4_EINVAL, "n_heads=%d must be a positive multiple of %d and at most %d", n_heads,
                INDEXER_FP4_HEAD_MULT, INDEXER_FP4_MAX_HEADS);
  if (n_req <= 0 || n_units <= 0 || n_pages < 0 || n_rows_padded <= 0 || n_rows_padded % kRowMultiple != 0)
    return fail(INDEXER_FP4_EINVAL,
                "score_prefill: n_req=%d > 0, n_units=%d > 0, n_pages=%lld >= 0, n_rows_padded=%d a positive multiple of %d",
                n_req, n_units, (long long)n_pages, n_rows_padded, kRowMultiple);
  if (bt_ld <= 0 || bt_ld > INT32_MAX)
    return fail(INDEXER_FP4_ENOSPC, "score_prefill: bt_ld=%lld must be in 1..2^31-1", (long long)bt_ld);
  if (logits_ld < bt_ld * kPage)
    return fail(INDEXER_FP4_ENOSPC, "score_prefill: logits_ld=%lld < 64*bt_ld=%lld", (long long)logits_ld,
                (long long)(bt_ld * kPage));
  if (!sched || !q_packed || !q_scale || !weights || !logits)
    return fail(INDEXER_FP4_EINVAL, "score_prefill: a required pointer is NULL");
  const int64_t need = 4 * PrefillSchedLayout(n_req, n_rows_padded, n_units, bt_ld).words;
  if (sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "score_prefill: sched_bytes=%lld < %lld for n_req=%d, n_rows_padded=%d, n_units=%d, "
                "bt_ld=%lld", (long long)sched_bytes, (long long)need, n_req, n_rows_padded, n_units, (long long)bt_ld);
  if (n_pages > 0 && (!kv_packed || !kv_scale)) return fail(INDEXER_FP4_EINVAL, "score_prefill: NULL cache plane");
  if (((uintptr_t)q_packed | (uintptr_t)weights | (uintptr_t)kv_packed | (uintptr_t)kv_scale) % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "score_prefill: q_packed, weights and both planes must be 16-byte aligned");
  if (((uintptr_t)sched | (uintptr_t)logits) % 4 != 0)
    return fail(INDEXER_FP4_EINVAL, "score_prefill: sched and logits must be 4-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t *sc = (int32_t *)sched;
  // heads in passes of at most 64: the first stores, the others add
  const int nh16 = n_heads / 16;
  for (int m0 = 0; m0 < nh16; m0 += kPrefillPassHeads16) {
    const int m = min(kPrefillPassHeads16, nh16 - m0);
    if (m0 == 0)
      launch_prefill<false>(m, st, n_units, q_packed, q_scale, weights, n_heads, 16 * m0, kv_packed, kv_scale,
                            n_pages, bt_ld, n_req, n_rows_padded, sc, logits, logits_ld);
    else
      launch_prefill<true>(m, st, n_units, q_packed, q_scale, weights, n_heads, 16 * m0, kv_packed, kv_scale,
                           n_pages, bt_ld, n_req, n_rows_padded, sc, logits, logits_ld);
    rc = launch_status("score_prefill");
    if (rc) return rc;
  }
  return INDEXER_FP4_OK;
}
