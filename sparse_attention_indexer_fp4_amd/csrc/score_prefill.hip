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
// physical page and gives each unit a start record. A unit is one workgroup of 8 waves and
// one unit runs per CU; it takes a contiguous range of items, and wave w scores rows w and
// w + 8 of each item's tile:
//   - the page goes straight into MFMA operand registers, as in the decode scorer (for key
//     tile t lane l loads the 16 bytes of key 16t + l%16 that hold elements [32(l/16), +32),
//     1 KiB of contiguous keys per instruction, and the scale dword at byte 4l, whose byte t
//     is that key's scale for group l/16); a step's keys (a few MB at most) stay in every
//     XCD's L2, and the unit's waves read the same page at about the same time, so the page
//     is fetched once per CU;
//   - each wave keeps D pages in flight in a register ring and runs on its own: no LDS, no
//     barrier, so the waves of a SIMD drift apart and one's MFMAs run while another reduces;
//   - the two rows share the page registers, and their MFMAs and epilogues interleave;
//   - an item's logits are stored after its slot's refill is issued, so waiting for a page
//     never waits for a store's completion, and with the non-temporal hint: a step writes
//     tens of MB of logits, which would otherwise push the step's key pages (read again and
//     again by every tile of their request) out of L2.
// The unit's first items come from its start record (one scalar load), so the first pages are
// in flight after a single round trip; the pages of later items come from the schedule's item
// table by scalar loads issued D items ahead. Each wave's two query rows sit in registers and
// are reloaded when the items cross into the next tile (at most a few times per unit). Every
// slot refill is unconditional (past the unit's last item it reloads that item, whose logits
// are dropped) and logits past a row's length fall outside the range-checked store, so the
// compiler waits only for the page being scored. A unit handles at most 64 heads (4 MFMA
// M-tiles); more heads are scored in further passes over the same schedule that add their
// partial sums with range-checked atomic adds (one add per logit, so the result does not
// depend on timing).
#include "score_common.h"

// pages in flight per wave
#ifndef IFP4_PREFILL_RING
#define IFP4_PREFILL_RING 2
#endif

namespace ifp4 {

constexpr int kRowsPerWave = 2;                                 // rows w and w + NW of a tile
constexpr int kPrefillWaves = kPrefillTileRows / kRowsPerWave;  // 8
constexpr int kPrefillPassHeads16 = 4;                          // M-tiles of 16 heads per pass

// A tile as the scorer tracks it (wave-uniform): its record from the schedule.
struct TileState {
  int t, row0, nvalid, pos0, pages, item0;
};

template <int NH16, bool ADD, int D>
__global__ __launch_bounds__(kPrefillWaves * 64) void score_prefill_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    int head0, const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages, int64_t bt_ld,
    int n_req, int n_rows_padded, int n_units, const int32_t *__restrict__ sched_g, int32_t *__restrict__ err,
    float *__restrict__ logits, int64_t ld) {
  static_assert(D >= 1 && D <= kUnitRecPhys, "the start record holds the first ring fill's pages");
  constexpr int RPW = kRowsPerWave, NW = kPrefillWaves;
  const PrefillSchedLayout L(n_req, n_rows_padded, n_units, bt_ld);
  const const_ptr<int32_t> sched = as_const(sched_g);
  const int u = xcd_local_index(blockIdx.x, n_units);  // neighbouring units share an XCD's L2
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
  const int wv = uniform(threadIdx.x >> 6);  // this wave's rows inside a tile: wv and wv + NW
  const int n_my = it1 - it0;

  // the current tile (from the start record)
  TileState T;
  T.t = min(max(rv[2], 0), n_tiles - 1);
  T.row0 = rv[4];
  T.nvalid = rv[6];
  T.pos0 = rv[7];
  T.pages = rv[9];
  T.item0 = rv[10];
  // physical page of item i of the unit (clamped to its last item): the first D from the start
  // record, the others from the schedule's item table (scalar loads: their own counter)
  const const_ptr<int32_t> item_phys = sched + L.item_phys + it0;

  // the ring: pages in registers, the unit-relative item each slot holds
  PageRegs P[D];
  int sitem[D];
  bool sok[D];  // the slot's page was resolved (an unresolved item stores nothing)
  auto issue = [&](auto kk, int i, int phys) {
    constexpr int K = decltype(kk)::value;
    sitem[K] = i;
    sok[K] = phys >= 0;
    load_page_cached(P[K], kvp, kvs, phys >= 0 ? phys : 0, lane);  // page 0 exists; an unreadable page is not scored
  };
  int sphys[D];  // pages of the next refill of each slot, loaded one round ahead
  auto next_phys = [&](int i) { return item_phys[min(i, n_my - 1)]; };

  // This wave's two query rows (operands, scales, weights of this pass's heads) in registers.
  RowRegs<NH16, RPW> R;
  int row[RPW], len[RPW];
  auto load_row = [&]() __attribute__((always_inline)) {
    // the pass's heads [head0, head0 + 16 NH16) of each row (rows past the tile's valid ones
    // are not loaded: their logits fall outside the store's range whatever the registers hold)
    const uint8_t *q = qp + (int64_t)head0 * kKeyBytes;
    const uint8_t *s = qs + (int64_t)head0 * kGroups;
    const float *ww = w + head0;
    static_for<RPW>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      const int rw = wv + NW * J;
      row[J] = T.row0 + rw;
      len[J] = rw < T.nvalid ? T.pos0 + rw + 1 : 0;
      if (len[J] > 0) load_row_into<NH16, RPW>(R, J, q, s, ww, row[J], n_heads, lane);
    });
    // wait here (vmcnt 0): the compiler would otherwise take these loads as the youngest in
    // flight at every page and drain the ring before each page's MFMAs
    __builtin_amdgcn_s_waitcnt(0x0F70);
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

  // the last scored item's logits, stored after the slot's refill is issued: the refill's
  // loads then sit behind the stores in the memory counter, and the wait for the next slot's
  // page never includes a store's completion
  float s_v[RPW];
  __amdgpu_buffer_rsrc_t s_dst[RPW];
  uint32_t s_off = 0;
  auto score = [&](auto kk) __attribute__((always_inline)) {
    constexpr int K = decltype(kk)::value;
    const int i = sitem[K];
    if (it0 + min(i, n_my - 1) >= T.item0 + T.pages && T.t < n_tiles - 1) {  // into the next tile(s)
      do next_tile();
      while (it0 + min(i, n_my - 1) >= T.item0 + T.pages && T.t < n_tiles - 1);
      load_row();
    }
    const int p = it0 + min(i, n_my - 1) - T.item0;  // the item's page within its tile
    // an item past the unit's last, or whose page the schedule could not resolve, stores nothing
    const bool ok = i < n_my && sok[K];
    float v[RPW];
    static_for<RPW>([&](auto jj) { v[decltype(jj)::value] = page_logit<NH16, RPW, decltype(jj)::value, true>(P[K], R, lane); });
    s_off = 4u * (uint32_t)(p * kPage + lane);
    static_for<RPW>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      const uint32_t bytes = ok ? 4u * (uint32_t)max(len[J], 0) : 0u;
      s_dst[J] = buffer_view(logits + (int64_t)row[J] * ld, bytes);
      s_v[J] = v[J];
    });
  };
  auto store = [&]() __attribute__((always_inline)) {
    static_for<RPW>([&](auto jj) {
      constexpr int J = decltype(jj)::value;
      if constexpr (ADD) __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(s_v[J], s_dst[J], (int)s_off, 0, 0);
      else buffer_store_f32_nt(s_v[J], s_dst[J], s_off);
    });
  };

  // the first D pages from the start record, then the query rows (their wait also covers the
  // pages), then the loop: score slot K, refill it D items ahead
  static_for<D>([&](auto kk) {
    constexpr int K = decltype(kk)::value;
    issue(kk, K, K < n_my ? rv[12 + K] : -1);
  });
  static_for<D>([&](auto kk) { sphys[decltype(kk)::value] = next_phys(D + decltype(kk)::value); });
  load_row();
  for (int i0 = 0; i0 < n_my; i0 += D) {
    static_for<D>([&](auto kk) {
      constexpr int K = decltype(kk)::value;
      score(kk);
      const int nxt = i0 + K + D;
      issue(kk, nxt, sphys[K]);
      store();
      sphys[K] = next_phys(nxt + D);
    });
  }
}

template <int NH16, bool ADD>
static void launch_prefill_pass(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                                int n_heads, int head0, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages,
                                int64_t bt_ld, int n_req, int n_rows_padded, int32_t *sched, float *logits,
                                int64_t ld) {
  constexpr int D = IFP4_PREFILL_RING;
  hipLaunchKernelGGL((score_prefill_kernel<NH16, ADD, D>), dim3(n_units), dim3(kPrefillWaves * 64), 0, st, qp, qs,
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
