// Prefill scorer: row groups of a prefill step against the paged FP4 key cache.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), commit message: the FP4 prefill
// variant scores the chunk's query rows straight out of the paged cache; ROCm/ATOM #2125
// section 3: the row-group kernel finds a group's page table as group b -> block_tables[b],
// and padding rows, folded into the last request's group, read no key. Each valid row r
// at position p sees keys [0, p] (causal, inclusive).
//
// Design for gfx950. Work items are (tile, page) pairs where a tile is up to 8 rows of one
// request's group (schedule.hip). A unit (workgroup of NW waves) takes a contiguous range
// of items; all its waves walk the same items and wave w scores rows w*RPW .. w*RPW+RPW-1
// of the tile, so one key page feeds 8 rows x n_heads query heads of MFMA work while its
// bytes come from HBM once (later waves of the workgroup hit the CU's cache). Query rows
// stay in registers while the unit stays on a tile. A wave skips a page that none of its
// rows reaches (the causal triangle) and rows past a row's length are never stored.
#include "score_common.h"

namespace ifp4 {

template <int NH16, int RPW, int NW, int D>
__global__ __launch_bounds__(NW * 64) void score_prefill_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages,
    const int32_t *__restrict__ bt_g, int64_t bt_ld, int n_req, int n_rows_padded, int n_units,
    const int32_t *__restrict__ sched_g, int32_t *__restrict__ err, const int32_t *__restrict__ row_len_g,
    float *__restrict__ logits, int64_t ld) {
  const PrefillSchedLayout L(n_req, n_rows_padded, n_units);
  const const_ptr<int32_t> sched = as_const(sched_g), bt = as_const(bt_g), row_len = as_const(row_len_g);
  const int u = blockIdx.x;
  const int it0 = sched[L.unit_begin + u];
  const int it1 = sched[L.unit_begin + u + 1];
  if (it0 >= it1) return;  // empty unit: nothing else is touched
  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);
  if (sched[0] != kPrefillMagic || sched[2] != n_req || sched[3] != n_rows_padded || sched[4] != n_units) {
    if (threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
    return;
  }
  const int n_tiles = sched[5];
  const const_ptr<int32_t> tiles = sched + L.tiles;  // {first row, rows, request, pages} per tile
  auto tile = [&](int t) { return make_int4(tiles[4 * t], tiles[4 * t + 1], tiles[4 * t + 2], tiles[4 * t + 3]); };
  const const_ptr<int32_t> cum = sched + L.cum;
  const int n_items = it1 - it0;
  const int my_row0 = wv * RPW;  // this wave's first row inside a tile

  int tb = sched[L.unit_tile + u];  // issue-side tile cursor
  // query rows of the unit's first tile, loaded before any page (see score_decode.hip)
  RowRegs<NH16, RPW> R;
  int qt = tb;
  int row0, n_valid;
  {
    const int4 T = tile(qt);
    row0 = T.x + my_row0;
    n_valid = min(RPW, T.y - my_row0);
    load_rows<NH16, RPW>(R, qp, qs, w, row0, n_valid, n_heads, lane);
  }

  // Batches of D items: issue the page loads this wave needs, then score them.
  for (int i0 = 0; i0 < n_items; i0 += D) {
    PageRegs P[D];
    int st[D], sp[D];
    bool sok[D];
    static_for<D>([&](auto kk) {
      constexpr int K = decltype(kk)::value;
      sok[K] = false;
      st[K] = tb;
      sp[K] = 0;
      if (i0 + K < n_items) {
        const int it = it0 + i0 + K;
        while (tb < n_tiles - 1 && it >= cum[tb + 1]) tb++;
        const int4 T = tile(tb);
        const int p = it - cum[tb];
        st[K] = tb;
        sp[K] = p;
        bool need = false;
#pragma unroll
        for (int j = 0; j < RPW; j++)
          if (my_row0 + j < T.y && row_len[T.x + my_row0 + j] > p * kPage) need = true;
        if (need && p < 0) {
          if (lane == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
        } else if (need) {
          if (p >= bt_ld) {
            if (lane == 0) atomicOr(err, INDEXER_FP4_DEV_TABLE_SHORT);
          } else {
            const int64_t phys = bt[(int64_t)T.z * bt_ld + p];
            if (phys < 0 || phys >= n_pages) {
              if (lane == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
            } else {
              sok[K] = true;
              load_page(P[K], kvp, kvs, phys, lane);
            }
          }
        }
      }
    });
    static_for<D>([&](auto kk) {
      constexpr int K = decltype(kk)::value;
      if (sok[K]) {
        if (st[K] != qt) {
          qt = st[K];
          const int4 T = tile(qt);
          row0 = T.x + my_row0;
          n_valid = min(RPW, T.y - my_row0);
          load_rows<NH16, RPW>(R, qp, qs, w, row0, n_valid, n_heads, lane);
        }
        const int col = sp[K] * kPage + lane;
        static_for<RPW>([&](auto jj) {
          constexpr int J = decltype(jj)::value;
          if (J < n_valid) {
            const int64_t r = row0 + J;
            const int len = row_len[r];
            if (sp[K] * kPage < len) {
              const float v = page_logit<NH16, RPW, J>(P[K], R, lane);
              if (col < len) logits[r * ld + col] = v;
            }
          }
        });
      }
    });
  }
}

template <int NH16>
static void launch_prefill(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                           int n_heads, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages, const int32_t *bt,
                           int64_t bt_ld, int n_req, int n_rows_padded, int32_t *sched, const int32_t *row_len,
                           float *logits, int64_t ld) {
  constexpr int RPW = 1, NW = kTileRows / RPW, D = 2;
  hipLaunchKernelGGL((score_prefill_kernel<NH16, RPW, NW, D>), dim3(n_units), dim3(NW * 64), 0, st, qp, qs, w,
                     n_heads, kvp, kvs, n_pages, bt, bt_ld, n_req, n_rows_padded, n_units, sched, sched + 1, row_len,
                     logits, ld);
}

}  // namespace ifp4

using namespace ifp4;

extern "C" int indexer_fp4_score_prefill(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                                         int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                                         int64_t n_pages, const int32_t *block_table, int64_t bt_ld, int32_t n_req,
                                         void *sched, int32_t n_units, int32_t n_rows_padded,
                                         const int32_t *row_len, float *logits, int64_t logits_ld, void *stream) {
  clear_error();
  if (n_heads <= 0 || n_heads % INDEXER_FP4_HEAD_MULT != 0 || n_heads > INDEXER_FP4_MAX_HEADS)
    return fail(INDEXER_FP4_EINVAL, "n_heads=%d must be a positive multiple of %d and at most %d", n_heads,
                INDEXER_FP4_HEAD_MULT, INDEXER_FP4_MAX_HEADS);
  if (n_req <= 0 || n_units <= 0 || n_pages < 0 || n_rows_padded <= 0 || n_rows_padded % kTileRows != 0)
    return fail(INDEXER_FP4_EINVAL,
                "score_prefill: n_req=%d > 0, n_units=%d > 0, n_pages=%lld >= 0, n_rows_padded=%d a positive multiple of %d",
                n_req, n_units, (long long)n_pages, n_rows_padded, kTileRows);
  if (bt_ld <= 0) return fail(INDEXER_FP4_ENOSPC, "score_prefill: bt_ld=%lld must be positive", (long long)bt_ld);
  if (logits_ld < bt_ld * kPage)
    return fail(INDEXER_FP4_ENOSPC, "score_prefill: logits_ld=%lld < 64*bt_ld=%lld", (long long)logits_ld,
                (long long)(bt_ld * kPage));
  if (!sched || !row_len || !q_packed || !q_scale || !weights || !block_table || !logits)
    return fail(INDEXER_FP4_EINVAL, "score_prefill: a required pointer is NULL");
  if (n_pages > 0 && (!kv_packed || !kv_scale)) return fail(INDEXER_FP4_EINVAL, "score_prefill: NULL cache plane");
  if (((uintptr_t)q_packed | (uintptr_t)weights | (uintptr_t)kv_packed | (uintptr_t)kv_scale) % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "score_prefill: q_packed, weights and both planes must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t *sc = (int32_t *)sched;
  switch (n_heads / 16) {
#define IFP4_CASE(X) \
  case X: launch_prefill<X>(st, n_units, q_packed, q_scale, weights, n_heads, kv_packed, kv_scale, n_pages, block_table, bt_ld, n_req, n_rows_padded, sc, row_len, logits, logits_ld); break;
    IFP4_CASE(1) IFP4_CASE(2) IFP4_CASE(3) IFP4_CASE(4) IFP4_CASE(5) IFP4_CASE(6) IFP4_CASE(7) IFP4_CASE(8)
#undef IFP4_CASE
  }
  return launch_status("score_prefill");
}
