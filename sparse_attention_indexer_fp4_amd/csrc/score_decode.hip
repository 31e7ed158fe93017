// Decode scorer: FP4 query rows against the paged FP4 key cache on a persistent grid.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216): the FP4 mqa-logits kernel scores
// straight out of the paged cache (commit message, PR description intro), driven by the
// CTA schedule published once a step (Decode grid floor); per key the index score is
// sum_h w[h] * ReLU(q_h . k) (the DSA indexer score the pages name as mqa logits with
// per-head weights).
//
// Design for gfx950. The work items are (sequence, page) pairs; unit u of the grid owns a
// contiguous range of them (see schedule.hip) and each of its waves a contiguous share. A wave
// scores one whole 64-key page for all heads of all next_n rows of that sequence:
//   - the page is read once, straight into MFMA operand registers: for the 16-key tile t
//     lane l loads the 16 bytes of key 16t + l%16 that hold elements [32(l/16), +32), so
//     each load instruction reads 1 KiB of contiguous keys, and lane l reads the scale
//     dword at byte 4l of the page's 256-byte scale plane, whose byte t is exactly that
//     key's e8m0 scale for group l/16 (the 16x4 transposed scale plane);
//   - 16 x (n_heads/16) block-scaled 16x16x128 FP4 MFMAs give all head x key dot products
//     (heads are the M axis, keys the N axis);
//   - ReLU and the head weights are applied in registers, partial head sums are
//     exchanged across the four 16-lane groups, and lane l ends with the logit of key l
//     of the page: one 256-byte store per row.
// Each wave keeps D pages in flight in a register ring. A unit with no work exits before
// any other load (empty CTAs of a large grid must cost nothing: the pages measured 8.75
// against 2.99 us per layer at 4096 against 512 units).
//
// With a row histogram the scorer also counts every logit it writes by its top 12 order-key
// bits, the first digit of the top-k's selection, so the top-k does not read the logits an
// extra time: rows of the unit's first sequence (nearly all its items) are counted in LDS and
// added to the device histogram at the end, the rare pages of later sequences straight into
// device memory.
#include "score_common.h"

// waves per unit and pages in flight per wave (tuned on MI355X at 8 x 131072, 64 heads)
#ifndef IFP4_DECODE_WAVES
#define IFP4_DECODE_WAVES 4
#endif
#ifndef IFP4_DECODE_RING
#define IFP4_DECODE_RING 2
#endif

namespace ifp4 {

// A device histogram addressed by bin (hist_slot places the bins).
struct SlottedHist {
  uint32_t *g;
  __device__ __forceinline__ uint32_t &operator[](uint32_t b) const { return g[hist_slot(b)]; }
};

template <class F, int NH16, int NN, int NW, int D>
__global__ __launch_bounds__(NW * 64) void score_decode_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages,
    const int32_t *__restrict__ bt_g, int64_t bt_ld, int batch, int n_units, const int32_t *__restrict__ sched_g,
    int32_t *__restrict__ err, const int32_t *__restrict__ row_len_g, float *__restrict__ logits, int64_t ld,
    uint32_t *__restrict__ row_hist) {
  extern __shared__ uint32_t uh[];  // [NN][kHistBins] with a row histogram
  const DecodeSchedLayout L(batch, n_units);
  const const_ptr<int32_t> sched = as_const(sched_g), row_len = as_const(row_len_g);
  const int u = blockIdx.x;
  // The host checked that the buffer holds a schedule of these sizes, so the unit table is
  // in bounds whatever it contains; its words are only used once the header shows that the
  // schedule was built for this batch, next_n and unit count (a stale or zeroed buffer is
  // flagged once, by unit 0, and nothing is scored).
  const int it0r = sched[L.unit_begin + u];
  const int it1r = sched[L.unit_begin + u + 1];
  if (sched[0] != kDecodeMagic || sched[2] != batch || sched[3] != NN || sched[4] != n_units) {
    if (u == 0 && threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
    return;
  }
  const int items = sched[5];
  const int it0 = max(it0r, 0), it1 = min(it1r, items);
  if (it0 >= it1) return;  // empty unit: nothing else is touched
  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);
  if (n_pages <= 0) {
    if (threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
    return;
  }
  const bool fuse = row_hist != nullptr;
  const int qs0 = sched[L.unit_seq + u];  // the unit's first sequence: histogram in LDS
  if (qs0 < 0 || qs0 >= batch) {
    if (threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
    return;
  }
  if (fuse) {
    for (int i = threadIdx.x; i < NN * kHistBins / 4; i += NW * 64)
      reinterpret_cast<uint4 *>(uh)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
  }
  // this wave's contiguous share of the unit's items (none for some waves of a short unit,
  // which still meet the workgroup's barriers)
  const int per = (it1 - it0 + NW - 1) / NW;
  const int w0 = it0 + wv * per;
  const int w1 = min(it1, w0 + per);
  const int n_my = max(0, w1 - w0);
  const int32_t *cum = sched_g + L.cum;

  // Item table, one lane per item, for 64 items at a time: sequence, page index within
  // it, and physical page (-1 if the page cannot be read). Built with one round of
  // per-lane loads instead of a chain of dependent scalar loads per page.
  int seq0 = sched[L.unit_seq + u];  // sequence of the unit's first item
  const int page0 = sched[L.unit_page + u];
  const int run0 = sched[L.unit_run + u];
  int tab_base = -64;
  int v_seq = 0, v_page = 0, v_phys = -1;
  auto fill = [&](int base) {
    tab_base = base;
    const int it = w0 + base + lane;
    int b = seq0, p = 0, phys = -1;
    if (it < w1) {
      const int k = it - it0;  // items past the unit's first one
      if (k < run0) {          // still in the unit's first sequence: no lookup
        b = sched[L.unit_seq + u];
        p = page0 + k;
      } else {
        while (b < batch - 1 && it >= cum[b + 1]) b++;
        p = it - cum[b];
      }
      if (p >= 0 && p < bt_ld) {
        phys = bt_g[(int64_t)b * bt_ld + p];
        if (phys < 0 || phys >= n_pages) {
          atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
          phys = -1;
        }
      } else {
        atomicOr(err, p < 0 ? INDEXER_FP4_DEV_BAD_SCHEDULE : INDEXER_FP4_DEV_TABLE_SHORT);
      }
    }
    v_seq = b;
    v_page = p;
    v_phys = phys;
    seq0 = __builtin_amdgcn_readlane(b, 63);  // sequences only advance with the items
  };

  // Software pipeline over a ring of D pages: scoring slot K overlaps the loads of the
  // other D-1 slots. Every slot refill is unconditional -- past the wave's last item it
  // reloads that item (a cache hit) and its logits are dropped -- so the compiler waits
  // only for the slot being scored.
  typename F::Page P[D];
  int sb[D], sp[D];
  bool sok[D];
  auto issue = [&](auto kk, int i) {
    constexpr int K = decltype(kk)::value;
    const bool live = i < n_my;
    const int ii = live ? i : n_my - 1;
    if (ii - tab_base >= 64) fill(ii & ~63);
    const int l = ii - tab_base;
    const int phys = __builtin_amdgcn_readlane(v_phys, l);
    sb[K] = __builtin_amdgcn_readlane(v_seq, l);
    sp[K] = __builtin_amdgcn_readlane(v_page, l);
    sok[K] = live && phys >= 0;
    F::page(P[K], kvp, kvs, phys >= 0 ? phys : 0, lane);
  };
  typename F::template Rows<NH16, NN> R;
  int qb = -1;
  auto score = [&](auto kk) {
    constexpr int K = decltype(kk)::value;
    if (sb[K] != qb) {  // a new sequence: its query rows (waits for everything in flight)
      qb = sb[K];
      F::template rows<NH16, NN>(R, qp, qs, w, (int64_t)qb * NN, NN, n_heads, lane);
    }
    const uint32_t col = (uint32_t)(sp[K] * kPage + lane);
    static_for<NN>([&](auto nn) {
      constexpr int N = decltype(nn)::value;
      const int64_t r = (int64_t)qb * NN + N;
      const int len = row_len[r];
      // logits past the row's length (or of a dropped slot) fall outside the view
      const uint32_t bytes = sok[K] ? 4u * (uint32_t)max(len, 0) : 0u;
      const float v = F::template logit<NH16, NN, N>(P[K], R, lane);
      buffer_store_f32(v, buffer_view(logits + r * ld, bytes), 4u * col);
      if (fuse) {  // exactly the logits stored above
        const bool kept = 4u * col < bytes;
        const uint32_t d = order_key(v) >> 20;
        if (qb == qs0) hist_put(uh + N * kHistBins, d, kept);
        else hist_put(SlottedHist{row_hist + r * kHistBins}, d, kept);
      }
    });
  };

  if (n_my > 0) {
    // the first pages are in flight before the query rows are fetched
    static_for<D>([&](auto kk) { issue(kk, decltype(kk)::value); });
    for (int i0 = 0; i0 < n_my; i0 += D) {
      static_for<D>([&](auto kk) {
        score(kk);
        issue(kk, i0 + decltype(kk)::value + D);
      });
    }
  }
  if (fuse) {  // occupied bins only, one device atomic each
    __syncthreads();
    uint32_t *g = row_hist + (int64_t)qs0 * NN * kHistBins;
    for (int i = threadIdx.x; i < NN * kHistBins; i += NW * 64) {
      const uint32_t c = uh[i];
      if (c) atomicAdd(&g[(i / kHistBins) * kHistBins + hist_slot(i % kHistBins)], c);
    }
  }
}

template <class F, int NH16, int NN>
static int launch_decode(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                          int n_heads, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages, const int32_t *bt,
                          int64_t bt_ld, int batch, int32_t *sched, const int32_t *row_len, float *logits,
                          int64_t ld, uint32_t *row_hist) {
  constexpr int NW = IFP4_DECODE_WAVES, D = IFP4_DECODE_RING;
  constexpr size_t kHistLds = (size_t)NN * kHistBins * 4;
  static bool lds_set = false;  // raise the dynamic LDS limit once per instantiation
  if (row_hist && !lds_set) {
    const hipError_t e = hipFuncSetAttribute((const void *)score_decode_kernel<F, NH16, NN, NW, D>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHistLds);
    if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "score_decode: hipFuncSetAttribute: %s", hipGetErrorString(e));
    lds_set = true;
  }
  hipLaunchKernelGGL((score_decode_kernel<F, NH16, NN, NW, D>), dim3(n_units), dim3(NW * 64), row_hist ? kHistLds : 0,
                     st, qp, qs, w, n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, n_units, sched, sched + 1, row_len,
                     logits, ld, row_hist);
  return INDEXER_FP4_OK;
}

template <class F, int NH16>
static int launch_decode_nn(int next_n, hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs,
                            const float *w, int n_heads, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages,
                            const int32_t *bt, int64_t bt_ld, int batch, int32_t *sched, const int32_t *row_len,
                            float *logits, int64_t ld, uint32_t *row_hist) {
  switch (next_n) {
    case 1: return launch_decode<F, NH16, 1>(st, n_units, qp, qs, w, n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, sched, row_len, logits, ld, row_hist);
    case 2: return launch_decode<F, NH16, 2>(st, n_units, qp, qs, w, n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, sched, row_len, logits, ld, row_hist);
    case 3: return launch_decode<F, NH16, 3>(st, n_units, qp, qs, w, n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, sched, row_len, logits, ld, row_hist);
    default: return launch_decode<F, NH16, 4>(st, n_units, qp, qs, w, n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, sched, row_len, logits, ld, row_hist);
  }
}

}  // namespace ifp4

using namespace ifp4;

template <class F>
static int score_decode(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights, int32_t n_heads,
                        const uint8_t *kv_packed, const uint8_t *kv_scale, int64_t n_pages,
                        const int32_t *block_table, int64_t bt_ld, int32_t batch, int32_t next_n, void *sched,
                        int64_t sched_bytes, int32_t n_units, const int32_t *row_len, float *logits,
                        int64_t logits_ld, uint32_t *row_hist, void *stream) {
  clear_error();
  if (n_heads <= 0 || n_heads % INDEXER_FP4_HEAD_MULT != 0 || n_heads > INDEXER_FP4_MAX_HEADS)
    return fail(INDEXER_FP4_EINVAL, "n_heads=%d must be a positive multiple of %d and at most %d", n_heads,
                INDEXER_FP4_HEAD_MULT, INDEXER_FP4_MAX_HEADS);
  if (batch < 0 || next_n < 1 || next_n > 4 || n_units <= 0 || n_pages < 0)
    return fail(INDEXER_FP4_EINVAL, "score_decode: batch=%d >= 0, next_n=%d in 1..4, n_units=%d > 0, n_pages=%lld >= 0",
                batch, next_n, n_units, (long long)n_pages);
  if (bt_ld <= 0) return fail(INDEXER_FP4_ENOSPC, "score_decode: bt_ld=%lld must be positive", (long long)bt_ld);
  if (logits_ld < bt_ld * kPage)
    return fail(INDEXER_FP4_ENOSPC, "score_decode: logits_ld=%lld < 64*bt_ld=%lld", (long long)logits_ld,
                (long long)(bt_ld * kPage));
  if (!sched || !row_len || (batch > 0 && (!q_packed || !q_scale || !weights || !block_table || !logits)))
    return fail(INDEXER_FP4_EINVAL, "score_decode: a required pointer is NULL");
  const int64_t need = 4 * DecodeSchedLayout(batch, n_units).words;
  if (sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "score_decode: sched_bytes=%lld < %lld for batch=%d, n_units=%d",
                (long long)sched_bytes, (long long)need, batch, n_units);
  if (n_pages > 0 && (!kv_packed || !kv_scale)) return fail(INDEXER_FP4_EINVAL, "score_decode: NULL cache plane");
  if (((uintptr_t)q_packed | (uintptr_t)weights | (uintptr_t)kv_packed | (uintptr_t)kv_scale) % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "score_decode: q_packed, weights and both planes must be 16-byte aligned");
  if ((uintptr_t)row_hist % 16 != 0) return fail(INDEXER_FP4_EINVAL, "score_decode: row_hist must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  if (batch == 0) return INDEXER_FP4_OK;
  hipStream_t st = (hipStream_t)stream;
  int32_t *sc = (int32_t *)sched;
  switch (n_heads / 16) {
#define IFP4_CASE(X) \
  case X: rc = launch_decode_nn<F, X>(next_n, st, n_units, q_packed, q_scale, weights, n_heads, kv_packed, kv_scale, n_pages, block_table, bt_ld, batch, sc, row_len, logits, logits_ld, row_hist); break;
    IFP4_CASE(1) IFP4_CASE(2) IFP4_CASE(3) IFP4_CASE(4) IFP4_CASE(5) IFP4_CASE(6) IFP4_CASE(7) IFP4_CASE(8)
#undef IFP4_CASE
  }
  return rc ? rc : launch_status("score_decode");
}

extern "C" int indexer_fp4_score_decode(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                                        int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                                        int64_t n_pages, const int32_t *block_table, int64_t bt_ld, int32_t batch,
                                        int32_t next_n, void *sched, int64_t sched_bytes, int32_t n_units,
                                        const int32_t *row_len, float *logits, int64_t logits_ld,
                                        uint32_t *row_hist, void *stream) {
  return score_decode<FmtFp4>(q_packed, q_scale, weights, n_heads, kv_packed, kv_scale, n_pages, block_table, bt_ld,
                              batch, next_n, sched, sched_bytes, n_units, row_len, logits, logits_ld, row_hist, stream);
}

// The FP8 comparator: the same scorer over MXFP8 queries and keys (128 bytes a vector).
extern "C" int indexer_fp8_score_decode(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                                        int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                                        int64_t n_pages, const int32_t *block_table, int64_t bt_ld, int32_t batch,
                                        int32_t next_n, void *sched, int64_t sched_bytes, int32_t n_units,
                                        const int32_t *row_len, float *logits, int64_t logits_ld,
                                        uint32_t *row_hist, void *stream) {
  return score_decode<FmtFp8>(q_packed, q_scale, weights, n_heads, kv_packed, kv_scale, n_pages, block_table, bt_ld,
                              batch, next_n, sched, sched_bytes, n_units, row_len, logits, logits_ld, row_hist, stream);
}
