// Prefill scorer: row groups of a prefill step against the paged FP4 key cache.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), commit message: the FP4 prefill
// variant scores the chunk's query rows straight out of the paged cache; ROCm/ATOM #2125
// section 3: the row-group kernel finds a group's page table as group b -> block_tables[b],
// and padding rows, folded into the last request's group, read no key. Each valid row r
// at position p sees keys [0, p] (causal, inclusive).
//
// Design for gfx950. Work items are (tile, page) pairs where a tile is up to 8 rows of one
// request's group (schedule.hip). A unit (workgroup of 8 waves) takes a contiguous range of
// items; all its waves walk the same items and wave w scores row w of the tile, so one key
// page feeds 8 rows x n_heads query heads of MFMA work. Pages go through a ring of P slots
// in LDS filled by direct global-to-LDS loads (no registers held while in flight, so the
// ring can be deep): four waves each copy one 1 KiB key tile, a fifth the 256-byte scale
// block, with lane i fetching exactly the 16 bytes that lane i of every wave later reads as
// its MFMA operand (same layout as the decode scorer's direct loads), so the LDS reads are
// linear. Items go in groups of B: per group the loader waves wait until their copies have
// landed (vmcnt counting in issue order), the unit meets at one barrier, the slots of the
// previous group are refilled P-B items ahead, and every wave scores its row for the whole
// group from LDS without further synchronisation. Each wave keeps a table of 64 items at a
// time (tile, page, physical page, whether its row reaches the page), built with one round
// of per-lane loads. Logits past a row's length fall outside the store's range.
//
// Each wave keeps its row's query operands in LDS, in operand order, and refills its
// registers from there at every group (per item in the rare group that crosses into a new
// tile, which first stages the new row from global memory). Holding them in registers
// across groups would put a join after every conditional reload, and the compiler resolves
// such joins with dozens of register copies per item, a third of the VALU work. The first
// tile's row is fetched at entry, while the item table is being built.
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

// One LDS array per ring slot: with every slot access indexed by a constant the compiler
// can tell the slots apart and adds no waits of its own between a slot's reads and the
// loads in flight into other slots.
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

template <int NH16, int NW, int P, int B>
__global__ __launch_bounds__(NW * 64) void score_prefill_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages,
    const int32_t *__restrict__ bt_g, int64_t bt_ld, int n_req, int n_rows_padded, int n_units,
    const int32_t *__restrict__ sched_g, int32_t *__restrict__ err, const int32_t *__restrict__ row_len_g,
    float *__restrict__ logits, int64_t ld) {
  static_assert(P <= kPrefillMaxRing && B >= 1 && P % B == 0 && P / B >= 2 && NW >= 5, "ring, groups, loaders");
  const PrefillSchedLayout L(n_req, n_rows_padded, n_units);
  const const_ptr<int32_t> sched = as_const(sched_g), row_len = as_const(row_len_g);
  const int u = blockIdx.x;
  // The unit table is in bounds (the host checked the buffer's size for these sizes); its
  // words are used only once the header shows a schedule built for this step's sizes (a
  // stale or zeroed buffer is flagged once, by unit 0, and nothing is scored).
  const int it0r = sched[L.unit_begin + u];
  const int it1r = sched[L.unit_begin + u + 1];
  if (sched[0] != kPrefillMagic || sched[2] != n_req || sched[3] != n_rows_padded || sched[4] != n_units) {
    if (u == 0 && threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
    return;
  }
  const int it0 = max(it0r, 0), it1 = min(it1r, sched[6]);
  if (it0 >= it1) return;  // empty unit (uniform over the workgroup): nothing else is touched
  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);  // this wave's row inside a tile
  if (n_pages <= 0) {  // the ring always copies some page: there must be one
    if (threadIdx.x == 0) atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
    return;
  }
  const int n_tiles = min(sched[5], (int)L.max_tiles);
  const int32_t *tiles = sched_g + L.tiles;  // {first row, rows, request, pages} per tile
  const int32_t *cum = sched_g + L.cum;
  const int n_my = it1 - it0;
  const bool loader = wv < 5;  // waves 0-3 copy key tiles, wave 4 the scale block

  // Item table, one lane per item, for 64 items at a time.
  int tcur = min(max(sched[L.unit_tile + u], 0), max(n_tiles - 1, 0));  // tile of the next item to look up
  int tab_base = -64;
  int v_tile = 0, v_page = 0, v_phys = 0, v_need = 0;
  auto fill = [&](int base) {
    tab_base = base;
    const int it = it0 + base + lane;
    int t = tcur, p = 0, phys = 0, need = 0;
    if (it < it1) {
      while (t < n_tiles - 1 && it >= cum[t + 1]) t++;
      p = it - cum[t];
      const int4 T = *reinterpret_cast<const int4 *>(tiles + 4 * t);
      need = wv < T.y && row_len[T.x + wv] > p * kPage;
      if (p < 0) {
        atomicOr(err, INDEXER_FP4_DEV_BAD_SCHEDULE);
        need = 0;
      } else if (p >= bt_ld) {
        if (need) atomicOr(err, INDEXER_FP4_DEV_TABLE_SHORT);
        need = 0;
      } else {
        phys = bt_g[(int64_t)T.z * bt_ld + p];
        if (phys < 0 || phys >= n_pages) {
          if (need) atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
          phys = 0;  // a page that exists; nobody scores it
          need = 0;
        }
      }
    }
    v_tile = t;
    v_page = p;
    v_phys = phys;
    v_need = need;
    tcur = __builtin_amdgcn_readlane(t, 63);  // tiles only advance with the items
  };

  int st[P], sp[P];
  bool sok[P];
  // copy item i (clamped to the unit's last item) into ring slot S, and note what scoring it
  // needs; every wave records the item, the loader waves issue one direct load each
  auto issue = [&](auto ss, int i) {
    constexpr int S = decltype(ss)::value;
    const bool live = i < n_my;
    const int ii = live ? i : n_my - 1;
    if (ii - tab_base >= 64) fill(ii & ~63);
    const int l = ii - tab_base;
    const int phys = __builtin_amdgcn_readlane(v_phys, l);
    st[S] = __builtin_amdgcn_readlane(v_tile, l);
    sp[S] = __builtin_amdgcn_readlane(v_page, l);
    sok[S] = live && __builtin_amdgcn_readlane(v_need, l) != 0;
    if (wv < 4) {
      const uint8_t *src = kvp + (int64_t)phys * kPageBytes + 1024 * wv + 64 * (lane & 15) + 16 * (lane >> 4);
      __builtin_amdgcn_global_load_lds(src, (lds_void *)(slot_keys<S>() + 64 * wv), 16, 0, 0);
    } else if (wv == 4) {
      const uint8_t *src = kvs + (int64_t)phys * kPageScaleBytes + 4 * lane;
      __builtin_amdgcn_global_load_lds(src, (lds_void *)slot_scales<S>(), 4, 0, 0);
    }
  };
  // a store that writes nothing (empty range): keeps every wave at one store per item
  auto idle_store = [&]() { buffer_store_f32(0.f, buffer_view(logits, 0u), 0u); };

  // This wave's query row in LDS: operands per M-tile and lane, weights per M-tile and lane
  // group (16 lanes read one address), scale words per lane. The helpers below are called
  // from every unrolled item and are forced inline: out of line, the row would be passed
  // through private (scratch) memory.
  constexpr int NQS = (NH16 + 3) / 4;
  // (native vector element types: copies of the HIP vector structs become memcpys that keep
  // the row in private memory; and every access indexes the arrays themselves, so the
  // compiler can tell them apart from the ring slots the direct loads write and adds no
  // wait for those loads before reading the row)
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ u32x4 q_lds[NW * NH16 * 64];
  __shared__ f32x4 w_lds[NW * NH16 * 4];
  __shared__ uint32_t qs_lds[NW * NQS * 64];
  const int qa0 = wv * NH16 * 64, w0i = wv * NH16 * 4, qs0i = wv * NQS * 64;
  auto stage_row = [&](const RowRegs<NH16, 1> &Q) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NH16; m++) {
      const uint4 a = Q.qa[0][m];
      q_lds[qa0 + m * 64 + lane] = u32x4{a.x, a.y, a.z, a.w};
      // all 16 lanes of a group store the same four weights to the same address (a
      // conditional store here would also keep the row in private memory)
      const float4 x = Q.w[0][m];
      w_lds[w0i + m * 4 + (lane >> 4)] = f32x4{x.x, x.y, x.z, x.w};
    }
#pragma unroll
    for (int j = 0; j < NQS; j++) qs_lds[qs0i + j * 64 + lane] = Q.qs[0][j];
  };
  auto read_row = [&](RowRegs<NH16, 1> &Q) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NH16; m++) {
      const u32x4 a = q_lds[qa0 + m * 64 + lane];
      Q.qa[0][m] = make_uint4(a.x, a.y, a.z, a.w);
      const f32x4 x = w_lds[w0i + m * 4 + (lane >> 4)];
      Q.w[0][m] = make_float4(x.x, x.y, x.z, x.w);
    }
#pragma unroll
    for (int j = 0; j < NQS; j++) Q.qs[0][j] = qs_lds[qs0i + j * 64 + lane];
  };
  // The first tile's row is requested before the item table is built and staged after the
  // prologue's copies are issued, so its loads overlap the table's and the first pages'.
  int qt = tcur, row = 0, row_bytes = 0;
  RowRegs<NH16, 1> Q0;
  const bool first_row = wv < tiles[4 * qt + 1];
  if (first_row) {
    row = tiles[4 * qt] + wv;
    row_bytes = 4 * max(row_len[row], 0);
    load_rows<NH16, 1, false>(Q0, qp, qs, w, row, 1, n_heads, lane);
  }
  // a new tile for this wave: stage its row (waits for everything in flight; once per tile)
  auto enter_tile = [&](int t) __attribute__((always_inline)) {
    qt = t;
    const int4 T = *reinterpret_cast<const int4 *>(tiles + 4 * qt);
    row = T.x + wv;  // only called for items this wave scores, so wv < T.y
    row_bytes = 4 * max(row_len[row], 0);
    RowRegs<NH16, 1> Q;
    load_rows<NH16, 1>(Q, qp, qs, w, row, 1, n_heads, lane);
    stage_row(Q);
  };
  auto score = [&](auto ss, const RowRegs<NH16, 1> &R) __attribute__((always_inline)) {
    constexpr int S = decltype(ss)::value;
    if (!sok[S]) {
      idle_store();
      return;
    }
    PageRegs pg;
#pragma unroll
    for (int t = 0; t < 4; t++) pg.k[t] = slot_keys<S>()[64 * t + lane];
    pg.s = slot_scales<S>()[lane];
    const uint32_t col = (uint32_t)(sp[S] * kPage + lane);
    const float v = page_logit<NH16, 1, 0>(pg, R, lane);
    buffer_store_f32(v, buffer_view(logits + (int64_t)row * ld, (uint32_t)row_bytes), 4u * col);
  };
  // score the B items of group GG with the current tile's row R (read from LDS before the
  // group's refills are issued: the compiler cannot tell the row from the ring slots being
  // filled and waits for every load in flight before reading it), or, in a group that enters
  // a new tile, per item after staging each new tile
  auto score_group = [&](auto gg, const RowRegs<NH16, 1> &R) __attribute__((always_inline)) {
    constexpr int GG = decltype(gg)::value;
    bool same = true;
    static_for<B>([&](auto bb) {
      constexpr int S = GG * B + decltype(bb)::value;
      same = same && (!sok[S] || st[S] == qt);
    });
    if (same) {
      static_for<B>([&](auto bb) { score(std::integral_constant<int, GG * B + decltype(bb)::value>{}, R); });
    } else {
      static_for<B>([&](auto bb) {
        constexpr int S = GG * B + decltype(bb)::value;
        if (sok[S] && st[S] != qt) enter_tile(st[S]);
        RowRegs<NH16, 1> R;
        read_row(R);
        score(std::integral_constant<int, S>{}, R);
      });
    }
  };

  // Items go in groups of B; the ring holds G = P / B groups. At the start of group k the
  // loader waves wait until the group's copies have landed, the unit meets once, the slots
  // of group k-1 are refilled with group k+G-1, and every wave scores its row for the B
  // items of group k without further synchronisation.
  constexpr int G = P / B;
  // Prologue: groups 0 .. G-2, each followed by B idle stores so that a loader wave issues
  // the same sequence (B loads, then B stores) before every group.
  static_for<G - 1>([&](auto gg) {
    constexpr int GG = decltype(gg)::value;
    static_for<B>([&](auto bb) { issue(std::integral_constant<int, GG * B + decltype(bb)::value>{}, GG * B + decltype(bb)::value); });
    if (loader) static_for<B>([&](auto) { idle_store(); });
  });
  if (first_row) stage_row(Q0);
  for (int i0 = 0; i0 < n_my; i0 += P) {
    static_for<G>([&](auto gg) {
      constexpr int GG = decltype(gg)::value;
      // After the last load of this group a loader wave issued the stores of the G-1 groups
      // before it and the loads of the G-2 groups after it, B each, and memory operations
      // complete in issue order: at most B(2G-3) outstanding means the group is in LDS.
      if (loader) __builtin_amdgcn_s_waitcnt(0x0F70 | (B * (2 * G - 3)));
      __builtin_amdgcn_s_barrier();  // the group landed; the previous group's slots are free
      asm volatile("" ::: "memory");
      RowRegs<NH16, 1> R;
      read_row(R);
      constexpr int GR = (GG + G - 1) % G;  // slots of the previous group
      static_for<B>([&](auto bb) {
        constexpr int BB = decltype(bb)::value;
        issue(std::integral_constant<int, GR * B + BB>{}, i0 + (GG + G - 1) * B + BB);
      });
      score_group(gg, R);
    });
  }
}

template <int NH16>
static void launch_prefill(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                           int n_heads, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages, const int32_t *bt,
                           int64_t bt_ld, int n_req, int n_rows_padded, int32_t *sched, const int32_t *row_len,
                           float *logits, int64_t ld) {
  constexpr int NW = kTileRows, P = IFP4_PREFILL_RING, B = IFP4_PREFILL_GROUP;
  hipLaunchKernelGGL((score_prefill_kernel<NH16, NW, P, B>), dim3(n_units), dim3(NW * 64), 0, st, qp, qs, w,
                     n_heads, kvp, kvs, n_pages, bt, bt_ld, n_req, n_rows_padded, n_units, sched, sched + 1, row_len,
                     logits, ld);
}

}  // namespace ifp4

using namespace ifp4;

extern "C" int indexer_fp4_score_prefill(const uint8_t *q_packed, const uint8_t *q_scale, const float *weights,
                                         int32_t n_heads, const uint8_t *kv_packed, const uint8_t *kv_scale,
                                         int64_t n_pages, const int32_t *block_table, int64_t bt_ld, int32_t n_req,
                                         void *sched, int64_t sched_bytes, int32_t n_units, int32_t n_rows_padded,
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
  const int64_t need = 4 * PrefillSchedLayout(n_req, n_rows_padded, n_units).words;
  if (sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "score_prefill: sched_bytes=%lld < %lld for n_req=%d, n_rows_padded=%d, n_units=%d",
                (long long)sched_bytes, (long long)need, n_req, n_rows_padded, n_units);
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

