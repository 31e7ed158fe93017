// Per-step work schedules for the persistent scorers.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), PR description, Decode grid
// floor: the scorer runs a persistent grid whose CTA schedule is built once a step at a
// graph-stable address (floor 512 units for decode, 4096 for prefill); review fixes: a
// schedule must never under-cover its rows silently. ROCm/ATOM #2125, section 3:
// padding rows fold into the last request's row group and read no key.
//
// Each schedule is built by one 1024-thread workgroup: block-wide prefix sums over the
// per-sequence (decode) or per-tile (prefill) page counts, then an even contiguous split
// of the resulting work items over the units. Both are O(batch + units) integer work.
#include "common.h"

namespace ifp4 {

constexpr int kSchedThreads = 1024;

// Inclusive block scan of one int per thread; *total receives the block sum.
__device__ int block_inclusive_scan(int v, int *lds, int *total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int nw = kSchedThreads / 64;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) lds[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? lds[lane] : 0;
#pragma unroll
    for (int o = 1; o < nw; o <<= 1) {
      const int s = __shfl_up(t, o, 64);
      if (lane >= o) t += s;
    }
    if (lane < nw) lds[lane] = t;
  }
  __syncthreads();
  if (w > 0) v += lds[w - 1];
  *total = lds[nw - 1];
  __syncthreads();
  return v;
}

// number of entries of the non-decreasing a[0..n) that are <= x
__device__ __forceinline__ int count_le(const int32_t *a, int n, int64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(const int32_t *__restrict__ ctx, int batch,
                                                                        int next_n, int n_units, int32_t *sched,
                                                                        int32_t *__restrict__ row_len) {
  __shared__ int lds[kSchedThreads / 64];
  __shared__ int bad;
  const DecodeSchedLayout L(batch, n_units);
  int32_t *cum = sched + L.cum;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < batch; base += kSchedThreads) {
    const int b = base + threadIdx.x;
    int pages = 0;
    if (b < batch) {
      int c = ctx[b];
      if (c < 0) {
        bad = 1;
        c = 0;
      }
      pages = (c + kPage - 1) / kPage;
      for (int t = 0; t < next_n; t++) {
        const int len = c - next_n + 1 + t;
        row_len[(int64_t)b * next_n + t] = len > 0 ? len : 0;
      }
    }
    int total;
    const int incl = block_inclusive_scan(pages, lds, &total);
    if (b < batch) cum[b + 1] = carry + incl;
    carry += total;
  }
  const int items = carry;
  if (threadIdx.x == 0) {
    cum[0] = 0;
    sched[0] = kDecodeMagic;
    sched[1] = bad ? INDEXER_FP4_DEV_BAD_LENGTH : 0;
    sched[2] = batch;
    sched[3] = next_n;
    sched[4] = n_units;
    sched[5] = items;
    sched[6] = 0;
    sched[7] = 0;
  }
  __syncthreads();
  for (int u = threadIdx.x; u <= n_units; u += kSchedThreads) {
    const int64_t ib = (int64_t)u * items / n_units;
    sched[L.unit_begin + u] = (int32_t)ib;
    if (u < n_units) {
      const int b = count_le(cum + 1, batch, ib);
      sched[L.unit_seq + u] = b;
      sched[L.unit_page + u] = b < batch ? (int32_t)ib - cum[b] : 0;
      sched[L.unit_run + u] = b < batch ? cum[b + 1] - (int32_t)ib : 0;
    }
  }
}

__global__ __launch_bounds__(kSchedThreads) void prefill_schedule_kernel(
    const int32_t *__restrict__ cu_rows, const int32_t *__restrict__ start_pos, int n_req, int n_rows_padded,
    int n_units, const int32_t *__restrict__ bt, int64_t bt_ld, int64_t n_pages, int32_t *sched,
    int32_t *__restrict__ row_len) {
  __shared__ int lds[kSchedThreads / 64];
  __shared__ int s_flags;
  const PrefillSchedLayout L(n_req, n_rows_padded, n_units, bt_ld);
  int32_t *tiles = sched + L.tiles;
  int32_t *cum = sched + L.cum;
  int32_t *req_tile = sched + L.req_tile;
  int32_t *item_phys = sched + L.item_phys;
  constexpr int TR = kPrefillTileRows;
  auto header = [&](int err, int n_tiles, int items) {
    sched[0] = kPrefillMagic;
    sched[1] = err;
    sched[2] = n_req;
    sched[3] = n_rows_padded;
    sched[4] = n_units;
    sched[5] = n_tiles;
    sched[6] = items;
    sched[7] = TR;
    sched[8] = (int32_t)bt_ld;
    sched[9] = (int32_t)min(n_pages, (int64_t)INT32_MAX);
    for (int i = 10; i < kPrefillHdrWords; i++) sched[i] = 0;
  };
  if (threadIdx.x == 0) s_flags = 0;
  // validate: cu_rows starts at 0, ascends, ends within the padded rows; positions >= 0
  int bad_local = 0;
  for (int i = threadIdx.x; i < n_req; i += kSchedThreads) {
    if (cu_rows[i + 1] < cu_rows[i] || start_pos[i] < 0) bad_local = 1;
  }
  if (threadIdx.x == 0 && (cu_rows[0] != 0 || cu_rows[n_req] > n_rows_padded)) bad_local = 1;
  const int bad = __syncthreads_or(bad_local);
  if (bad) {  // an empty schedule: no unit has work, every row has length 0
    for (int r = threadIdx.x; r < n_rows_padded; r += kSchedThreads) row_len[r] = 0;
    for (int u = threadIdx.x; u <= n_units; u += kSchedThreads) {
      sched[L.unit_begin + u] = 0;
      if (u < n_units) {
        sched[L.unit_tile + u] = 0;
        for (int j = 0; j < kUnitRecWords; j++) sched[L.urec + (int64_t)kUnitRecWords * u + j] = 0;
      }
    }
    if (threadIdx.x == 0) {
      header(INDEXER_FP4_DEV_BAD_LENGTH, 0, 0);
      cum[0] = 0;
    }
    return;
  }
  // tiles per request group; the last group runs to n_rows_padded (padding rows)
  int carry = 0;
  for (int base = 0; base < n_req; base += kSchedThreads) {
    const int i = base + threadIdx.x;
    int nt = 0;
    if (i < n_req) {
      const int gend = (i == n_req - 1) ? n_rows_padded : cu_rows[i + 1];
      nt = (gend - cu_rows[i] + TR - 1) / TR;
    }
    int total;
    const int incl = block_inclusive_scan(nt, lds, &total);
    if (i < n_req) req_tile[i + 1] = carry + incl;
    carry += total;
  }
  const int n_tiles = carry;
  if (threadIdx.x == 0) req_tile[0] = 0;
  __syncthreads();
  // tile records and their page counts, then the pages' prefix sum (first item per tile)
  carry = 0;
  for (int base = 0; base < n_tiles; base += kSchedThreads) {
    const int t = base + threadIdx.x;
    int pages = 0, r0 = 0, nr = 0, nv = 0, pos0 = 0, i = 0;
    if (t < n_tiles) {
      i = count_le(req_tile + 1, n_req - 1, t);  // request whose tiles hold t
      const int first = cu_rows[i];
      r0 = first + TR * (t - req_tile[i]);
      const int gend = (i == n_req - 1) ? n_rows_padded : cu_rows[i + 1];
      nr = min(TR, gend - r0);
      nv = max(0, min(r0 + nr, cu_rows[i + 1]) - r0);
      pos0 = start_pos[i] + (r0 - first);
      if (nv > 0) pages = (pos0 + nv + kPage - 1) / kPage;  // the tile's longest row sees pos0 + nv keys
    }
    int total;
    const int incl = block_inclusive_scan(pages, lds, &total);
    if (t < n_tiles) {
      int32_t *T = tiles + (int64_t)kTileRecWords * t;
      T[0] = r0;
      T[1] = nr;
      T[2] = nv;
      T[3] = pos0;
      T[4] = i;
      T[5] = pages;
      T[6] = carry + incl - pages;
      T[7] = 0;
      cum[t + 1] = carry + incl;
    }
    carry += total;
  }
  const int items = carry;
  if (threadIdx.x == 0) cum[0] = 0;
  // rows: causal length = position + 1; padding rows see nothing
  const int n_valid = cu_rows[n_req];
  for (int r = threadIdx.x; r < n_rows_padded; r += kSchedThreads) {
    int len = 0;
    if (r < n_valid) {
      const int i = count_le(cu_rows + 1, n_req, r);
      len = start_pos[i] + (r - cu_rows[i]) + 1;
    }
    row_len[r] = len;
  }
  __syncthreads();
  // every item's physical page: one wave per tile, lanes over its pages; a page the table
  // cannot give is -1 and flagged (every item of a tile is needed by the tile's longest row)
  {
    int flags = 0;
    const int lane = threadIdx.x & 63;
    for (int t = threadIdx.x >> 6; t < n_tiles; t += kSchedThreads / 64) {
      const int32_t *T = tiles + (int64_t)kTileRecWords * t;
      const int req = T[4], pages = T[5], i0 = T[6];
      for (int p = lane; p < pages; p += 64) {
        int phys = -1;
        if (p < bt_ld) {
          const int e = bt[(int64_t)req * bt_ld + p];
          if (e >= 0 && e < n_pages) phys = e;
          else flags |= INDEXER_FP4_DEV_BAD_PAGE;
        } else {
          flags |= INDEXER_FP4_DEV_TABLE_SHORT;
        }
        item_phys[i0 + p] = phys;
      }
    }
    if (flags) atomicOr(&s_flags, flags);
  }
  __syncthreads();
  if (threadIdx.x == 0) header(s_flags, n_tiles, items);
  // unit ranges and start records
  for (int u = threadIdx.x; u <= n_units; u += kSchedThreads) {
    const int64_t ib = (int64_t)u * items / n_units;
    sched[L.unit_begin + u] = (int32_t)ib;
    if (u < n_units) {
      const int ie = (int)(((int64_t)u + 1) * items / n_units);
      const int t = count_le(cum + 1, n_tiles, ib);
      sched[L.unit_tile + u] = t;
      int32_t *R = sched + L.urec + (int64_t)kUnitRecWords * u;
      R[0] = (int32_t)ib;
      R[1] = ie;
      R[2] = t;
      R[3] = 0;
      for (int j = 0; j < kTileRecWords; j++) R[4 + j] = t < n_tiles ? tiles[(int64_t)kTileRecWords * t + j] : 0;
      for (int j = 0; j < kUnitRecPhys; j++) R[12 + j] = (int)ib + j < ie ? item_phys[ib + j] : -1;
    }
  }
}

}  // namespace ifp4

using namespace ifp4;

extern "C" int64_t indexer_fp4_decode_sched_bytes(int32_t batch, int32_t next_n, int32_t n_units) {
  if (batch < 0 || next_n <= 0 || n_units <= 0) return -1;
  return 4 * DecodeSchedLayout(batch, n_units).words;
}

extern "C" int64_t indexer_fp4_prefill_sched_bytes(int32_t n_req, int32_t n_rows_padded, int32_t n_units,
                                                   int64_t bt_ld) {
  if (n_req <= 0 || n_rows_padded <= 0 || n_units <= 0 || bt_ld <= 0 || bt_ld > INT32_MAX) return -1;
  return 4 * PrefillSchedLayout(n_req, n_rows_padded, n_units, bt_ld).words;
}

extern "C" int indexer_fp4_decode_schedule(const int32_t *context_lens, int32_t batch, int32_t next_n,
                                           int32_t n_units, void *sched, int64_t sched_bytes, int32_t *row_len,
                                           void *stream) {
  clear_error();
  if (batch < 0 || next_n < 1 || next_n > 4 || n_units <= 0)
    return fail(INDEXER_FP4_EINVAL, "decode schedule: batch=%d must be >= 0, next_n=%d in 1..4, n_units=%d > 0",
                batch, next_n, n_units);
  if ((int64_t)batch * next_n > INT32_MAX / 2)
    return fail(INDEXER_FP4_EINVAL, "decode schedule: batch*next_n=%lld too large", (long long)batch * next_n);
  const int64_t need = indexer_fp4_decode_sched_bytes(batch, next_n, n_units);
  if (!sched || sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "decode schedule needs %lld bytes, buffer has %lld", (long long)need,
                (long long)sched_bytes);
  if ((uintptr_t)sched % 16 != 0) return fail(INDEXER_FP4_EINVAL, "schedule buffer must be 16-byte aligned");
  if (batch > 0 && (!context_lens || !row_len))
    return fail(INDEXER_FP4_EINVAL, "decode schedule needs context_lens and row_len");
  int rc = check_device();
  if (rc) return rc;
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, (hipStream_t)stream, context_lens,
                     batch, next_n, n_units, (int32_t *)sched, row_len);
  return launch_status("decode_schedule");
}

extern "C" int indexer_fp4_prefill_schedule(const int32_t *cu_rows, const int32_t *start_pos, int32_t n_req,
                                            int32_t n_rows_padded, int32_t n_units, const int32_t *block_table,
                                            int64_t bt_ld, int64_t n_pages, void *sched, int64_t sched_bytes,
                                            int32_t *row_len, void *stream) {
  clear_error();
  if (n_req <= 0 || n_units <= 0 || n_rows_padded <= 0 || n_rows_padded % kRowMultiple != 0)
    return fail(INDEXER_FP4_EINVAL,
                "prefill schedule: n_req=%d must be > 0, n_units=%d > 0, n_rows_padded=%d a positive multiple of %d",
                n_req, n_units, n_rows_padded, kRowMultiple);
  if (bt_ld <= 0 || bt_ld > INT32_MAX || n_pages < 0)
    return fail(INDEXER_FP4_EINVAL, "prefill schedule: bt_ld=%lld in 1..2^31-1, n_pages=%lld >= 0", (long long)bt_ld,
                (long long)n_pages);
  const int64_t need = indexer_fp4_prefill_sched_bytes(n_req, n_rows_padded, n_units, bt_ld);
  if (!sched || sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "prefill schedule needs %lld bytes, buffer has %lld", (long long)need,
                (long long)sched_bytes);
  if ((uintptr_t)sched % 16 != 0) return fail(INDEXER_FP4_EINVAL, "schedule buffer must be 16-byte aligned");
  if (!cu_rows || !start_pos || !row_len || !block_table)
    return fail(INDEXER_FP4_EINVAL, "prefill schedule needs cu_rows, start_pos, block_table and row_len");
  int rc = check_device();
  if (rc) return rc;
  hipLaunchKernelGGL(prefill_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, (hipStream_t)stream, cu_rows,
                     start_pos, n_req, n_rows_padded, n_units, block_table, bt_ld, n_pages, (int32_t *)sched, row_len);
  return launch_status("prefill_schedule");
}
