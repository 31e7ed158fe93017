// Per-row top-k over fp32 logits.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), review fixes: top_k_per_row
// bounds its scan by the row's context, so the logits tail past it is never read; PR
// description, Accuracy: a row with at most index_topk keys keeps them all (the
// index_topk short-circuit).
//
// Exact selection by radix select on order-preserving 32-bit keys (flip the sign bit of
// non-negative floats, invert negative ones; -0.0 is folded onto +0.0): three histogram
// passes (11, 11 and 10 bits) narrow the key of the k-th largest value to one value T,
// then a gather keeps every key above T plus the lowest-column keys equal to T, writing
// columns in ascending order. Rows up to 16384 keys take one 1024-thread workgroup per
// row, with the histograms in LDS (several copies spread the atomic traffic of lanes that
// hit the same bin); longer rows take the chunked path further below.
#include "common.h"

namespace ifp4 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kCopies = 4;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(const float *__restrict__ logits, int64_t ld,
                                                               const int32_t *__restrict__ row_len, int64_t max_len,
                                                               int k, int32_t *__restrict__ out, int64_t out_ld) {
  __shared__ uint32_t hist[kCopies][kBins];
  __shared__ int s_scan[kTopkWaves];
  __shared__ int s_digit, s_above;
  __shared__ int s_gt[kTopkWaves], s_eq[kTopkWaves];

  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t len = row_len[r];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const float *row = logits + r * ld;
  int32_t *o = out + r * out_ld;

  if (len <= k) {  // short row: every key is kept
    for (int j = tid; j < k; j += kTopkThreads) o[j] = j < len ? j : -1;
    return;
  }
  const int n = (int)len;

  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
#pragma unroll 1
  for (int pass = 0; pass < 3; pass++) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);  // digits of 11, 11, 10 bits
    const uint32_t nb = pass == 2 ? 1024u : 2048u;
    for (int i = tid; i < kCopies * kBins; i += kTopkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    uint32_t *h = hist[tid & (kCopies - 1)];
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t key = order_key(row[j]);
      if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // Digit d with count(digit >= d) >= remaining > count(digit > d). Thread t owns bins
    // 2t, 2t+1; a suffix scan over threads (reversed thread order) gives counts from the top.
    const int b0 = 2 * tid, b1 = 2 * tid + 1;
    int c0 = 0, c1 = 0;
    if ((uint32_t)b1 < nb) {
#pragma unroll
      for (int c = 0; c < kCopies; c++) {
        c0 += hist[c][b0];
        c1 += hist[c][b1];
      }
    }
    int v = c0 + c1;
    {
      // suffix scan: x = sum of v over lanes >= this lane, then add the waves above
      int x = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(x, off, 64);
        if (lane + off < 64) x += y;
      }
      if (lane == 0) s_scan[wv] = x;  // sum of this wave
      __syncthreads();
      int above_waves = 0;
      for (int w2 = wv + 1; w2 < kTopkWaves; w2++) above_waves += s_scan[w2];
      v = x + above_waves;  // count of bins >= b0 (held by threads >= tid)
    }
    const int s_b0 = v;        // count(digit >= b0)
    const int s_b1 = v - c0;   // count(digit >= b1)
    const int s_b2 = s_b1 - c1;  // count(digit >= b1 + 1)
    if ((uint32_t)b1 < nb) {
      if (s_b1 >= remaining && s_b2 < remaining) {
        s_digit = b1;
        s_above = s_b2;
      } else if (s_b0 >= remaining && s_b1 < remaining) {
        s_digit = b0;
        s_above = s_b1;
      }
    }
    __syncthreads();
    remaining -= s_above;
    prefix |= (uint32_t)s_digit << shift;
    pmask |= (nb - 1) << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need_eq = remaining;  // keys equal to T still to take, lowest columns first

  // gather: wave wv owns the contiguous column range [c_lo, c_hi)
  const int chunk = ((n + kTopkWaves - 1) / kTopkWaves + 63) & ~63;
  const int c_lo = min(n, wv * chunk), c_hi = min(n, c_lo + chunk);
  int n_gt = 0, n_eq = 0;
  for (int j0 = c_lo; j0 < c_hi; j0 += 64) {
    const int j = j0 + lane;
    uint32_t key = 0;
    if (j < c_hi) key = order_key(row[j]);
    const uint64_t gt = __ballot(j < c_hi && key > T);
    const uint64_t eq = __ballot(j < c_hi && key == T);
    n_gt += __popcll(gt);
    n_eq += __popcll(eq);
  }
  if (lane == 0) {
    s_gt[wv] = n_gt;
    s_eq[wv] = n_eq;
  }
  __syncthreads();
  int eq_base = 0, out_base = 0;
  for (int w2 = 0; w2 < wv; w2++) {
    const int take_eq = min(max(need_eq - eq_base, 0), s_eq[w2]);
    out_base += s_gt[w2] + take_eq;
    eq_base += s_eq[w2];
  }
  for (int j0 = c_lo; j0 < c_hi; j0 += 64) {
    const int j = j0 + lane;
    uint32_t key = 0;
    if (j < c_hi) key = order_key(row[j]);
    const bool is_gt = j < c_hi && key > T;
    const bool is_eq = j < c_hi && key == T;
    const uint64_t eq = __ballot(is_eq);
    const bool take = is_gt || (is_eq && eq_base + (int)lanes_below(eq) < need_eq);
    const uint64_t tk = __ballot(take);
    const int pos = out_base + (int)lanes_below(tk);
    if (take && pos < k) o[pos] = j;  // exactly k are taken; the bound is insurance
    out_base += __popcll(tk);
    eq_base += __popcll(eq);
  }
}

// ---------------------------------------------------------------------------------------
// Long rows (decode at long context: few rows of 10^5 .. 10^6 keys). One workgroup per row
// would leave the GPU idle, so each row is cut into chunks of kChunk keys, one workgroup
// each, in three launches and without any grid-wide barrier:
//   clear    zero the row's histogram, counters and tickets in the workspace;
//   hist     histogram the top 12 key bits per chunk and add them into the row's histogram;
//            the last chunk to finish (atomic ticket) picks the bin b1 that holds the k-th
//            largest key and the count of keys above it;
//   collect  every chunk appends its keys above b1 ("sure") and its keys in b1
//            ("candidates") to the workspace; the last chunk to finish selects the
//            remaining keys exactly among the candidates (radix select on the low 20 bits,
//            ties resolved to the lowest columns by a second radix select on the column),
//            marks the chosen columns in an LDS bitmap and writes them out in ascending
//            order.
constexpr int kLongThreads = 256;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kChunk = 4096;
constexpr int kBins1 = 4096;                  // first digit: key bits 31..20
constexpr int64_t kShortMax = 16384;          // longer rows take the chunked path
constexpr int64_t kLongMaxLen = 1 << 20;      // bitmap of the finishing workgroup fits LDS
constexpr int kStateWords = 8;
enum { kTicket1 = 0, kTicket2 = 1, kBin1 = 2, kAbove1 = 3, kNSure = 4, kNCand = 5 };

struct LongWs {  // word offsets of the per-row areas in the workspace
  int64_t state, hist, sure, ckey, cidx, words;
  __host__ __device__ LongWs(int rows, int64_t cap, int k) {
    state = 0;
    hist = state + (int64_t)rows * kStateWords;
    sure = hist + (int64_t)rows * kBins1;
    ckey = sure + (int64_t)rows * k;
    cidx = ckey + (int64_t)rows * cap;
    words = cidx + (int64_t)rows * cap;
  }
};

__device__ __forceinline__ uint32_t coherent_load(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive suffix sum of v over the workgroup's threads (threads >= tid).
__device__ __forceinline__ int block_suffix_sum(int v, int *s_scan) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_down(v, off, 64);
    if (lane + off < 64) v += y;
  }
  if (lane == 0) s_scan[wv] = v;
  __syncthreads();
  for (int w2 = wv + 1; w2 < kLongWaves; w2++) v += s_scan[w2];
  __syncthreads();
  return v;
}

__global__ __launch_bounds__(kLongThreads) void topk_clear_kernel(uint32_t *__restrict__ ws, int rows) {
  const int r = blockIdx.x;
  uint32_t *st = ws + (int64_t)r * kStateWords;
  uint32_t *h = ws + (int64_t)rows * kStateWords + (int64_t)r * kBins1;
  if (threadIdx.x < kStateWords) st[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < kBins1; i += kLongThreads) h[i] = 0;
}

__global__ __launch_bounds__(kLongThreads) void topk_hist_kernel(const float *__restrict__ logits, int64_t ld,
                                                                const int32_t *__restrict__ row_len,
                                                                int64_t max_len, int k, uint32_t *ws, int rows,
                                                                int64_t cap) {
  __shared__ uint32_t h[kCopies][kBins1];
  __shared__ int s_scan[kLongWaves];
  __shared__ int s_last, s_bin, s_above;
  const int r = blockIdx.y, tid = threadIdx.x;
  const LongWs L(rows, cap, k);
  uint32_t *st = ws + L.state + (int64_t)r * kStateWords;
  uint32_t *gh = ws + L.hist + (int64_t)r * kBins1;
  int64_t len = row_len[r];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const int64_t start = (int64_t)blockIdx.x * kChunk;
  if (len > k && start < len) {
    for (int i = tid; i < kCopies * kBins1; i += kLongThreads) (&h[0][0])[i] = 0;
    __syncthreads();
    const float *row = logits + r * ld;
    const int64_t end = min(len, start + kChunk);
    uint32_t *hc = h[tid & (kCopies - 1)];
    for (int64_t j = start + tid; j < end; j += kLongThreads) atomicAdd(&hc[order_key(row[j]) >> 20], 1u);
    __syncthreads();
    for (int b = tid; b < kBins1; b += kLongThreads) {
      const uint32_t c = h[0][b] + h[1][b] + h[2][b] + h[3][b];
      if (c) atomicAdd(&gh[b], c);
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&st[kTicket1], 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last || len <= k) return;
  __threadfence();
  // the last chunk: bin holding the k-th largest key, from the row's full histogram
  constexpr int kPer = kBins1 / kLongThreads;  // bins per thread, consecutive
  uint32_t cnt[kPer];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    cnt[i] = coherent_load(&gh[kPer * tid + i]);
    sum += (int)cnt[i];
  }
  int acc = block_suffix_sum(sum, s_scan);  // keys in bins >= kPer*tid
#pragma unroll
  for (int i = 0; i < kPer; i++) {
    if (acc >= k && acc - (int)cnt[i] < k) {
      s_bin = kPer * tid + i;
      s_above = acc - (int)cnt[i];
    }
    acc -= (int)cnt[i];
  }
  __syncthreads();
  if (tid == 0) {
    st[kBin1] = (uint32_t)s_bin;
    st[kAbove1] = (uint32_t)s_above;
  }
}

// Radix select inside the finishing workgroup: among keys[i] (i < n) whose bits under
// `pmask` equal `prefix`, find the value of the bits below bit `top` that makes the
// `rem`-th largest key; returns the full key and leaves in *rem how many keys equal to it
// are still to be taken, in *n_eq how many keys equal it.
template <class KeyOf>
__device__ uint32_t block_select(int n, KeyOf key_of, uint32_t prefix, uint32_t pmask, int top, int *rem, int *n_eq,
                                 uint32_t *hist, int *s_scan, int *s_digit, int *s_above, int *s_cnt) {
  const int tid = threadIdx.x;
  while (top > 0) {
    const int nbits = top >= 8 ? 8 : top;
    const int shift = top - nbits;
    const uint32_t nb = 1u << nbits;
    for (uint32_t i = tid; i < 256; i += kLongThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kLongThreads) {
      const uint32_t key = key_of(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    const int c = (uint32_t)tid < nb ? (int)hist[tid] : 0;
    const int s = block_suffix_sum(c, s_scan);  // count(digit >= tid)
    if ((uint32_t)tid < nb && s >= *rem && s - c < *rem) {
      *s_digit = tid;
      *s_above = s - c;
      *s_cnt = c;
    }
    __syncthreads();
    *rem -= *s_above;
    *n_eq = *s_cnt;
    prefix |= (uint32_t)*s_digit << shift;
    pmask |= (nb - 1) << shift;
    top = shift;
    __syncthreads();
  }
  return prefix;
}

__global__ __launch_bounds__(kLongThreads) void topk_collect_kernel(const float *__restrict__ logits, int64_t ld,
                                                                   const int32_t *__restrict__ row_len,
                                                                   int64_t max_len, int k, uint32_t *ws, int rows,
                                                                   int64_t cap, int32_t *__restrict__ out,
                                                                   int64_t out_ld) {
  extern __shared__ uint32_t bitmap[];  // ceil(max_len / 32) words, used by the finishing chunk
  __shared__ uint32_t hist[256];
  __shared__ int s_scan[kLongWaves];
  __shared__ int s_last, s_digit, s_above, s_cnt;
  const int r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const LongWs L(rows, cap, k);
  uint32_t *st = ws + L.state + (int64_t)r * kStateWords;
  uint32_t *sure = ws + L.sure + (int64_t)r * k;
  uint32_t *ckey = ws + L.ckey + (int64_t)r * cap;
  uint32_t *cidx = ws + L.cidx + (int64_t)r * cap;
  int64_t len = row_len[r];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const int64_t start = (int64_t)blockIdx.x * kChunk;
  if (len > k && start < len) {
    const uint32_t bin1 = st[kBin1];
    const float *row = logits + r * ld;
    const int64_t end = min(len, start + kChunk);
    for (int64_t j0 = start + 64 * wv; j0 < end; j0 += kLongThreads) {
      const int64_t j = j0 + lane;
      const uint32_t key = j < end ? order_key(row[j]) : 0u;
      const uint32_t d = key >> 20;
      const bool is_sure = j < end && d > bin1;
      const bool is_cand = j < end && d == bin1;
      const uint64_t ms = __ballot(is_sure);
      const uint64_t mc = __ballot(is_cand);
      if (ms) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&st[kNSure], (uint32_t)__popcll(ms));
        base = __shfl(base, 0, 64);
        if (is_sure) sure[base + lanes_below(ms)] = (uint32_t)j;
      }
      if (mc) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&st[kNCand], (uint32_t)__popcll(mc));
        base = __shfl(base, 0, 64);
        if (is_cand) {
          ckey[base + lanes_below(mc)] = key;
          cidx[base + lanes_below(mc)] = (uint32_t)j;
        }
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&st[kTicket2], 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  int32_t *o = out + r * out_ld;
  if (len <= k) {  // short row: every key is kept
    for (int j = tid; j < k; j += kLongThreads) o[j] = j < len ? j : -1;
    return;
  }
  const int n_sure = (int)coherent_load(&st[kNSure]);
  const int n_cand = (int)coherent_load(&st[kNCand]);
  const uint32_t bin1 = coherent_load(&st[kBin1]);
  const int nwords = (int)((len + 31) / 32);
  for (int i = tid; i < nwords; i += kLongThreads) bitmap[i] = 0;
  __syncthreads();
  for (int i = tid; i < n_sure; i += kLongThreads) {
    const uint32_t j = coherent_load(&sure[i]);
    atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  // the remaining k - n_sure keys come from the candidates (all in bin b1)
  int rem = k - n_sure, n_eq = 0;
  const uint32_t T = block_select(n_cand, [&](int i) { return coherent_load(&ckey[i]); }, bin1 << 20, 0xFFF00000u,
                                  20, &rem, &n_eq, hist, s_scan, &s_digit, &s_above, &s_cnt);
  // keys equal to T: keep the rem lowest columns (select the largest of 2^20-1-column)
  uint32_t cut = 0;  // ties with column <= cut are kept
  if (rem < n_eq) {
    int rem2 = rem, n_eq2 = 0;
    const uint32_t sel = block_select(
        n_cand,
        [&](int i) { return coherent_load(&ckey[i]) == T ? (0xFFFFFu - coherent_load(&cidx[i])) : 0xFFFFFFFFu; },
        0u, 0xFFF00000u, 20, &rem2, &n_eq2, hist, s_scan, &s_digit, &s_above, &s_cnt);
    cut = 0xFFFFFu - sel;
  } else {
    cut = 0xFFFFFFFFu;
  }
  for (int i = tid; i < n_cand; i += kLongThreads) {
    const uint32_t key = coherent_load(&ckey[i]);
    const uint32_t j = coherent_load(&cidx[i]);
    if (key > T || (key == T && j <= cut)) atomicOr(&bitmap[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // columns out in ascending order: each thread owns a contiguous run of bitmap words
  const int per = (nwords + kLongThreads - 1) / kLongThreads;
  const int w0 = min(nwords, tid * per), w1 = min(nwords, w0 + per);
  int mine = 0;
  for (int i = w0; i < w1; i++) mine += __popc(bitmap[i]);
  // exclusive prefix over threads = total - suffix(tid); the total is exactly k when the
  // selection is consistent, and the bounds below hold either way
  const int suffix = block_suffix_sum(mine, s_scan);
  if (tid == 0) s_cnt = suffix;
  __syncthreads();
  const int total = s_cnt;
  int pos = total - suffix;
  for (int i = w0; i < w1; i++) {
    uint32_t m = bitmap[i];
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      if (pos >= 0 && pos < k) o[pos] = 32 * i + b;
      pos++;
    }
  }
  for (int j = max(total, 0) + tid; j < k; j += kLongThreads) o[j] = -1;
}

}  // namespace ifp4

using namespace ifp4;

static bool use_long_path(int64_t max_len, int32_t k) {
  return max_len > kShortMax && max_len <= kLongMaxLen && k < max_len;
}

extern "C" int64_t indexer_topk_workspace_bytes(int32_t n_rows, int64_t max_len, int32_t k) {
  if (n_rows < 0 || max_len < 0 || k <= 0) return -1;
  if (!use_long_path(max_len, k)) return 0;
  return 4 * LongWs(n_rows, max_len, k).words;
}

extern "C" int indexer_topk(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                            int64_t max_len, int32_t k, int32_t *topk_idx, int64_t topk_ld, void *workspace,
                            int64_t ws_bytes, void *stream) {
  clear_error();
  (void)workspace;
  if (k <= 0 || n_rows < 0 || max_len < 0)
    return fail(INDEXER_FP4_EINVAL, "topk: k=%d must be > 0, n_rows=%d >= 0, max_len=%lld >= 0", k, n_rows,
                (long long)max_len);
  if (max_len > logits_ld)
    return fail(INDEXER_FP4_EINVAL, "topk: max_len=%lld exceeds logits_ld=%lld", (long long)max_len,
                (long long)logits_ld);
  if (max_len > INT32_MAX) return fail(INDEXER_FP4_EINVAL, "topk: max_len=%lld too large", (long long)max_len);
  if (topk_ld < k) return fail(INDEXER_FP4_ENOSPC, "topk: topk_ld=%lld < k=%d", (long long)topk_ld, k);
  const int64_t need = indexer_topk_workspace_bytes(n_rows, max_len, k);
  if (ws_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "topk: workspace needs %lld bytes, has %lld", (long long)need, (long long)ws_bytes);
  if (n_rows > 0 && (!logits || !row_len || !topk_idx)) return fail(INDEXER_FP4_EINVAL, "topk: NULL pointer");
  int rc = check_device();
  if (rc) return rc;
  if (n_rows == 0) return INDEXER_FP4_OK;
  hipStream_t st = (hipStream_t)stream;
  if (!use_long_path(max_len, k)) {
    hipLaunchKernelGGL(topk_row_kernel, dim3(n_rows), dim3(kTopkThreads), 0, st, logits, logits_ld, row_len, max_len,
                       k, topk_idx, topk_ld);
    return launch_status("topk");
  }
  if (!workspace || (uintptr_t)workspace % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "topk: rows up to %lld keys need a 16-byte aligned workspace", (long long)max_len);
  uint32_t *ws = (uint32_t *)workspace;
  const unsigned chunks = (unsigned)((max_len + kChunk - 1) / kChunk);
  const size_t lds = 4 * (size_t)((max_len + 31) / 32);
  static bool lds_set = false;  // the bitmap may exceed the default LDS limit of a launch
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute((const void *)topk_collect_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(4 * ((kLongMaxLen + 31) / 32)));
    if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "topk: hipFuncSetAttribute: %s", hipGetErrorString(e));
    lds_set = true;
  }
  hipLaunchKernelGGL(topk_clear_kernel, dim3(n_rows), dim3(kLongThreads), 0, st, ws, n_rows);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(chunks, n_rows), dim3(kLongThreads), 0, st, logits, logits_ld, row_len,
                     max_len, k, ws, n_rows, max_len);
  hipLaunchKernelGGL(topk_collect_kernel, dim3(chunks, n_rows), dim3(kLongThreads), lds, st, logits, logits_ld,
                     row_len, max_len, k, ws, n_rows, max_len, topk_idx, topk_ld);
  return launch_status("topk");
}
