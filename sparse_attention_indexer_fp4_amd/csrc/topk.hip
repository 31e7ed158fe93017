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
// columns in ascending order. One 1024-thread workgroup per row; the histograms live in
// LDS, in several copies to spread the atomic traffic of lanes that hit the same bin.
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

}  // namespace ifp4

using namespace ifp4;

extern "C" int64_t indexer_topk_workspace_bytes(int32_t n_rows, int64_t max_len, int32_t k) {
  if (n_rows < 0 || max_len < 0 || k <= 0) return -1;
  return 0;
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
  hipLaunchKernelGGL(topk_row_kernel, dim3(n_rows), dim3(kTopkThreads), 0, (hipStream_t)stream, logits, logits_ld,
                     row_len, max_len, k, topk_idx, topk_ld);
  return launch_status("topk");
}
