// Per-row top-k over fp32 logits.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), review fixes: top_k_per_row
// bounds its scan by the row's context, so the logits tail past it is never read; PR
// description, Accuracy: a row with at most index_topk keys keeps them all (the
// index_topk short-circuit).
//
// Exact selection by radix select on order-preserving 32-bit keys (flip the sign bit of
// non-negative floats, invert negative ones; -0.0 is folded onto +0.0): histogram passes
// over digits of the keys (each path's width is given with it below) narrow the key of the
// k-th largest value to one value T, then every key above T is kept together with the
// lowest-column keys equal to T, and the columns are written in ascending order.
//
// Rows up to 6144 keys: one workgroup per row with the row's keys in registers; up to 16384
// keys: one workgroup per row with the row's keys held in LDS (512 threads in launches of up
// to 2047 rows, 256 in larger ones). Longer rows: the chunked path further below. Every loop
// that reads global memory issues all of a thread's loads before it uses them, so a pass
// costs one memory latency rather than one per element.
#include <mutex>

#include "common.h"

namespace ifp4 {

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the lanes of a wave (lanes <= this one): DPP shifts within rows of
// 16 lanes, then row broadcasts across rows (no LDS round trips).
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, into rows 2 and 3
  return v;
}

// Wave-wide sum, returned to every lane (the DPP prefix sum's last lane: no LDS round trips).
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_prefix_sum(v), 63); }

// Inclusive suffix sum of v over the workgroup's threads (threads >= tid): within a wave,
// the wave's total less the prefix before this lane.
template <int NT>
__device__ __forceinline__ int block_suffix_sum(int v, int *s_scan) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int incl = wave_prefix_sum(v);
  const int wtot = __builtin_amdgcn_readlane(incl, 63);
  v = wtot - incl + v;
  if (lane == 0) s_scan[wv] = wtot;
  __syncthreads();
  for (int w2 = wv + 1; w2 < NT / 64; w2++) v += s_scan[w2];
  __syncthreads();
  return v;
}

// Inclusive prefix sum of v over the workgroup's threads (threads <= tid); *total gets the
// sum over all of them. s_w (one word a wave) must not be reused before another barrier.
template <int NT>
__device__ __forceinline__ int block_prefix_sum(int v, int *s_w, int &total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_prefix_sum(v);
  if (lane == 63) s_w[wv] = v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; w2++) {
    const int x = s_w[w2];
    before += w2 < wv ? x : 0;
    total += x;
  }
  return v + before;
}

// Histogram increment of digit d (for lanes with `active`). Keys of one row cluster in a
// few digits, so plain LDS atomics from a wave would mostly hit one address and serialize;
// the two most common digits of the wave are added once each by a leader lane.
__device__ __forceinline__ void hist_add(uint32_t *h, uint32_t d, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t act = __ballot(active);
#pragma unroll
  for (int round = 0; round < 2; round++) {
    if (!act) break;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t dl = __builtin_amdgcn_readlane(d, leader);
    const uint64_t m = __ballot(active && d == dl);
    if (lane == leader) atomicAdd(&h[dl], (uint32_t)__popcll(m));
    if ((m >> lane) & 1ull) active = false;
    act &= ~m;
  }
  if (active) atomicAdd(&h[d], 1u);
}

// Radix select over items i < n whose key bits under `pmask` equal `prefix`: resolves the
// bits below bit `top` of the rem-th largest such key, 8 bits a pass. Returns that key T;
// *rem becomes how many keys equal to T still have to be taken, *n_eq how many equal T.
// Callers pass a prefix that every item matches or top > 0 (with top == 0 every item then
// equals T). hist has 4 x 256 words.
template <int NT, class KeyOf>
__device__ uint32_t block_select(int n, KeyOf key_of, uint32_t prefix, uint32_t pmask, int top, int *rem, int *n_eq,
                                 uint32_t *hist, int *s_scan, int *s_misc) {
  const int tid = threadIdx.x;
  *n_eq = n;
  while (top > 0) {
    const int nbits = top >= 8 ? 8 : top;
    const int shift = top - nbits;
    const uint32_t nb = 1u << nbits;
    for (int i = tid; i < 4 * 256; i += NT) hist[i] = 0;
    __syncthreads();
    uint32_t *h = hist + 256 * ((tid >> 6) & 3);
    for (int i0 = 0; i0 < n; i0 += NT) {
      const int i = i0 + tid;
      const uint32_t key = i < n ? key_of(i) : 0u;
      hist_add(h, (key >> shift) & (nb - 1), i < n && (key & pmask) == prefix);
    }
    __syncthreads();
    const int c = (uint32_t)tid < nb ? (int)(hist[tid] + hist[256 + tid] + hist[512 + tid] + hist[768 + tid]) : 0;
    const int s = block_suffix_sum<NT>(c, s_scan);  // count(digit >= tid)
    if ((uint32_t)tid < nb && s >= *rem && s - c < *rem) {
      s_misc[0] = tid;
      s_misc[1] = s - c;
      s_misc[2] = c;
    }
    __syncthreads();
    *rem -= s_misc[1];
    *n_eq = s_misc[2];
    prefix |= (uint32_t)s_misc[0] << shift;
    pmask |= (nb - 1) << shift;
    top = shift;
    __syncthreads();
  }
  return prefix;
}

// Number of leading bits shared by every key of a set (from its smallest and largest key):
// the search can start below them. __clz(0) is 32.
__device__ __forceinline__ int shared_bits(uint32_t kmin, uint32_t kmax) { return __clz((int)(kmin ^ kmax)); }

// Mask of the top sb bits, sb in [0, 32]. Written with a 64-bit shift instead of a select:
// this compiler turned the select form `sb >= 32 ? ~0u : ~(~0u >> sb)` into a scalar
// conditional move that read a stale condition code and returned ~0u for sb = 6.
__device__ __forceinline__ uint32_t top_bits_mask(int sb) { return (uint32_t)~(0xFFFFFFFFull >> sb); }

// Wave-wide min and max in the last lane (the prefix pattern of wave_prefix_sum, with the
// identity of each operation for lanes that have no source): DPP moves, no LDS round trips.
__device__ __forceinline__ uint32_t wave_min_last(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_max_last(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}

// Block-wide min and max, returned to every thread, with one barrier (which also publishes
// whatever the block wrote to LDS before the call). s_mm (two words a wave) is read after
// the barrier, so it must not be written again by this launch.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t &kmin, uint32_t &kmax, uint32_t *s_mm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  kmin = wave_min_last(kmin);
  kmax = wave_max_last(kmax);
  if (lane == 63) {
    s_mm[2 * wv] = kmin;
    s_mm[2 * wv + 1] = kmax;
  }
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
  for (int w2 = 0; w2 < NT / 64; w2++) {
    kmin = min(kmin, s_mm[2 * w2]);
    kmax = max(kmax, s_mm[2 * w2 + 1]);
  }
}

// ---------------------------------------------------------------------------------------
// Rows up to kShortMax keys: one workgroup per row (several rows share a CU). The
// row's keys are staged in LDS with their smallest and largest value; a 1024-bin histogram
// spread linearly over that range (d = min((key - kmin) >> s, 1023)) finds the bin b that
// holds the k-th largest key; keys in higher bins are kept and the few keys in b are ranked
// by counting (radix select when there are many), ties to the lowest columns. Each wave owns
// one contiguous column range: one walk over it counts the keys above b and lists the keys
// of b in the wave's own part of the list (no shared counter), and after the selection a
// second walk writes the kept columns in ascending order.
// Workgroups of 512 threads for launches of at most kWideRows rows, whose rows gain from each
// row's walks spreading over more waves (prefill steps of 120, 824 and 1784 rows of up to
// 4.3 K keys: 15.9 -> 11.8, 19.2 -> 17.4, 30.0 -> 27.5 us against 256 threads); 256 threads
// for launches of more rows, where the two measured alike (2048-row steps: within 0.4 us).
constexpr int64_t kShortMax = 16384;
constexpr int kShortBins = 1024;
constexpr int kShortRank = 256;  // bin-b keys ranked by counting
constexpr int kWideRows = 2047;

template <int kShortThreads>
__global__ __launch_bounds__(kShortThreads) void topk_row_kernel(const float *__restrict__ logits, int64_t ld,
                                                                const int32_t *__restrict__ row_len, int64_t max_len,
                                                                int k, uint32_t *__restrict__ row_hist,
                                                                int32_t *__restrict__ out, int64_t out_ld) {
  constexpr int kShortWaves = kShortThreads / 64;
  extern __shared__ uint32_t keys[];  // max_len words
  __shared__ uint32_t hist[kShortBins];
  __shared__ uint32_t sel[kShortMax / 32];  // chosen bin-b keys, by column
  __shared__ __attribute__((aligned(16))) uint32_t ckey[kShortWaves * kShortRank];  // per-wave lists
  __shared__ __attribute__((aligned(16))) uint32_t ccol[kShortWaves * kShortRank];
  __shared__ int s_nb[kShortWaves];
  __shared__ int s_scan[3 * kShortWaves], s_misc[8];
  __shared__ uint32_t s_mm[2 * kShortWaves];
  __shared__ int s_gt[kShortWaves];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t len64 = row_len[r];
  len64 = len64 < 0 ? 0 : (len64 > max_len ? max_len : len64);
  const int n = (int)len64;
  int32_t *o = out + r * out_ld;
  if (row_hist)  // not used for rows this short: left zero for the next scorer call
    for (int i = tid; i < kHistBins; i += kShortThreads) row_hist[r * kHistBins + i] = 0u;
  if (n <= k) {  // short row: every key is kept
    for (int j = tid; j < k; j += kShortThreads) o[j] = j < n ? j : -1;
    return;
  }
  // stage the row (16 loads in flight per thread and round), clear the histogram and bitmap
  const float *row = logits + r * ld;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int base = 0; base < n; base += 16 * kShortThreads) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; u++) {
      const int j = base + u * kShortThreads + tid;
      v[u] = j < n ? row[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; u++) {
      const int j = base + u * kShortThreads + tid;
      if (j < n) {
        const uint32_t key = order_key(v[u]);
        keys[j] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
  for (int i = tid; i < kShortBins; i += kShortThreads) hist[i] = 0u;
  const int nwords = (n + 31) / 32;
  for (int i = tid; i < nwords; i += kShortThreads) sel[i] = 0u;
  if (tid == 0) s_misc[3] = 0;
  block_minmax<kShortThreads>(kmin, kmax, s_mm);  // its barrier publishes all of the above
  const int bl = 32 - __clz((int)(kmax - kmin));
  const int sh = bl > 10 ? bl - 10 : 0;
  auto digit = [&](uint32_t key) { return min((key - kmin) >> sh, (uint32_t)(kShortBins - 1)); };
  for (int i0 = 0; i0 < n; i0 += kShortThreads) {
    const int i = i0 + tid;
    hist_put(hist, i < n ? digit(keys[i]) : 0u, i < n);
  }
  __syncthreads();
  // the bin b of the k-th largest key (thread t owns bins kPer t .. kPer t + kPer - 1)
  {
    constexpr int kPer = kShortBins / kShortThreads;
    static_assert(kPer * kShortThreads == kShortBins, "bins per thread");
    uint32_t c[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      c[i] = hist[kPer * tid + i];
      sum += (int)c[i];
    }
    int tot;
    const int incl = block_prefix_sum<kShortThreads>(sum, s_scan, tot);
    int acc = tot - incl + sum;  // keys in bins >= kPer*tid
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      if (acc >= k && acc - (int)c[i] < k) {
        s_misc[0] = kPer * tid + i;         // b
        s_misc[1] = k - (acc - (int)c[i]);  // keys of b to take
        s_misc[2] = (int)c[i];              // keys in b
      }
      acc -= (int)c[i];
    }
    __syncthreads();
  }
  const uint32_t b = (uint32_t)s_misc[0];
  const int need = s_misc[1], nb = s_misc[2];
  const bool rank_path = nb <= kShortRank;
  // wave wv owns the contiguous column range [c_lo, c_hi)
  const int chunk = ((n + kShortWaves - 1) / kShortWaves + 63) & ~63;
  const int c_lo = min(n, wv * chunk), c_hi = min(n, c_lo + chunk);
  // one walk: keys above b are counted, keys of b listed (rank path) in this wave's list
  {
    int n_gt = 0, n_b = 0;
    uint32_t *wkey = ckey + wv * kShortRank, *wcol = ccol + wv * kShortRank;
    for (int j0 = c_lo; j0 < c_hi; j0 += 64) {
      const int j = j0 + lane;
      const bool ok = j < c_hi;
      const uint32_t key = ok ? keys[j] : 0u;
      const uint32_t d = digit(key);
      n_gt += __popcll(__ballot(ok && d > b));
      if (rank_path) {
        const bool in_b = ok && d == b;
        const uint64_t m = __ballot(in_b);
        if (in_b) {
          const int at = n_b + (int)lanes_below(m);
          wkey[at] = key;
          wcol[at] = (uint32_t)j;
        }
        n_b += __popcll(m);
      }
    }
    if (lane == 0) {
      s_gt[wv] = n_gt;
      s_nb[wv] = n_b;
    }
  }
  __syncthreads();
  if (rank_path) {
    // the lists hold the nb keys of b; keep those ranked below `need` (key descending,
    // column ascending). Thread t takes the t-th entry of the lists in wave order.
    if (tid < nb) {
      int w = 0, t = tid;
      while (w < kShortWaves - 1 && t >= s_nb[w]) t -= s_nb[w++];
      const uint32_t key = ckey[w * kShortRank + t], col = ccol[w * kShortRank + t];
      int rank = 0;
      for (int w2 = 0; w2 < kShortWaves; w2++) {
        const int m2 = s_nb[w2];
        const uint4 *k4 = reinterpret_cast<const uint4 *>(ckey + w2 * kShortRank);
        const uint4 *c4 = reinterpret_cast<const uint4 *>(ccol + w2 * kShortRank);
        // four entries per read (entries past m2 are in the list's space and not counted)
        for (int g = 0; g < m2; g += 4) {
          const uint4 kq = k4[g / 4], cq = c4[g / 4];
          const uint32_t kv[4] = {kq.x, kq.y, kq.z, kq.w}, cv[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
          for (int e = 0; e < 4; e++)
            rank += (g + e < m2 && (kv[e] > key || (kv[e] == key && cv[e] < col))) ? 1 : 0;
        }
      }
      if (rank < need) atomicOr(&sel[col >> 5], 1u << (col & 31));
    }
  } else {
    // many keys in b (ties, clusters): radix select over key - kmin among them. Their offsets
    // lie in [b << sh, (b + 1) << sh), so they share the top 32 - sh bits (b); keys of other
    // bins are mapped to a value whose top bits differ from b's
    const uint32_t other = b == 0 ? 0xFFFFFFFFu : 0u;
    auto off_of = [&](int i) {
      const uint32_t key = keys[i];
      return digit(key) == b ? key - kmin : other;
    };
    int rem = need, n_eq = 0;
    const uint32_t T = kmin + block_select<kShortThreads>(n, off_of, b << sh, top_bits_mask(32 - sh), sh, &rem,
                                                          &n_eq, hist, s_scan, s_misc + 4);
    uint32_t cut = 0xFFFFFFFFu;  // keys equal to T with column <= cut are kept
    if (rem < n_eq) {
      int rem2 = rem, n_eq2 = 0;
      const uint32_t selc = block_select<kShortThreads>(
          n, [&](int i) { return keys[i] == T ? (0xFFFFFu - (uint32_t)i) : 0xFFFFFFFFu; }, 0u, 0xFFF00000u, 20,
          &rem2, &n_eq2, hist, s_scan, s_misc + 4);
      cut = 0xFFFFFu - selc;
    }
    for (int i = tid; i < n; i += kShortThreads) {
      const uint32_t key = keys[i];
      if (digit(key) == b && (key > T || (key == T && (uint32_t)i <= cut)))
        atomicOr(&sel[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  // kept columns of this wave: those above b plus the chosen keys of b (set bits of its
  // range of the bitmap; a non-empty range starts at a multiple of 64, and no bit past n is
  // ever set)
  {
    int n_sel = 0;
    if (c_lo < c_hi)
      for (int wd = c_lo / 32 + lane; wd < (c_hi + 31) / 32; wd += 64) n_sel += __popc(sel[wd]);
    n_sel = wave_sum(n_sel);
    if (lane == 0) s_gt[wv] += n_sel;  // each wave updates only its own entry
  }
  __syncthreads();
  int out_base = 0;
  for (int w2 = 0; w2 < wv; w2++) out_base += s_gt[w2];
  auto take = [&](int j) {
    const uint32_t key = keys[j];
    return digit(key) > b || ((sel[j >> 5] >> (j & 31)) & 1u);
  };
  for (int j0 = c_lo; j0 < c_hi; j0 += 64) {
    const int j = j0 + lane;
    const bool t = j < c_hi && take(j);
    const uint64_t tk = __ballot(t);
    const int pos = out_base + (int)lanes_below(tk);
    if (t && pos < k) o[pos] = j;  // exactly k are taken; the bound is insurance
    out_base += __popcll(tk);
  }
}

// ---------------------------------------------------------------------------------------
// Rows up to kRegMax keys (prefill chunks of a few thousand keys a row, short decode rows):
// the row's keys stay in registers, so a workgroup holds no LDS copy of them and every row
// of a 2048-row launch is resident at once. The row is cut into one contiguous column range
// per wave (a multiple of 64 columns, the last ones possibly empty); lane l of wave w holds
// the columns c_w + 64 u + l. The exact k-th largest key T comes first: a 1024-bin
// histogram spread linearly over the row's [min, max], then, while the bin that holds T has
// more than kShortRank keys, histograms of the next 10 bits of key - min over that bin's
// keys, and finally the bin's keys ranked by counting (or nothing more when a bin is one
// value). Each wave then counts its keys above and equal to T, and one walk in column order
// writes every key above T and the lowest-column keys equal to T.
constexpr int64_t kRegMax = 6144;
// Launches of up to kRegWideRows rows take 512-thread workgroups (a row's passes spread over
// 8 waves), larger ones 256 threads: either way every workgroup of a launch up to 2048 rows
// is resident at once on 256 CUs (32 waves a CU).
constexpr int kRegWideRows = 1024;

template <int NT, int R>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void topk_reg_kernel(
    const float *__restrict__ logits, int64_t ld, const int32_t *__restrict__ row_len, int64_t max_len, int k,
    uint32_t *__restrict__ row_hist, int32_t *__restrict__ out, int64_t out_ld) {
  constexpr int NW = NT / 64;
  static_assert(NW * 64 * R == kRegMax, "the launch shapes cover kRegMax keys");
  __shared__ uint32_t hist[kShortBins];
  __shared__ __attribute__((aligned(16))) uint32_t lst[NW * kShortRank];  // per-wave candidate keys
  __shared__ int s_scan[NW], s_nb[NW], s_gt[NW], s_eq[NW], s_misc[4];
  __shared__ uint32_t s_mm[2 * NW];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t len64 = row_len[r];
  len64 = len64 < 0 ? 0 : (len64 > max_len ? max_len : len64);
  const int n = (int)len64;
  int32_t *o = out + r * out_ld;
  if (row_hist)  // not used for rows this short: left zero for the next scorer call
    for (int i = tid; i < kHistBins; i += NT) row_hist[r * kHistBins + i] = 0u;
  if (n <= k) {  // every key is kept
    for (int j = tid; j < k; j += NT) o[j] = j < n ? j : -1;
    return;
  }
  // this wave's columns [c0, c1) in ns slots of 64 (wave-uniform); all loads in one round
  const int chunk = ((n + NW - 1) / NW + 63) & ~63;
  const int c0 = min(n, wv * chunk), c1 = min(n, c0 + chunk);
  const int ns = (c1 - c0 + 63) >> 6;
  const __amdgpu_buffer_rsrc_t src = buffer_view(const_cast<float *>(logits + r * ld), 4u * (uint32_t)n);
  uint32_t key[R];
#pragma unroll
  for (int u = 0; u < R; u++)
    key[u] = u < ns ? __builtin_amdgcn_raw_buffer_load_b32(src, 4 * (c0 + 64 * u + lane), 0, 0) : 0u;
  for (int i = tid; i < kShortBins; i += NT) hist[i] = 0u;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  const int lim = c1 - c0 - lane;  // the lane's slot u holds a column iff 64 u < lim
#pragma unroll
  for (int u = 0; u < R; u++) {
    if (u < ns) {
      const bool ok = 64 * u < lim;
      const uint32_t kk = order_key(__uint_as_float(key[u]));
      key[u] = ok ? kk : 0u;
      kmax = max(kmax, key[u]);
      kmin = min(kmin, ok ? kk : 0xFFFFFFFFu);
    }
  }
  block_minmax<NT>(kmin, kmax, s_mm);  // its barrier also publishes the cleared histogram
  // From here on a key is held as key - kmin, and a lane of the last slot past the row's end
  // as 0, the row's smallest value: it sorts below or ties with every key of the row and
  // comes after all of them in column order, so it is never among the k kept (the
  // lowest-column keys win ties) and needs no mask below. Slots u >= ns hold nothing and are
  // skipped.
#pragma unroll
  for (int u = 0; u < R; u++) key[u] = max(key[u], kmin) - kmin;
  // the bin of the want-th largest counted key: s_misc[0] bin, [1] keys in higher bins, [2] in it
  auto find_bin = [&](int want) __attribute__((always_inline)) {
    constexpr int kPer = kShortBins / NT;
    uint32_t c[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      c[i] = hist[kPer * tid + i];
      sum += (int)c[i];
    }
    int tot;
    const int incl = block_prefix_sum<NT>(sum, s_scan, tot);
    int acc = tot - incl + sum;  // keys in bins >= kPer * tid
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      if (acc >= want && acc - (int)c[i] < want) {
        s_misc[0] = kPer * tid + i;
        s_misc[1] = acc - (int)c[i];
        s_misc[2] = (int)c[i];
      }
      acc -= (int)c[i];
    }
    __syncthreads();
  };
  // level 0: bins over the whole range (key - kmin < 2^bl)
  const int bl = 32 - __clz((int)(kmax - kmin));
  int sh = bl > 10 ? bl - 10 : 0;
#pragma unroll
  for (int u = 0; u < R; u++)
    if (u < ns) atomicAdd(&hist[key[u] >> sh], 1u);
  __syncthreads();
  find_bin(k);
  uint32_t pre = (uint32_t)s_misc[0] << sh;  // bits of T - kmin under pmask
  uint32_t pmask = top_bits_mask(32 - sh);
  int need = k - s_misc[1], nb = s_misc[2];  // keys of the bin still to take; keys in it
  // further levels while the bin is crowded
  while (nb > kShortRank && sh > 0) {
    const int s2 = sh > 10 ? sh - 10 : 0;
    const uint32_t dm = (1u << (sh - s2)) - 1u;
    __syncthreads();  // every thread has read s_misc and the histogram of the last level
    for (int i = tid; i < kShortBins; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < R; u++)
      if (u < ns) hist_put(hist, (key[u] >> s2) & dm, (key[u] & pmask) == pre);
    __syncthreads();
    find_bin(need);
    pre |= (uint32_t)s_misc[0] << s2;
    pmask |= dm << s2;
    need -= s_misc[1];
    nb = s_misc[2];
    sh = s2;
  }
  // One pass over the slots: per wave, the keys in bins above T's and the keys of T's bin,
  // the latter listed when they still have to be ranked.
  int gt = 0, cnt = 0;
  uint32_t *wl = lst + wv * kShortRank;
#pragma unroll
  for (int u = 0; u < R; u++) {
    if (u < ns) {
      const uint32_t hi = key[u] & pmask;
      gt += __popcll(__ballot(hi > pre));
      const uint64_t m = __ballot(hi == pre);
      if (sh > 0 && m != 0 && hi == pre) wl[cnt + (int)lanes_below(m)] = key[u];
      cnt += __popcll(m);
    }
  }
  uint32_t T;  // T - kmin
  int eq;      // this wave's keys equal to T
  if (sh == 0) {
    T = pre;  // the bin is one value
    eq = cnt;
  } else {
    // rank the bin's keys by counting: the need-th largest of them is T
    if (lane == 0) s_nb[wv] = cnt;
    __syncthreads();
    if (tid < nb) {
      int w = 0, t = tid;
      while (w < NW - 1 && t >= s_nb[w]) t -= s_nb[w++];
      const uint32_t mine = lst[w * kShortRank + t];
      int g = 0, e = 0;
      for (int w2 = 0; w2 < NW; w2++) {
        const int m2 = s_nb[w2];
        const uint4 *k4 = reinterpret_cast<const uint4 *>(lst + w2 * kShortRank);
        for (int q = 0; q < m2; q += 4) {  // four entries a read; those past m2 are not counted
          const uint4 kq = k4[q / 4];
          const uint32_t kv[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
          for (int x = 0; x < 4; x++) {
            g += (q + x < m2 && kv[x] > mine) ? 1 : 0;
            e += (q + x < m2 && kv[x] == mine) ? 1 : 0;
          }
        }
      }
      if (g < need && g + e >= need) s_misc[3] = (int)mine;  // every such thread holds T
    }
    __syncthreads();
    T = (uint32_t)s_misc[3];
    // the wave's own listed keys above and equal to T
    eq = 0;
    for (int i0 = 0; i0 < cnt; i0 += 64) {
      const bool ok = i0 + lane < cnt;
      const uint32_t x = ok ? wl[i0 + lane] : 0u;
      gt += __popcll(__ballot(ok && x > T));
      eq += __popcll(__ballot(ok && x == T));
    }
  }
  if (lane == 0) {
    s_gt[wv] = gt;
    s_eq[wv] = eq;
  }
  __syncthreads();
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; w2++) {
    n_gt += s_gt[w2];
    n_eq += s_eq[w2];
  }
  const int need_t = k - n_gt;  // keys equal to T kept, those of the lowest columns
  int out_base = 0, eq_run = 0;
  for (int w2 = 0; w2 < wv; w2++) {
    out_base += s_gt[w2] + min(max(need_t - eq_run, 0), s_eq[w2]);
    eq_run += s_eq[w2];
  }
  // the lane's first column, recomputed here: held from the start, the compiler would keep
  // every column index of the walk in its own register all along
  int j0 = c0 + lane;
  asm volatile("" : "+v"(j0));
  // stores through a view of the row's k outputs: a lane that keeps nothing stores past it
  // and is dropped, so the walk has no branches on lanes (exactly k keys are kept)
  const __amdgpu_buffer_rsrc_t dst = buffer_view(o, 4u * (uint32_t)k);
  if (n_eq == need_t) {  // every key equal to T is kept (T is usually one key)
#pragma unroll
    for (int u = 0; u < R; u++) {
      if (u < ns) {
        const bool keep = key[u] >= T;
        const uint64_t km = __ballot(keep);
        const uint32_t off = keep ? 4u * (uint32_t)(out_base + (int)lanes_below(km)) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(j0 + 64 * u), dst, (int)off, 0, 0);
        out_base += __popcll(km);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < R; u++) {
      if (u < ns) {
        const bool is_eq = key[u] == T;
        const uint64_t em = __ballot(is_eq);
        const bool keep = key[u] > T || (is_eq && eq_run + (int)lanes_below(em) < need_t);
        const uint64_t km = __ballot(keep);
        const uint32_t off = keep ? 4u * (uint32_t)(out_base + (int)lanes_below(km)) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(j0 + 64 * u), dst, (int)off, 0, 0);
        out_base += __popcll(km);
        eq_run += __popcll(em);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Long rows (decode at long context: few rows of 10^5 .. 10^6 keys). One workgroup per row
// would be bound by one CU's ALUs and memory port, so each row is cut into chunks of kChunk
// keys, one workgroup each, and the selection is a radix select over the key bits in
// launches ordered by the stream (two when the decode scorer has already filled the digit-1
// histograms):
//   hist     histogram of digit 1 (key bits 31..20) of every chunk, merged into the row's
//            histogram with one atomic per occupied bin (after a fill kernel clears it);
//   collect  every chunk finds the bin b1 that holds the row's k-th largest key, counts its
//            keys above b1 ("sure") and writes its keys in b1 ("candidates") into its own
//            region of the workspace in column order, with both counts and b1;
//   emit     every chunk again: it reads the counts and candidates of all the row's chunks
//            (into registers: group cc of threads holds chunk cc's) and resolves from them,
//            with LDS histograms over the candidates (key bits 19..8, then 7..0 unless T's
//            bin of bits 19..8 is taken whole, as it is when it holds one candidate), the
//            row's k-th largest key T and how many keys equal to T are kept (those of the
//            lowest columns). Its offset in the output is the number of kept keys of the
//            earlier chunks (their sure keys, their candidates above T and their share of the
//            keys equal to T), which the same histograms count when they are restricted to
//            the earlier chunks' candidates; it re-reads its own logits and writes its kept
//            columns in ascending order. Every chunk of a row resolves T for itself, so no
//            workgroup waits for another, and it zeroes its share of the row's digit-1
//            histogram for the next call.
// Each step after the loads is a barrier-separated phase of about half a microsecond, so
// the emit kernel keeps them few: the counts' sums share the first histogram's barrier, the
// two histograms' scans share one, and the candidates never go through LDS. (One launch
// where the last chunk of a row to finish selects, after a device-wide counter, measured
// slower: the stores and loads that make the lists visible across the chip's L2s, and the
// counter's atomics, cost more than the launch they save.)
// The candidates of a row are the keys of one digit-1 bin, an eighth of an octave of logit
// values: a few thousand at most on the decode workloads, read by every chunk of the row in
// one round of loads (more are read in further rounds). Device-wide atomics on one cache
// line serialize, so the histogram merge sends one atomic per occupied bin.
// Chunk workgroups of 512 threads (8 keys each).
constexpr int kLongThreads = 512;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kChunk = 4096;
constexpr int kPerThread = kChunk / kLongThreads;  // 8
constexpr int kWaveCols = kChunk / kLongWaves;      // columns of a chunk held by one wave
constexpr int kBins = 4096;                         // 12-bit digits
constexpr int64_t kLongMaxLen = 1 << 20;
constexpr int kMaxChunks = (int)(kLongMaxLen / kChunk);
static_assert(kMaxChunks <= kLongThreads, "the emit kernel gives every chunk of a row at least one thread");
static_assert(kBins == kHistBins, "the digit-1 histograms are the row histograms the decode scorer fills");
constexpr int kCandPer = 16;    // candidate slots of its chunk a thread of the emit kernel reads at once
constexpr int kCountWords = 4;  // per chunk: sure count, candidate count, b1, unused

// Workspace words: the row histograms of digit 1 first (used when the decode scorer has not
// filled them), then per row the chunks' counts and the chunks' candidate regions. A call
// writes each word before it reads it, so the workspace may hold anything when a call
// starts (another call's lists, of another shape, included).
struct LongWs {
  int64_t hist1, counts, ckey, words;
  __host__ __device__ LongWs(int rows, int64_t max_len) {
    const int64_t chunks = (max_len + kChunk - 1) / kChunk;
    const int64_t cap = chunks * kChunk;
    hist1 = 0;
    counts = hist1 + (int64_t)rows * kBins;
    ckey = counts + (int64_t)rows * kCountWords * chunks;
    words = ckey + (int64_t)rows * cap;
  }
};

__device__ __forceinline__ int64_t clamped_len(const int32_t *row_len, int r, int64_t max_len) {
  const int64_t len = row_len[r];
  return len < 0 ? 0 : (len > max_len ? max_len : len);
}

__global__ void zero_fill_kernel(uint4 *p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(kLongThreads) void topk_hist_kernel(const float *__restrict__ logits, int64_t ld,
                                                                const int32_t *__restrict__ row_len,
                                                                int64_t max_len, int k, uint32_t *__restrict__ h1) {
  __shared__ uint32_t h[kBins];
  const int r = blockIdx.y, tid = threadIdx.x;
  const int64_t len = clamped_len(row_len, r, max_len);
  const int64_t start = (int64_t)blockIdx.x * kChunk;
  if (len <= k || start >= len) return;
  const float *row = logits + r * ld;
  const int64_t end = min(len, start + kChunk);
  float v[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    const int64_t j = start + u * kLongThreads + tid;
    v[u] = j < end ? row[j] : 0.f;
  }
  for (int i = tid; i < kBins; i += kLongThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPerThread; u++) hist_put(h, order_key(v[u]) >> 20, start + u * kLongThreads + tid < end);
  __syncthreads();
  uint32_t *g = h1 + (int64_t)r * kHistBins;  // occupied bins only, one atomic each
  for (int b = tid; b < kBins; b += kLongThreads) {
    const uint32_t c = h[b];
    if (c) atomicAdd(&g[hist_slot(b)], c);
  }
}

__global__ __launch_bounds__(kLongThreads) void topk_collect_kernel(const float *__restrict__ logits, int64_t ld,
                                                                   const int32_t *__restrict__ row_len,
                                                                   int64_t max_len, int k, uint32_t *__restrict__ ws,
                                                                   int rows, const uint32_t *__restrict__ h1) {
  __shared__ uint32_t s_h[kBins];
  __shared__ int s_scan[kLongWaves];
  __shared__ int s_bin;
  __shared__ uint32_t s_ws[kLongWaves], s_wc[kLongWaves];
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t start = (int64_t)c * kChunk;
  // Every load goes out before the row length is known (a second memory round trip
  // otherwise): the chunk's logits (columns clamped into the row; those past its length are
  // masked below) and the row's digit-1 histogram, read in its slot order (whole lines).
  // Wave wv holds the chunk's columns [kWaveCols wv, kWaveCols (wv + 1)) in 64-column steps,
  // so wave-major order is column order.
  const float *row = logits + r * ld;
  float lv[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; u++) lv[u] = row[min(start + kWaveCols * wv + 64 * u + lane, max_len - 1)];
  static_assert(kBins / 4 == 2 * kLongThreads, "two 16-byte histogram reads a thread");
  const uint4 *gh = reinterpret_cast<const uint4 *>(h1 + (int64_t)r * kHistBins);
  const uint4 hv0 = gh[tid], hv1 = gh[tid + kLongThreads];
  // A chunk past the row's length, or of a row of at most k keys (left to the emit kernel),
  // runs through with no key counted and writes nothing: an early return here would let the
  // compiler move the loads above behind the length's round trip.
  const int64_t len = clamped_len(row_len, r, max_len);
  const bool active = len > k && start < len;
  const LongWs L(rows, max_len);
  const int64_t chunks = (max_len + kChunk - 1) / kChunk;
  const int64_t cap = chunks * kChunk;
  const int64_t end = active ? min(len, start + kChunk) : start;
  uint32_t key[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; u++) key[u] = order_key(lv[u]);
  // the histogram goes to LDS in slot order and is taken in bin order
  reinterpret_cast<uint4 *>(s_h)[tid] = hv0;
  reinterpret_cast<uint4 *>(s_h)[tid + kLongThreads] = hv1;
  if (tid == 0) s_bin = 0;  // published by the scan's barriers
  __syncthreads();
  {
    constexpr int kPer = kBins / kLongThreads;
    uint32_t cnt[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) cnt[i] = s_h[hist_slot(kPer * tid + i)];
#pragma unroll
    for (int i = 0; i < kPer; i++) sum += (int)cnt[i];
    int tot;
    const int incl = block_prefix_sum<kLongThreads>(sum, s_scan, tot);
    int acc = tot - incl + sum;  // keys in bins >= kPer*tid
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      if (acc >= k && acc - (int)cnt[i] < k) s_bin = kPer * tid + i;
      acc -= (int)cnt[i];
    }
    __syncthreads();
  }
  const uint32_t bin1 = (uint32_t)s_bin;
  uint64_t mc[kPerThread];
  uint32_t n_s = 0, n_c = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    const bool ok = start + kWaveCols * wv + 64 * u + lane < end;
    const uint32_t d = key[u] >> 20;
    n_s += (uint32_t)__popcll(__ballot(ok && d > bin1));
    mc[u] = __ballot(ok && d == bin1);
    n_c += (uint32_t)__popcll(mc[u]);
  }
  if (lane == 0) {
    s_ws[wv] = n_s;
    s_wc[wv] = n_c;
  }
  __syncthreads();
  uint32_t bc = 0, ts = 0, tc = 0;
  for (int w2 = 0; w2 < kLongWaves; w2++) {
    if (w2 < wv) bc += s_wc[w2];
    ts += s_ws[w2];
    tc += s_wc[w2];
  }
  uint32_t *ckey = ws + L.ckey + (int64_t)r * cap + start;
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    if ((mc[u] >> lane) & 1ull) ckey[bc + lanes_below(mc[u])] = key[u];
    bc += (uint32_t)__popcll(mc[u]);
  }
  if (tid == 0 && active) {
    uint32_t *cnt = ws + L.counts + ((int64_t)r * chunks + c) * kCountWords;
    cnt[0] = ts;
    cnt[1] = tc;
    cnt[2] = bin1;
  }
}

// Inclusive prefix sums of a and b over the workgroup's threads, with one barrier; ta and tb
// get the totals. s_w (two words a wave) must not be reused before another barrier.
template <int NT>
__device__ __forceinline__ void block_prefix_sum2(int &a, int &b, int *s_w, int &ta, int &tb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  a = wave_prefix_sum(a);
  b = wave_prefix_sum(b);
  if (lane == 63) {
    s_w[wv] = a;
    s_w[NT / 64 + wv] = b;
  }
  __syncthreads();
  int ba = 0, bb = 0;
  ta = tb = 0;
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; w2++) {
    const int x = s_w[w2], y = s_w[NT / 64 + w2];
    ba += w2 < wv ? x : 0;
    bb += w2 < wv ? y : 0;
    ta += x;
    tb += y;
  }
  a += ba;
  b += bb;
}

__global__ __launch_bounds__(kLongThreads) void topk_emit_kernel(const float *__restrict__ logits, int64_t ld,
                                                                const int32_t *__restrict__ row_len,
                                                                int64_t max_len, int k,
                                                                const uint32_t *__restrict__ ws, int rows,
                                                                uint32_t *__restrict__ h1, int32_t *__restrict__ out,
                                                                int64_t out_ld) {
  // the candidates' digit 2 (key bits 19..8) and low byte: of all chunks, and of the chunks
  // before this one
  __shared__ __attribute__((aligned(16))) uint32_t s_h2[kBins], s_h2b[kBins];
  __shared__ __attribute__((aligned(16))) uint32_t s_h3[256], s_h3b[256];
  __shared__ int s_red[4 * kLongWaves];
  __shared__ int s_scan[2 * kLongWaves];
  __shared__ int s_sel[8];
  __shared__ uint32_t s_we[kLongWaves], s_wk[kLongWaves];
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunks = (int)((max_len + kChunk - 1) / kChunk);
  const LongWs L(rows, max_len);
  const int64_t cap = (int64_t)chunks * kChunk;
  // Everything is requested at once, before the row length is known (a second memory round
  // trip otherwise): the counts of every chunk of the row and the first candidates of every
  // chunk's region (group cc of tpc threads holds chunk cc's slots t0 + tpc u, u < kCandPer,
  // in one wave or part of one; slots past a chunk's count hold stale words and are dropped
  // once the counts are in), and this chunk's logits (columns clamped into the row, those
  // past its length masked).
  const int tpc_log = 9 - (32 - __clz(chunks - 1));  // tpc: the power of two <= kLongThreads / chunks
  const int tpc = 1 << tpc_log;
  const int cc = tid >> tpc_log, t0 = tid & (tpc - 1);
  const int ccq = min(cc, chunks - 1);
  const uint32_t *cw = ws + L.counts + (int64_t)r * chunks * kCountWords;
  const uint32_t ns_raw = cw[ccq * kCountWords], nc_raw = cw[ccq * kCountWords + 1];
  const uint32_t b1 = cw[2] & (kBins - 1);  // chunk 0 holds keys of every long row
  const uint32_t *ckc = ws + L.ckey + (int64_t)r * cap + (int64_t)ccq * kChunk;
  uint32_t cand[kCandPer];
#pragma unroll
  for (int u = 0; u < kCandPer; u++) cand[u] = ckc[min(t0 + u * tpc, kChunk - 1)];  // (slots past kChunk unused)
  const int64_t start = (int64_t)c * kChunk;
  const float *row = logits + r * ld;
  float lv[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; u++) lv[u] = row[min(start + kWaveCols * wv + 64 * u + lane, max_len - 1)];
  asm volatile("" ::: "memory");  // (keeps the length check, and its wait, behind the loads)
  // the histograms are cleared while the loads are in flight
  static_assert(kBins / 4 == 2 * kLongThreads, "two 16-byte stores a thread and histogram");
  reinterpret_cast<uint4 *>(s_h2)[tid] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4 *>(s_h2)[tid + kLongThreads] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4 *>(s_h2b)[tid] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4 *>(s_h2b)[tid + kLongThreads] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 64) {
    reinterpret_cast<uint4 *>(s_h3)[tid] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4 *>(s_h3b)[tid] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const int64_t len = clamped_len(row_len, r, max_len);
  // the collect kernel has read the row's digit-1 histogram: this chunk's share of it is
  // zeroed for the next call
  {
    const int per = (kHistBins / 4 + chunks - 1) / chunks;
    uint4 *g = reinterpret_cast<uint4 *>(h1 + (int64_t)r * kHistBins);
    const int i1 = min(kHistBins / 4, (c + 1) * per);
    for (int i = c * per + tid; i < i1; i += kLongThreads) g[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  int32_t *o = out + r * out_ld;
  if (len <= k) {  // a row of at most k keys keeps them all (the collect kernel left it alone)
    const int64_t span = ((int64_t)k + chunks - 1) / chunks;
    const int64_t j1 = min((int64_t)k, (c + 1) * span);
    for (int64_t j = c * span + tid; j < j1; j += kLongThreads) o[j] = j < len ? (int32_t)j : -1;
    return;
  }
  const int used = (int)((len + kChunk - 1) / kChunk);  // chunks that hold keys of this row
  if (c >= used) return;
  const bool live = cc < used, before = cc < c;  // chunk cc holds keys; it precedes this one
  const int64_t end = min(len, start + kChunk);
  const int nvalid = (int)(end - start);  // keys of this chunk
  uint32_t key[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; u++) key[u] = order_key(lv[u]);
  const int nc = live ? (int)min(nc_raw, (uint32_t)kChunk) : 0;
  const int ns = live ? (int)min(ns_raw, (uint32_t)kChunk) : 0;
  const int E = kCandPer * tpc;  // slots of a chunk held in registers
  // f(v) for every candidate v of chunk cc held by this thread: the registers, then (chunks
  // with more candidates than slots, rare) the rest from the workspace
  auto for_cands = [&](auto f) {
#pragma unroll
    for (int u = 0; u < kCandPer; u++)
      if (t0 + u * tpc < nc) f(cand[u]);
    for (int i = E + t0; i < nc; i += tpc) f(ckc[i]);
  };
  // The sure keys and candidates of the row and of the chunks before this one (group
  // leaders' counts summed over the workgroup), and the candidates' digit 2 (plain LDS
  // atomics: their digits are nearly all distinct, and rows of ties only cost conflicts),
  // under one barrier.
  {
    const bool lead = t0 == 0;
    const int a0 = wave_sum(lead ? ns : 0), a1 = wave_sum(lead && before ? ns : 0);
    const int a2 = wave_sum(lead ? nc : 0), a3 = wave_sum(lead && before ? nc : 0);
    if (lane == 0) {
      s_red[wv] = a0;
      s_red[kLongWaves + wv] = a1;
      s_red[2 * kLongWaves + wv] = a2;
      s_red[3 * kLongWaves + wv] = a3;
    }
    for_cands([&](uint32_t v) {
      const uint32_t d = (v >> 8) & (kBins - 1);
      atomicAdd(&s_h2[d], 1u);
      if (before) atomicAdd(&s_h2b[d], 1u);
    });
    __syncthreads();
  }
  int sure_all = 0, sure_bef = 0, n_cand = 0, cand_bef = 0;
#pragma unroll
  for (int w2 = 0; w2 < kLongWaves; w2++) {
    sure_all += s_red[w2];
    sure_bef += s_red[kLongWaves + w2];
    n_cand += s_red[2 * kLongWaves + w2];
    cand_bef += s_red[3 * kLongWaves + w2];
  }
  const int need = k - sure_all;  // candidates to take after the sure keys
  uint32_t T;                     // the k-th largest key, or a bound that selects the same keys
  bool keep_eq;                   // every key equal to T is kept (else the lowest-column rem_all)
  int rem_all = 0;                // keys equal to T that are kept, when not all are
  int eq_bef = 0;                 // keys equal to T in earlier chunks
  int kept_bef;                   // candidates of earlier chunks that are kept (ties included)
  if (need <= 0) {  // more sure keys than k (a histogram of other logits): no candidate
    T = (b1 << 20) | 0xFFFFFu;
    keep_eq = false;
    kept_bef = 0;
  } else if (need >= n_cand) {  // every candidate (short of k when fewer)
    T = b1 << 20;
    keep_eq = true;
    kept_bef = cand_bef;
  } else {
    {  // the digit-2 bin b2 of the need-th largest candidate
      constexpr int kPer = kBins / kLongThreads;
      static_assert(kPer == 8, "two 16-byte reads a thread");
      const uint4 lo = reinterpret_cast<const uint4 *>(s_h2)[2 * tid];
      const uint4 hi = reinterpret_cast<const uint4 *>(s_h2)[2 * tid + 1];
      const uint4 lob = reinterpret_cast<const uint4 *>(s_h2b)[2 * tid];
      const uint4 hib = reinterpret_cast<const uint4 *>(s_h2b)[2 * tid + 1];
      const int cnt[kPer] = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int cnb[kPer] = {(int)lob.x, (int)lob.y, (int)lob.z, (int)lob.w,
                             (int)hib.x, (int)hib.y, (int)hib.z, (int)hib.w};
      int sum = 0, sumb = 0;
#pragma unroll
      for (int i = 0; i < kPer; i++) {
        sum += cnt[i];
        sumb += cnb[i];
      }
      int incl = sum, inclb = sumb, tot, totb;
      block_prefix_sum2<kLongThreads>(incl, inclb, s_scan, tot, totb);
      int acc = tot - incl + sum, accb = totb - inclb + sumb;  // in bins >= kPer*tid
#pragma unroll
      for (int i = 0; i < kPer; i++) {
        acc -= cnt[i];
        accb -= cnb[i];
        if (acc + cnt[i] >= need && acc < need) {
          s_sel[0] = kPer * tid + i;
          s_sel[1] = need - acc;  // candidates of b2 still to take
          s_sel[2] = accb;        // earlier chunks' candidates above b2
          s_sel[3] = cnt[i];      // candidates in b2
          s_sel[4] = cnb[i];      // earlier chunks' candidates in b2
        }
      }
      __syncthreads();
    }
    const uint32_t hi20 = (b1 << 12) | (uint32_t)s_sel[0];
    const int need2 = s_sel[1];
    if (need2 == s_sel[3]) {  // b2 is kept whole (the usual case: it holds one candidate)
      T = hi20 << 8;
      keep_eq = true;
      kept_bef = s_sel[2] + s_sel[4];
    } else {  // its low byte
      const int above_b2 = s_sel[2];
      for_cands([&](uint32_t v) {
        if ((v >> 8) == hi20) {
          atomicAdd(&s_h3[v & 255u], 1u);
          if (before) atomicAdd(&s_h3b[v & 255u], 1u);
        }
      });
      __syncthreads();
      if (wv == 0) {  // 256 bins, four a lane
        const uint4 q = reinterpret_cast<const uint4 *>(s_h3)[lane];
        const uint4 qb = reinterpret_cast<const uint4 *>(s_h3b)[lane];
        const int cnt[4] = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
        const int cnb[4] = {(int)qb.x, (int)qb.y, (int)qb.z, (int)qb.w};
        const int sum = cnt[0] + cnt[1] + cnt[2] + cnt[3], sumb = cnb[0] + cnb[1] + cnb[2] + cnb[3];
        const int incl = wave_prefix_sum(sum), inclb = wave_prefix_sum(sumb);
        int acc = __builtin_amdgcn_readlane(incl, 63) - incl + sum;  // b2's candidates in bins >= 4 lane
        int accb = __builtin_amdgcn_readlane(inclb, 63) - inclb + sumb;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          acc -= cnt[i];
          accb -= cnb[i];
          if (acc + cnt[i] >= need2 && acc < need2) {
            s_sel[5] = 4 * lane + i;
            s_sel[6] = need2 - acc;  // keys equal to T that are kept
            s_sel[7] = accb;         // earlier chunks' candidates of b2 above T
            s_red[0] = cnb[i];       // earlier chunks' keys equal to T
            s_red[1] = cnt[i];       // keys equal to T
          }
        }
      }
      __syncthreads();
      T = (hi20 << 8) | (uint32_t)s_sel[5];
      rem_all = s_sel[6];
      eq_bef = s_red[0];
      keep_eq = rem_all >= s_red[1];
      kept_bef = above_b2 + s_sel[7] + min(eq_bef, rem_all);
    }
  }
  const int total = min(k, need <= 0 ? sure_all : sure_all + min(need, n_cand));
  const int pre = sure_bef + kept_bef;
  // Keys equal to T are ranked by column only where the kept ones stop among them.
  const int rem_c = keep_eq ? 0 : max(0, rem_all - eq_bef);  // this chunk's ties that are kept
  const bool rank_t = rem_c > 0;
  // this chunk's keys equal to T in column order (wave-major), then the kept keys (the
  // predicates are combined without short-circuits, which would branch per key)
  uint64_t me[kPerThread];
  int e_run = 0;
  if (rank_t) {
    uint32_t n_e = 0;
#pragma unroll
    for (int u = 0; u < kPerThread; u++) {
      const bool ok = kWaveCols * wv + 64 * u + lane < nvalid;
      me[u] = __ballot(ok & (key[u] == T));
      n_e += (uint32_t)__popcll(me[u]);
    }
    if (lane == 0) s_we[wv] = n_e;
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < kLongWaves; w2++) e_run += w2 < wv ? (int)s_we[w2] : 0;
  } else {
#pragma unroll
    for (int u = 0; u < kPerThread; u++) me[u] = 0;
  }
  uint64_t mk[kPerThread];
  uint32_t n_k = 0;
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    const bool ok = kWaveCols * wv + 64 * u + lane < nvalid;
    const bool eq = (me[u] >> lane) & 1ull;
    const bool keep =
        ok & ((key[u] > T) | (keep_eq & (key[u] == T)) | (eq & (e_run + (int)lanes_below(me[u]) < rem_c)));
    e_run += (int)__popcll(me[u]);
    mk[u] = __ballot(keep);
    n_k += (uint32_t)__popcll(mk[u]);
  }
  if (lane == 0) s_wk[wv] = n_k;
  __syncthreads();
  int pos = pre;
#pragma unroll
  for (int w2 = 0; w2 < kLongWaves; w2++) pos += w2 < wv ? (int)s_wk[w2] : 0;
#pragma unroll
  for (int u = 0; u < kPerThread; u++) {
    const int at = pos + (int)lanes_below(mk[u]);
    if (((mk[u] >> lane) & 1ull) && at >= 0 && at < k) o[at] = (int32_t)(start + kWaveCols * wv + 64 * u + lane);
    pos += (int)__popcll(mk[u]);
  }
  if (c == used - 1)  // a selection short of k (a histogram of other logits) is padded
    for (int j = max(total, 0) + tid; j < k; j += kLongThreads) o[j] = -1;
}

// ---------------------------------------------------------------------------------------
// Candidate merge for context-parallel decode ("Score a DSA sparse indexer in FP4", DCP
// commit: every rank takes a local top-k over its share of a sequence's pages, the ranks
// exchange (score, index) candidates and a merge top-k reads the exchanged fp32 scores).
// One 1024-thread workgroup per row: the row's candidates are staged in LDS with the range
// of their keys, a 1024-bin histogram spread over that range finds the bin of the k-th best,
// the few candidates in it are ranked by counting (ties to the smaller index; radix select
// when there are many), and the chosen indices are put in ascending order through an LDS
// bitmap over the candidates' index range (8 rows x 8192 candidates, k 2048: 46.1 -> 27.5 us
// a launch), or by a bitonic sort in LDS when that range is too wide or an index repeats.
constexpr int kMergeThreads = 1024;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeMaxCand = 16384;
constexpr int kMergeMaxK = 4096;
constexpr int kMergeBins = 1024;
constexpr int kMergeLds = 150 * 1024;  // dynamic LDS: the lists, the sort buffer, the index bitmap
static_assert(4 * (2 * kMergeMaxCand + 4096) <= kMergeLds, "lists and sort buffer fit");

__host__ __device__ inline int merge_sort_len(int k) {  // smallest power of two >= k
  int p = 1;
  while (p < k) p <<= 1;
  return p;
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(const float *__restrict__ score,
                                                                  const int32_t *__restrict__ index, int64_t ld,
                                                                  int n_cand, int k, int32_t *__restrict__ out,
                                                                  int64_t out_ld, int bm_words) {
  // keys[n_cand], indices[n_cand], sort buffer[merge_sort_len(k)], index bitmap[bm_words]
  extern __shared__ uint32_t lds[];
  __shared__ uint32_t hist[kMergeBins];
  __shared__ uint32_t chosen[kMergeMaxCand / 32];  // chosen candidates of bin b, by position
  __shared__ uint32_t ckey[kShortRank], cpos[kShortRank];
  __shared__ int s_scan[3 * kMergeWaves], s_misc[8];
  __shared__ uint32_t s_red[8 * kMergeWaves];
  __shared__ int s_gathered;  // indices gathered for the sort (block_select uses s_misc[4..6])
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t *keys = lds, *idx = lds + n_cand, *buf = lds + 2 * n_cand;
  const int P2 = merge_sort_len(k);
  uint32_t *bm = buf + P2;
  // stage; an empty slot (index < 0) gets index 0xFFFFFFFF and never counts. All of a
  // thread's loads go out before any is used (slots past n_cand load the last candidate and
  // are dropped): a loop that used each load before the next waited one round trip a slot.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, imin = 0xFFFFFFFFu, imax = 0u;
  int nv = 0;
  constexpr int kStage = kMergeMaxCand / kMergeThreads;  // candidate slots a thread holds
  if (n_cand > 0) {
    int32_t ixv[kStage];
    float scv[kStage];
#pragma unroll
    for (int u = 0; u < kStage; u++) {
      const int64_t c = r * ld + min(tid + u * kMergeThreads, n_cand - 1);
      ixv[u] = index[c];
      scv[u] = score[c];
    }
#pragma unroll
    for (int u = 0; u < kStage; u++) {
      const int c = tid + u * kMergeThreads;
      if (c < n_cand) {
        const int32_t ix = ixv[u];
        const bool ok = ix >= 0;
        const uint32_t key = order_key(scv[u]);
        keys[c] = key;
        idx[c] = ok ? (uint32_t)ix : 0xFFFFFFFFu;
        if (ok) {
          kmin = min(kmin, key);
          kmax = max(kmax, key);
          imin = min(imin, (uint32_t)ix);
          imax = max(imax, (uint32_t)ix);
          nv++;
        }
      }
    }
  }
  for (int i = tid; i < kMergeBins; i += kMergeThreads) hist[i] = 0u;
  for (int i = tid; i < (n_cand + 31) / 32; i += kMergeThreads) chosen[i] = 0u;
  if (tid == 0) {
    s_misc[3] = 0;  // bin-b candidates listed
    s_gathered = 0;
  }
  {  // the block's key and index ranges and valid count: DPP reductions, one LDS exchange
    const int wv = tid >> 6;
    const uint32_t a0 = wave_min_last(kmin), a1 = wave_max_last(kmax);
    const uint32_t a2 = wave_min_last(imin), a3 = wave_max_last(imax);
    const int a4 = wave_prefix_sum(nv);
    if (lane == 63) {
      s_red[8 * wv] = a0;
      s_red[8 * wv + 1] = a1;
      s_red[8 * wv + 2] = a2;
      s_red[8 * wv + 3] = a3;
      s_red[8 * wv + 4] = (uint32_t)a4;
    }
    __syncthreads();
    nv = 0;
#pragma unroll
    for (int w2 = 0; w2 < kMergeWaves; w2++) {
      kmin = min(kmin, s_red[8 * w2]);
      kmax = max(kmax, s_red[8 * w2 + 1]);
      imin = min(imin, s_red[8 * w2 + 2]);
      imax = max(imax, s_red[8 * w2 + 3]);
      nv += (int)s_red[8 * w2 + 4];
    }
  }
  // the chosen indices are put in order through a bitmap over [imin, imax] when it fits LDS
  const int span_words = imin <= imax ? (int)min(((uint64_t)(imax - imin) + 32) / 32, (uint64_t)bm_words + 1) : 0;
  const bool use_bm = span_words > 0 && span_words <= bm_words;
  if (use_bm)
    for (int i = tid; i < span_words; i += kMergeThreads) bm[i] = 0u;
  __syncthreads();
  const int take_n = min(k, nv);
  const int bl = 32 - __clz((int)(kmax - kmin));
  const int sh = bl > 10 ? bl - 10 : 0;
  auto digit = [&](uint32_t key) { return min((key - kmin) >> sh, (uint32_t)(kMergeBins - 1)); };
  uint32_t pre_b = 0, pmask_b = 0;  // T's bin: the bits of key - kmin its keys share
  if (nv > k) {
    for (int c0 = 0; c0 < n_cand; c0 += kMergeThreads) {
      const int c = c0 + tid;
      const bool ok = c < n_cand && idx[c] != 0xFFFFFFFFu;
      hist_put(hist, ok ? digit(keys[c]) : 0u, ok);
    }
    __syncthreads();
    {
      const uint32_t h = hist[tid];  // one bin per thread
      const int acc = block_suffix_sum<kMergeThreads>((int)h, s_scan);
      if (acc >= k && acc - (int)h < k) {
        s_misc[0] = tid;
        s_misc[1] = k - (acc - (int)h);
        s_misc[2] = (int)h;
      }
      __syncthreads();
    }
    // the bits of key - kmin that every key of T's bin shares (pre under pmask); further
    // linear levels of 10 bits over that bin's keys while it is crowded
    uint32_t pre = (uint32_t)s_misc[0] << sh;
    uint32_t pmask = top_bits_mask(32 - sh);
    int need = s_misc[1], nb = s_misc[2];
    int sc = sh;
    while (nb > kShortRank && sc > 0) {
      const int s2 = sc > 10 ? sc - 10 : 0;
      const uint32_t dm = (1u << (sc - s2)) - 1u;
      __syncthreads();  // every thread has read s_misc and the last level's histogram
      hist[tid] = 0u;
      __syncthreads();
      for (int c0 = 0; c0 < n_cand; c0 += kMergeThreads) {
        const int c = c0 + tid;
        const bool ok = c < n_cand && idx[c] != 0xFFFFFFFFu && ((keys[c] - kmin) & pmask) == pre;
        hist_put(hist, ok ? ((keys[c] - kmin) >> s2) & dm : 0u, ok);
      }
      __syncthreads();
      {
        const uint32_t h = hist[tid];
        const int acc = block_suffix_sum<kMergeThreads>((int)h, s_scan);
        if (acc >= need && acc - (int)h < need) {
          s_misc[0] = tid;
          s_misc[1] = need - (acc - (int)h);
          s_misc[2] = (int)h;
        }
        __syncthreads();
      }
      pre |= (uint32_t)s_misc[0] << s2;
      pmask |= dm << s2;
      need = s_misc[1];
      nb = s_misc[2];
      sc = s2;
    }
    pre_b = pre;
    pmask_b = pmask;
    auto in_bin = [&](int c) { return idx[c] != 0xFFFFFFFFu && ((keys[c] - kmin) & pmask) == pre; };
    if (nb <= kShortRank) {  // the bin's keys ranked by counting
      for (int c0 = 0; c0 < n_cand; c0 += kMergeThreads) {
        const int c = c0 + tid;
        const bool in_b = c < n_cand && in_bin(c);
        const uint64_t m = __ballot(in_b);
        if (m) {
          int at = 0;
          if (lane == 0) at = atomicAdd(&s_misc[3], __popcll(m));
          at = __builtin_amdgcn_readfirstlane(at) + (int)lanes_below(m);
          if (in_b && at < nb) {
            ckey[at] = keys[c];
            cpos[at] = (uint32_t)c;
          }
        }
      }
      __syncthreads();
      if (tid < nb) {
        const uint32_t key = ckey[tid], ix = idx[cpos[tid]];
        int rank = 0;
        for (int g = 0; g < nb; g++) {
          const uint32_t kg = ckey[g];
          rank += (kg > key || (kg == key && idx[cpos[g]] < ix)) ? 1 : 0;
        }
        if (rank < need) atomicOr(&chosen[cpos[tid] >> 5], 1u << (cpos[tid] & 31));
      }
    } else {  // a crowded bin of one value T: its need smallest indices
      const uint32_t T = kmin + pre;
      int rem2 = need, n_eq2 = 0;
      const uint32_t sel = block_select<kMergeThreads>(
          n_cand,
          [&](int c) { return (idx[c] != 0xFFFFFFFFu && keys[c] == T) ? (0x7FFFFFFFu - idx[c]) : 0xFFFFFFFFu; },
          0u, 0x80000000u, 31, &rem2, &n_eq2, hist, s_scan, s_misc + 4);
      const uint32_t cut = 0x7FFFFFFFu - sel;  // keys equal to T with index <= cut are kept
      for (int c = tid; c < n_cand; c += kMergeThreads)
        if (idx[c] != 0xFFFFFFFFu && keys[c] == T && idx[c] <= cut) atomicOr(&chosen[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
  }
  // gather the chosen indices (any order), pad to a power of two, sort ascending
  for (int c0 = 0; c0 < n_cand; c0 += kMergeThreads) {
    const int c = c0 + tid;
    bool t = c < n_cand && idx[c] != 0xFFFFFFFFu;
    if (t && nv > k) t = ((keys[c] - kmin) & pmask_b) > pre_b || ((chosen[c >> 5] >> (c & 31)) & 1u);
    const uint64_t m = __ballot(t);
    if (m) {
      int at = 0;
      if (lane == 0) at = atomicAdd(&s_gathered, __popcll(m));
      at = __builtin_amdgcn_readfirstlane(at) + (int)lanes_below(m);
      if (t && at < take_n) buf[at] = idx[c];
      if (t && use_bm) atomicOr(&bm[(idx[c] - imin) >> 5], 1u << ((idx[c] - imin) & 31));
    }
  }
  __syncthreads();
  if (use_bm) {
    // indices in ascending order from the bitmap: each thread owns a contiguous run of words;
    // repeated indices share a bit, and then the sort below runs instead
    const int per = (span_words + kMergeThreads - 1) / kMergeThreads;
    const int w0 = min(span_words, tid * per), w1 = min(span_words, w0 + per);
    int bits = 0;
    for (int i = w0; i < w1; i++) bits += __popc(bm[i]);
    const int suffix = block_suffix_sum<kMergeThreads>(bits, s_scan);
    if (tid == 0) s_misc[7] = suffix;
    __syncthreads();
    const int total = s_misc[7];
    if (total == take_n) {
      int32_t *o = out + r * out_ld;
      int pos = total - suffix;
      for (int i = w0; i < w1; i++) {
        uint32_t m = bm[i];
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1;
          if (pos < k) o[pos] = (int32_t)(imin + 32u * (uint32_t)i + (uint32_t)bit);
          pos++;
        }
      }
      for (int j = total + tid; j < k; j += kMergeThreads) o[j] = -1;
      return;
    }
  }
  for (int i = take_n + tid; i < P2; i += kMergeThreads) buf[i] = 0xFFFFFFFFu;
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2; i += kMergeThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t a = buf[i], c = buf[j];
          const bool up = (i & size) == 0;
          if ((a > c) == up) {
            buf[i] = c;
            buf[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  int32_t *o = out + r * out_ld;
  for (int j = tid; j < k; j += kMergeThreads) o[j] = j < take_n ? (int32_t)buf[j] : -1;
}

}  // namespace ifp4

using namespace ifp4;

static bool use_long_path(int64_t max_len, int32_t k) {
  return max_len > kShortMax && max_len <= kLongMaxLen && k < max_len;
}

extern "C" int64_t indexer_topk_workspace_bytes(int32_t n_rows, int64_t max_len, int32_t k) {
  if (n_rows < 0 || max_len < 0 || k <= 0) return -1;
  if (!use_long_path(max_len, k)) return 0;
  return 4 * LongWs(n_rows, max_len).words;
}

// Checks and launches of indexer_topk, on a workspace the caller (or the scratch array below)
// provides; `ws_what` names it in messages.
static int topk_check(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                      int64_t max_len, int32_t k, const int32_t *topk_idx, int64_t topk_ld, int64_t ws_bytes,
                      const char *ws_what, const uint32_t *row_hist) {
  if (k <= 0 || n_rows < 0 || max_len < 0)
    return fail(INDEXER_FP4_EINVAL, "topk: k=%d must be > 0, n_rows=%d >= 0, max_len=%lld >= 0", k, n_rows,
                (long long)max_len);
  if (max_len > logits_ld)
    return fail(INDEXER_FP4_EINVAL, "topk: max_len=%lld exceeds logits_ld=%lld", (long long)max_len,
                (long long)logits_ld);
  if (max_len > kLongMaxLen)
    return fail(INDEXER_FP4_EINVAL, "topk: max_len=%lld above the supported %lld", (long long)max_len,
                (long long)kLongMaxLen);
  if (topk_ld < k) return fail(INDEXER_FP4_ENOSPC, "topk: topk_ld=%lld < k=%d", (long long)topk_ld, k);
  const int64_t need = indexer_topk_workspace_bytes(n_rows, max_len, k);
  if (ws_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "topk: n_rows=%d, max_len=%lld, k=%d need %lld bytes of %s, which has %lld",
                n_rows, (long long)max_len, k, (long long)need, ws_what, (long long)ws_bytes);
  if (n_rows > 0 && (!logits || !row_len || !topk_idx)) return fail(INDEXER_FP4_EINVAL, "topk: NULL pointer");
  if ((uintptr_t)row_hist % 16 != 0) return fail(INDEXER_FP4_EINVAL, "topk: row_hist must be 16-byte aligned");
  return INDEXER_FP4_OK;
}

static int topk_impl(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                     int64_t max_len, int32_t k, int32_t *topk_idx, int64_t topk_ld, void *workspace,
                     int64_t ws_bytes, const char *ws_what, uint32_t *row_hist, void *stream) {
  int rc = topk_check(logits, logits_ld, n_rows, row_len, max_len, k, topk_idx, topk_ld, ws_bytes, ws_what,
                      row_hist);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  if (n_rows == 0) return INDEXER_FP4_OK;
  hipStream_t st = (hipStream_t)stream;
  // the short-row kernels size their dynamic LDS from max_len; raise the launch limit once
  static bool lds_set = false;
  if (!lds_set) {
    hipError_t e = hipFuncSetAttribute((const void *)topk_row_kernel<256>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(4 * kShortMax));
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void *)topk_row_kernel<512>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(4 * kShortMax));
    if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "topk: hipFuncSetAttribute: %s", hipGetErrorString(e));
    lds_set = true;
  }
  if (max_len <= kRegMax) {
    if (n_rows <= kRegWideRows)
      hipLaunchKernelGGL((topk_reg_kernel<512, 12>), dim3(n_rows), dim3(512), 0, st, logits, logits_ld, row_len,
                         max_len, k, row_hist, topk_idx, topk_ld);
    else
      hipLaunchKernelGGL((topk_reg_kernel<256, 24>), dim3(n_rows), dim3(256), 0, st, logits, logits_ld, row_len,
                         max_len, k, row_hist, topk_idx, topk_ld);
    return launch_status("topk");
  }
  if (!use_long_path(max_len, k)) {
    // rows of at most kShortMax keys, or k >= max_len (every row keeps all its keys and
    // the kernel returns before staging anything)
    const size_t lds = max_len <= kShortMax ? (size_t)(4 * max_len) : 0;
    if (n_rows <= kWideRows)
      hipLaunchKernelGGL(topk_row_kernel<512>, dim3(n_rows), dim3(512), lds, st, logits, logits_ld, row_len,
                         max_len, k, row_hist, topk_idx, topk_ld);
    else
      hipLaunchKernelGGL(topk_row_kernel<256>, dim3(n_rows), dim3(256), lds, st, logits, logits_ld, row_len,
                         max_len, k, row_hist, topk_idx, topk_ld);
    return launch_status("topk");
  }
  if (!workspace || (uintptr_t)workspace % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "topk: rows up to %lld keys need a 16-byte aligned workspace", (long long)max_len);
  uint32_t *ws = (uint32_t *)workspace;
  const unsigned chunks = (unsigned)((max_len + kChunk - 1) / kChunk);
  // the digit-1 histograms: filled by the decode scorer, or built here in the workspace
  uint32_t *h1 = row_hist ? row_hist : ws + LongWs(n_rows, max_len).hist1;
  if (!row_hist) {  // cleared first: the workspace may hold another call's lists there
    const int64_t n16 = (int64_t)n_rows * kBins / 4;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)std::min<int64_t>(1024, (n16 + 255) / 256)), dim3(256), 0, st,
                       (uint4 *)h1, n16);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(chunks, n_rows), dim3(kLongThreads), 0, st, logits, logits_ld, row_len,
                       max_len, k, h1);
  }
  hipLaunchKernelGGL(topk_collect_kernel, dim3(chunks, n_rows), dim3(kLongThreads), 0, st, logits, logits_ld,
                     row_len, max_len, k, ws, n_rows, h1);
  hipLaunchKernelGGL(topk_emit_kernel, dim3(chunks, n_rows), dim3(kLongThreads), 0, st, logits, logits_ld, row_len,
                     max_len, k, ws, n_rows, h1, topk_idx, topk_ld);
  return launch_status("topk");
}

extern "C" int indexer_topk(const float *logits, int64_t logits_ld, int32_t n_rows, const int32_t *row_len,
                            int64_t max_len, int32_t k, int32_t *topk_idx, int64_t topk_ld, void *workspace,
                            int64_t ws_bytes, uint32_t *row_hist, void *stream) {
  clear_error();
  return topk_impl(logits, logits_ld, n_rows, row_len, max_len, k, topk_idx, topk_ld, workspace, ws_bytes,
                   "workspace", row_hist, stream);
}

// ---------------------------------------------------------------------------------------
// indexer_topk_noalloc: the same selection with the long-row workspace in a fixed array of
// device memory that the library owns, for callers that cannot allocate. Each device holds
// its own copy of the array; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name in host code is a
// host-side stand-in, not a device address). As with a caller's workspace, a call writes
// each word of the array it reads first, so the array needs no clearing.
constexpr int64_t kScratchBytes = INDEXER_TOPK_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint32_t scratch[kScratchBytes / 4];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64];  // per device: the array's device address, once looked up

extern "C" int indexer_topk_noalloc(const float *logits, int64_t logits_ld, int32_t n_rows,
                                    const int32_t *row_len, int64_t max_len, int32_t k, int32_t *topk_idx,
                                    int64_t topk_ld, uint32_t *row_hist, void *stream) {
  clear_error();
  int rc = topk_check(logits, logits_ld, n_rows, row_len, max_len, k, topk_idx, topk_ld, kScratchBytes,
                      "the fixed scratch array", row_hist);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "topk_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  void *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess || !g_scratch_ptr[dev]) {
        g_scratch_ptr[dev] = nullptr;
        return fail(INDEXER_FP4_EHIP, "topk_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  return topk_impl(logits, logits_ld, n_rows, row_len, max_len, k, topk_idx, topk_ld, ptr, kScratchBytes,
                   "scratch", row_hist, stream);
}

extern "C" int indexer_topk_merge(const float *cand_score, const int32_t *cand_index, int64_t cand_ld,
                                  int32_t n_rows, int32_t n_cand, int32_t k, int32_t *topk_idx, int64_t topk_ld,
                                  void *stream) {
  clear_error();
  if (k <= 0 || k > kMergeMaxK || n_rows < 0 || n_cand < 0 || n_cand > kMergeMaxCand)
    return fail(INDEXER_FP4_EINVAL, "topk_merge: k=%d in 1..%d, n_rows=%d >= 0, n_cand=%d in 0..%d", k, kMergeMaxK,
                n_rows, n_cand, kMergeMaxCand);
  if (cand_ld < n_cand)
    return fail(INDEXER_FP4_EINVAL, "topk_merge: cand_ld=%lld < n_cand=%d", (long long)cand_ld, n_cand);
  if (topk_ld < k) return fail(INDEXER_FP4_ENOSPC, "topk_merge: topk_ld=%lld < k=%d", (long long)topk_ld, k);
  if (n_rows > 0 && (!topk_idx || (n_cand > 0 && (!cand_score || !cand_index))))
    return fail(INDEXER_FP4_EINVAL, "topk_merge: NULL pointer");
  int rc = check_device();
  if (rc) return rc;
  if (n_rows == 0) return INDEXER_FP4_OK;
  static bool lds_set = false;
  if (!lds_set) {
    const hipError_t e = hipFuncSetAttribute((const void *)topk_merge_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kMergeLds);
    if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "topk_merge: hipFuncSetAttribute: %s", hipGetErrorString(e));
    lds_set = true;
  }
  const int64_t fixed = 4 * ((int64_t)2 * n_cand + merge_sort_len(k));
  const int bm_words = (int)((kMergeLds - fixed) / 4);  // the rest of the LDS budget
  const size_t lds = (size_t)fixed + 4 * (size_t)bm_words;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n_rows), dim3(kMergeThreads), lds, (hipStream_t)stream, cand_score,
                     cand_index, cand_ld, n_cand, k, topk_idx, topk_ld, bm_words);
  return launch_status("topk_merge");
}
