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
#include "quant_common.h"
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

// The step's writer work, for the entry point that writes the step's key and query rows
// itself (next_n = 1): the arguments of indexer_fp4_norm_rope_quant_and_cache.
struct StepWrite {
  const uint16_t *k;          // [batch][k_ld] bf16: each sequence's new key
  int64_t k_ld;
  const float *gamma, *beta;  // k_norm (gamma NULL: none)
  float eps;
  const int64_t *positions;   // [batch] rotary positions
  const float *cos_sin;       // [max_pos][rope_dim]
  int64_t max_pos;
  int rope_dim;
  int interleaved;
  const int64_t *slots;       // [batch] cache slot of each new key
  const uint16_t *q;          // [batch][n_heads][128] bf16
  const float *weights;       // [batch][n_heads]
  float weight_scale;
  int all_q;
  uint8_t *kvp, *kvs;         // the cache planes, written
};

// A sequence's area in LDS: its quantized query heads (codes [H][64], scales [H][4], weights
// [H] -- what the writer stores as q_packed, q_scale, weights_mqa) and its new key (codes
// [64], scales [4], then whether the writer would store it and its slot).
constexpr int kQVecBytes = kKeyBytes + kGroups + 4;
constexpr int kKeyAreaBytes = 80;
__host__ __device__ constexpr int seq_area_bytes(int n_heads) { return n_heads * kQVecBytes + kKeyAreaBytes; }

// The inputs of lane-tasks first + task0 + kb * stride (16 lanes a query head, stride a
// multiple of 16), and of the sequence's key for the lanes whose task0 is below 16.
template <int KB>
struct SeqLoad {
  uint4 raw[KB];
  float wv[KB];
  uint4 kraw;
  float4 g[2], be[2];  // k_norm weight and bias as loaded (selected where they are used)
  float4 ang[4];       // the rotary row's cos and sin as loaded (arranged where they are used)
  float c[8], sn[8];
  int64_t pos, slot;
};

// The sequence's position and slot (the rotary table row waits for the position) ...
// (scalar loads, b being wave-uniform: they count on their own counter, apart from the vector
// loads in flight)
template <int KB>
__device__ __forceinline__ void seq_load_pos(SeqLoad<KB> &Q, const StepWrite W, int b) {
  const int64_t pos = as_const(W.rope_dim > 0 ? W.positions : W.slots)[b];
  Q.pos = W.rope_dim > 0 ? pos : 0;
  Q.slot = as_const(W.slots)[b];
}

// ... and its query heads' and key's inputs. Every lane loads the key's (the lanes whose task0
// is below 16 use them): loads under a lane condition would make the compiler wait for them
// where the branch ends.
template <int KB>
__device__ __forceinline__ void seq_load_data(SeqLoad<KB> &Q, const StepWrite W, int b, int n_heads, int task0,
                                              int stride, int first) {
  const int l = task0 & 15;
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
    const int h = min((first + task0 + kb * stride) >> 4, n_heads - 1);
    Q.raw[kb] = *reinterpret_cast<const uint4 *>(W.q + ((int64_t)b * n_heads + h) * kHeadDim + 8 * l);
    Q.wv[kb] = W.weights[(int64_t)b * n_heads + h];
  }
  Q.kraw = *reinterpret_cast<const uint4 *>(W.k + (int64_t)b * W.k_ld + 8 * l);
  // the k_norm parameters with no condition on the loads either: a missing one is read from
  // the query rows instead (in bounds) and not used
  const float *gp = W.gamma ? W.gamma : reinterpret_cast<const float *>(W.q);
  const float *bp = W.beta ? W.beta : gp;
  Q.g[0] = *reinterpret_cast<const float4 *>(gp + 8 * l);
  Q.g[1] = *reinterpret_cast<const float4 *>(gp + 8 * l + 4);
  Q.be[0] = *reinterpret_cast<const float4 *>(bp + 8 * l);
  Q.be[1] = *reinterpret_cast<const float4 *>(bp + 8 * l + 4);
}

template <int KB>
__device__ __forceinline__ void seq_load(SeqLoad<KB> &Q, const StepWrite W, int b, int n_heads, int task0, int stride,
                                         int first) {
  seq_load_pos<KB>(Q, W, b);
  seq_load_data<KB>(Q, W, b, n_heads, task0, stride, first);
}

// ... the rotary angles of the sequence's position (a second round: the table row waits for
// the position) ...
template <int KB>
__device__ __forceinline__ void seq_angles(SeqLoad<KB> &Q, const StepWrite W, int task0) {
  const int l = task0 & 15;
  const bool bad_pos = W.rope_dim > 0 && (Q.pos < 0 || Q.pos >= W.max_pos);
  // Four 16-byte loads for either pair layout, with no condition on them (a load under a
  // condition, even a uniform one, makes the compiler wait for it where the branches meet);
  // lanes past the rotary part load lane 0's angles and do not use them. seq_arrange_angles
  // puts them in place once they are needed.
  if (W.rope_dim > 0) {
    const float *row = W.cos_sin + (bad_pos ? 0 : Q.pos) * W.rope_dim;
    const int la = 8 * l < W.rope_dim ? l : 0, half = W.rope_dim >> 1;
    const int o0 = W.interleaved ? 4 * la : (8 * la) % half;
    const int o1 = W.interleaved ? 4 * la : o0 + 4;
    Q.ang[0] = *reinterpret_cast<const float4 *>(row + o0);
    Q.ang[1] = *reinterpret_cast<const float4 *>(row + o1);
    Q.ang[2] = *reinterpret_cast<const float4 *>(row + half + o0);
    Q.ang[3] = *reinterpret_cast<const float4 *>(row + half + o1);
  }
}

// The loaded angles as rope8 takes them (rope_angles' arrangement): interleaved pairs use
// each of the four values twice, half-split pairs the eight in order.
template <int KB>
__device__ __forceinline__ void seq_arrange_angles(SeqLoad<KB> &Q, const StepWrite W) {
  const float a0[4] = {Q.ang[0].x, Q.ang[0].y, Q.ang[0].z, Q.ang[0].w};
  const float a1[4] = {Q.ang[1].x, Q.ang[1].y, Q.ang[1].z, Q.ang[1].w};
  const float s0[4] = {Q.ang[2].x, Q.ang[2].y, Q.ang[2].z, Q.ang[2].w};
  const float s1[4] = {Q.ang[3].x, Q.ang[3].y, Q.ang[3].z, Q.ang[3].w};
  const bool il = W.interleaved != 0;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    Q.c[j] = il ? a0[j >> 1] : (j < 4 ? a0[j] : a1[j - 4]);
    Q.sn[j] = il ? s0[j >> 1] : (j < 4 ? s0[j] : s1[j - 4]);
  }
}

// ... then the query heads and the key quantized into the sequence's area.
template <int KB>
__device__ __forceinline__ void seq_store(SeqLoad<KB> &Q, const StepWrite W, int n_heads, int64_t n_pages,
                                          uint8_t *area, int task0, int stride, int first, bool key) {
  const int l = task0 & 15, g = l >> 2;
  const bool bad_pos = W.rope_dim > 0 && (Q.pos < 0 || Q.pos >= W.max_pos);
  const bool live = !bad_pos && (Q.slot >= 0 || W.all_q != 0);
  if (W.rope_dim > 0) seq_arrange_angles<KB>(Q, W);
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
    const int i = first + task0 + kb * stride;
    if (i >= 16 * n_heads) break;  // uniform over the head's 16 lanes
    const int h = i >> 4;
    uint32_t sc = 0, d = 0;
    if (live) d = norm_rope_encode(Q.raw[kb], l, false, Q.c, Q.c, 0.f, W.rope_dim, W.interleaved != 0, Q.c, Q.sn, sc);
    *reinterpret_cast<uint32_t *>(area + h * kKeyBytes + 4 * l) = d;
    if ((l & 3) == 0) area[n_heads * kKeyBytes + h * kGroups + g] = (uint8_t)sc;
    if (l == 0)
      reinterpret_cast<float *>(area + n_heads * (kKeyBytes + kGroups))[h] = live ? W.weight_scale * Q.wv[kb] : 0.f;
  }
  if (key) {  // the writer stores the key when its position and slot are good
    uint8_t *ka = area + n_heads * kQVecBytes;
    const bool store = !bad_pos && Q.slot >= 0 && Q.slot < n_pages * kPage;
    const float gm[8] = {Q.g[0].x, Q.g[0].y, Q.g[0].z, Q.g[0].w, Q.g[1].x, Q.g[1].y, Q.g[1].z, Q.g[1].w};
    float bt[8] = {Q.be[0].x, Q.be[0].y, Q.be[0].z, Q.be[0].w, Q.be[1].x, Q.be[1].y, Q.be[1].z, Q.be[1].w};
    if (!W.beta) {
#pragma unroll
      for (int j = 0; j < 8; j++) bt[j] = 0.f;
    }
    uint32_t sc = 0;
    const uint32_t d = norm_rope_encode(Q.kraw, l, W.gamma != nullptr, gm, bt, W.eps, W.rope_dim,
                                        W.interleaved != 0, Q.c, Q.sn, sc);
    *reinterpret_cast<uint32_t *>(ka + 4 * l) = d;
    if ((l & 3) == 0) ka[kKeyBytes + g] = (uint8_t)sc;
    if (l == 0) {
      reinterpret_cast<int32_t *>(ka + 68)[0] = (store ? 1 : 0) | (bad_pos ? 2 : 0);
      *reinterpret_cast<int64_t *>(ka + 72) = Q.slot;
    }
  }
}

// The scorer on the page that holds the sequence's new key: the key's codes and scales go
// into the page's operand registers at its position p (the lanes of key p % 16 of tile
// p / 16), and the wave stores them at the key's slot, as the writer would. Nothing is
// patched unless the slot is that position of this page (the writer would have written the
// key elsewhere, and this page keeps what it holds).
__device__ __forceinline__ void patch_new_key(PageRegs &P, const uint8_t *ka, int p, int64_t phys, const StepWrite W,
                                              int64_t n_pages, int32_t *err, int lane) {
  const int flags = reinterpret_cast<const int32_t *>(ka + 68)[0];
  const int64_t slot = *reinterpret_cast<const int64_t *>(ka + 72);
  if (lane == 0 && (flags & 2)) atomicOr(err, INDEXER_FP4_DEV_BAD_POSITION);
  if (lane == 0 && !(flags & 2) && slot >= n_pages * kPage) atomicOr(err, INDEXER_FP4_DEV_SLOT_OUT_OF_POOL);
  if (!(flags & 1)) return;
  if (lane < 16) {  // the writer's store
    const int g = lane >> 2;
    const int64_t page = slot / kPage;
    const int sp = (int)(slot % kPage);
    *reinterpret_cast<uint32_t *>(W.kvp + slot * kKeyBytes + 4 * lane) = *reinterpret_cast<const uint32_t *>(ka + 4 * lane);
    if ((lane & 3) == 0) W.kvs[(page * kGroups + g) * kPage + (sp % 16) * 4 + sp / 16] = ka[kKeyBytes + g];
  }
  if (slot != phys * kPage + p) return;
  const int t = p >> 4;  // uniform
  if ((lane & 15) == (p & 15)) {
    const uint4 v = *reinterpret_cast<const uint4 *>(ka + 16 * (lane >> 4));
    if (t == 0) P.k[0] = v;
    else if (t == 1) P.k[1] = v;
    else if (t == 2) P.k[2] = v;
    else P.k[3] = v;
    P.s = (P.s & ~(0xFFu << (8 * t))) | ((uint32_t)ka[kKeyBytes + (lane >> 4)] << (8 * t));
  }
}

// One query row from a sequence's area (what load_rows reads from memory).
template <int NH16, int NN>
__device__ __forceinline__ void rows_from_area(RowRegs<NH16, NN> &R, const uint8_t *area, int n_heads, int lane) {
  const int hl = lane & 15, g = lane >> 4;
  const uint8_t *aqs = area + n_heads * kKeyBytes;
  const float *aw = reinterpret_cast<const float *>(area + n_heads * (kKeyBytes + kGroups));
#pragma unroll
  for (int j = 0; j < (NH16 + 3) / 4; j++) R.qs[0][j] = 0;
#pragma unroll
  for (int m = 0; m < NH16; m++) {
    const int v = 16 * m + hl;
    R.qa[0][m] = *reinterpret_cast<const uint4 *>(area + v * kKeyBytes + 16 * g);
    R.qs[0][m / 4] |= (uint32_t)aqs[v * kGroups + g] << (8 * (m % 4));
    R.w[0][m] = *reinterpret_cast<const float4 *>(aw + 16 * m + 4 * g);
  }
}

template <class F, int NH16, int NN, int NW, int D, bool WR>
__global__ __launch_bounds__(NW * 64) void score_decode_kernel(
    const uint8_t *__restrict__ qp, const uint8_t *__restrict__ qs, const float *__restrict__ w, int n_heads,
    const uint8_t *__restrict__ kvp, const uint8_t *__restrict__ kvs, int64_t n_pages,
    const int32_t *__restrict__ bt_g, int64_t bt_ld, int batch, int n_units, const int32_t *__restrict__ sched_g,
    int32_t *__restrict__ err, const int32_t *__restrict__ row_len_g, float *__restrict__ logits, int64_t ld,
    uint32_t *__restrict__ row_hist, const StepWrite Wr_arg) {
  static_assert(!WR || (NN == 1 && NH16 <= 8), "the writing scorer takes one row a sequence, up to 128 heads");
  const StepWrite Wr = Wr_arg;  // (a copy: no address of the kernel argument is taken)
  // dynamic LDS: [NN][kHistBins] with a row histogram; then, when writing, query areas
  extern __shared__ uint32_t uh[];
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
  // Writing: the query heads of the unit's first sequence (one lane-task each, 16 a head) are
  // requested right after the first pages and quantized into the unit's LDS area while those
  // are in flight.
  uint8_t *qarea = reinterpret_cast<uint8_t *>(uh + (fuse ? NN * kHistBins : 0));
  const int area_bytes = seq_area_bytes(n_heads);
  constexpr int KBC = WR ? (16 * 16 * NH16 + NW * 64 - 1) / (NW * 64) : 1;
  // this wave's contiguous share of the unit's items (none for some waves of a short unit,
  // which still meet the workgroup's barriers)
  const int per = (it1 - it0 + NW - 1) / NW;
  const int w0 = it0 + wv * per;
  const int w1 = min(it1, w0 + per);
  const int n_my = max(0, w1 - w0);
  const int32_t *cum = sched_g + L.cum;

  // Item table, one lane per item, for 64 items at a time: sequence, page index within
  // it, and physical page (-1 if the page cannot be read); when writing, whether the item is
  // its sequence's last page (the one that holds the step's new key). Built with one round
  // of per-lane loads instead of a chain of dependent scalar loads per page.
  int seq0 = sched[L.unit_seq + u];  // sequence of the unit's first item
  const int page0 = sched[L.unit_page + u];
  const int run0 = sched[L.unit_run + u];
  const int end0 = WR ? sched[L.cum + min(seq0, batch - 1) + 1] : 0;  // past the first sequence's last item
  int tab_base = -64;
  int v_seq = 0, v_page = 0, v_phys = -1;
  bool v_last = false;
  // in two halves, so that the writing scorer can issue other loads between the table entries'
  // request and their use: every lane loads an entry of the table (clamped into it), and the
  // check afterwards keeps the ones of real items
  int f_raw = 0, f_b = 0, f_p = 0;
  bool f_in = false, f_ok = false, f_last = false;
  auto fill_issue = [&](int base) __attribute__((always_inline)) {
    tab_base = base;
    const int it = w0 + base + lane;
    int b = seq0, p = 0;
    bool last = false;
    if (it < w1) {
      const int k = it - it0;  // items past the unit's first one
      if (k < run0) {          // still in the unit's first sequence: no lookup
        b = sched[L.unit_seq + u];
        p = page0 + k;
        if constexpr (WR) last = it + 1 == end0;
      } else {
        while (b < batch - 1 && it >= cum[b + 1]) b++;
        p = it - cum[b];
        if constexpr (WR) last = it + 1 == cum[b + 1];
      }
    }
    const int64_t bc = min(max(b, 0), batch - 1), pc = min(max((int64_t)p, (int64_t)0), bt_ld - 1);
    f_raw = bt_g[bc * bt_ld + pc];
    f_b = b;
    f_p = p;
    f_in = it < w1;
    f_ok = p >= 0 && p < bt_ld;
    f_last = last;
  };
  auto fill_check = [&]() __attribute__((always_inline)) {
    int phys = -1;
    if (f_in) {
      if (f_ok) {
        phys = f_raw;
        if (phys < 0 || phys >= n_pages) {
          atomicOr(err, INDEXER_FP4_DEV_BAD_PAGE);
          phys = -1;
        }
      } else {
        atomicOr(err, f_p < 0 ? INDEXER_FP4_DEV_BAD_SCHEDULE : INDEXER_FP4_DEV_TABLE_SHORT);
      }
    }
    v_seq = f_b;
    v_page = f_p;
    v_phys = phys;
    v_last = f_last;
    seq0 = __builtin_amdgcn_readlane(f_b, 63);  // sequences only advance with the items
  };
  auto fill = [&](int base) __attribute__((always_inline)) {
    fill_issue(base);
    fill_check();
  };
  // Software pipeline over a ring of D pages: scoring slot K overlaps the loads of the
  // other D-1 slots. Every slot refill is unconditional -- past the wave's last item it
  // reloads that item (a cache hit) and its logits are dropped -- so the compiler waits
  // only for the slot being scored.
  typename F::Page P[D];
  int sb[D], sp[D];
  bool sok[D];
  bool slast[D];     // writing: the slot holds its sequence's last page
  int64_t sphys[D];  // writing: its physical page
  auto issue = [&](auto kk, int i) __attribute__((always_inline)) {
    constexpr int K = decltype(kk)::value;
    const bool live = i < n_my;
    const int ii = live ? i : max(n_my - 1, 0);  // (a wave with no item loads the table's first entry, dropped)
    if (ii - tab_base >= 64) fill(ii & ~63);
    const int l = ii - tab_base;
    const int phys = __builtin_amdgcn_readlane(v_phys, l);
    sb[K] = __builtin_amdgcn_readlane(v_seq, l);
    sp[K] = __builtin_amdgcn_readlane(v_page, l);
    sok[K] = live && phys >= 0;
    if constexpr (WR) {
      slast[K] = live && __builtin_amdgcn_readlane((int)v_last, l) != 0;
      sphys[K] = phys;
    }
    F::page(P[K], kvp, kvs, phys >= 0 ? phys : 0, lane);
  };
  typename F::template Rows<NH16, NN> R;
  int qb = -1;
  uint8_t *warea = qarea + (1 + wv) * area_bytes;  // this wave's area, for other sequences
  auto score = [&](auto kk) __attribute__((always_inline)) {
    constexpr int K = decltype(kk)::value;
    if (sb[K] != qb) {  // a new sequence: its query rows (waits for everything in flight)
      qb = sb[K];
      if constexpr (WR) {
        if (qb == qs0) {
          rows_from_area<NH16, NN>(R, qarea, n_heads, lane);
        } else {  // quantized by this wave alone, two lane-tasks a lane at a time
          for (int first = 0; first < 16 * n_heads; first += 2 * 64) {
            SeqLoad<2> Qw;
            seq_load<2>(Qw, Wr, qb, n_heads, lane, 64, first);
            seq_angles<2>(Qw, Wr, lane);
            seq_store<2>(Qw, Wr, n_heads, n_pages, warea, lane, 64, first, first == 0 && lane < 16);
          }
          rows_from_area<NH16, NN>(R, warea, n_heads, lane);
        }
      } else {
        F::template rows<NH16, NN>(R, qp, qs, w, (int64_t)qb * NN, NN, n_heads, lane);
      }
    }
    if constexpr (WR) {  // the page that holds the sequence's new key
      if (slast[K]) {
        const int p = (row_len[qb] - 1) & (kPage - 1);
        patch_new_key(P[K], (qb == qs0 ? qarea : warea) + n_heads * kQVecBytes, p, sphys[K], Wr, n_pages, err, lane);
      }
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

  // Writing: the first sequence's query heads and key are requested with the item table
  // (one lane-task each, 16 a head; the key by the first 16 lanes), its rotary table row ahead
  // of the first pages, and all of it quantized while those pages are in flight.
  SeqLoad<KBC> Q0;
  if constexpr (WR) {
    // Loads go out in the order they are needed (the vector memory counter completes in
    // order, so a wait for one load is a wait for every older one): the position (a scalar
    // load, on its own counter), the table entries, the rotary row (its wait covers the
    // position only), the query and key inputs; then the first pages (their wait covers the
    // table) and the quantization, whose inputs are all older than the pages. A wave with no
    // item still issues its first pages (page 0, dropped), so no load sits under a condition
    // the compiler would have to merge.
    seq_load_pos<KBC>(Q0, Wr, qs0);
    fill_issue(0);
    asm volatile("" ::: "memory");
    seq_angles<KBC>(Q0, Wr, threadIdx.x);
    asm volatile("" ::: "memory");
    seq_load_data<KBC>(Q0, Wr, qs0, n_heads, threadIdx.x, NW * 64, 0);
    asm volatile("" ::: "memory");
    fill_check();
    static_for<D>([&](auto kk) { issue(kk, decltype(kk)::value); });
    seq_store<KBC>(Q0, Wr, n_heads, n_pages, qarea, threadIdx.x, NW * 64, 0, threadIdx.x < 16);
  } else if (n_my > 0) {
    fill(0);
    static_for<D>([&](auto kk) { issue(kk, decltype(kk)::value); });
  }
  if (fuse) {
    for (int i = threadIdx.x; i < NN * kHistBins / 4; i += NW * 64)
      reinterpret_cast<uint4 *>(uh)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (fuse || WR) __syncthreads();  // the histogram cleared, the query area written
  if (n_my > 0) {
    for (int i0 = 0; i0 < n_my; i0 += D) {
      static_for<D>([&](auto kk) {
        score(kk);
        issue(kk, i0 + decltype(kk)::value + D);
      });
    }
  }
  if (fuse) {  // occupied bins only, one device atomic each; four bins a 16-byte LDS read
    __syncthreads();
    uint32_t *g = row_hist + (int64_t)qs0 * NN * kHistBins;
    for (int i4 = threadIdx.x; i4 < NN * kHistBins / 4; i4 += NW * 64) {
      const uint4 c4 = reinterpret_cast<const uint4 *>(uh)[i4];
      if ((c4.x | c4.y | c4.z | c4.w) == 0u) continue;
      const uint32_t cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = 4 * i4 + e;
        if (cv[e]) atomicAdd(&g[(i / kHistBins) * kHistBins + hist_slot(i % kHistBins)], cv[e]);
      }
    }
  }
}

template <class F, int NH16, int NN, bool WR = false>
static int launch_decode(hipStream_t st, int n_units, const uint8_t *qp, const uint8_t *qs, const float *w,
                          int n_heads, const uint8_t *kvp, const uint8_t *kvs, int64_t n_pages, const int32_t *bt,
                          int64_t bt_ld, int batch, int32_t *sched, const int32_t *row_len, float *logits,
                          int64_t ld, uint32_t *row_hist, const StepWrite &Wr = StepWrite{}) {
  constexpr int NW = IFP4_DECODE_WAVES, D = IFP4_DECODE_RING;
  // dynamic LDS: the histogram, then (writing) the unit's and each wave's query area
  const size_t lds = (row_hist ? (size_t)NN * kHistBins * 4 : 0) + (WR ? (size_t)(1 + NW) * seq_area_bytes(n_heads) : 0);
  static bool lds_set = false;  // raise the dynamic LDS limit once per instantiation
  if (!lds_set) {
    const size_t most = (size_t)NN * kHistBins * 4 + (WR ? (size_t)(1 + NW) * seq_area_bytes(16 * NH16) : 0);
    const hipError_t e = hipFuncSetAttribute((const void *)score_decode_kernel<F, NH16, NN, NW, D, WR>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)most);
    if (e != hipSuccess) return fail(INDEXER_FP4_EHIP, "score_decode: hipFuncSetAttribute: %s", hipGetErrorString(e));
    lds_set = true;
  }
  hipLaunchKernelGGL((score_decode_kernel<F, NH16, NN, NW, D, WR>), dim3(n_units), dim3(NW * 64), lds, st, qp, qs, w,
                     n_heads, kvp, kvs, n_pages, bt, bt_ld, batch, n_units, sched, sched + 1, row_len, logits, ld,
                     row_hist, Wr);
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

// Write and score in one launch (next_n = 1): the scorer quantizes its query rows itself and
// writes each sequence's new key from the wave that scores the key's page, before loading it.
extern "C" int indexer_fp4_write_and_score_decode(
    const void *k_bf16, int64_t k_ld, const float *k_norm_weight, const float *k_norm_bias, float eps,
    const int64_t *positions, const float *cos_sin, int64_t max_pos, int32_t rope_dim, int32_t rope_interleaved,
    const int64_t *slot_mapping, const void *q_bf16, const float *weights, float weight_scale, int32_t all_q,
    int32_t n_heads, uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const int32_t *block_table, int64_t bt_ld,
    int32_t batch, void *sched, int64_t sched_bytes, int32_t n_units, const int32_t *row_len, float *logits,
    int64_t logits_ld, uint32_t *row_hist, void *stream) {
  clear_error();
  if (n_heads <= 0 || n_heads % INDEXER_FP4_HEAD_MULT != 0 || n_heads > 128)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: n_heads=%d must be a positive multiple of %d and at most 128",
                n_heads, INDEXER_FP4_HEAD_MULT);
  if (batch < 0 || n_units <= 0 || n_pages < 0)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: batch=%d >= 0, n_units=%d > 0, n_pages=%lld >= 0", batch,
                n_units, (long long)n_pages);
  if (rope_dim < 0 || rope_dim > kHeadDim || rope_dim % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: rope_dim=%d must be a multiple of 16 in 0..%d", rope_dim,
                kHeadDim);
  if (!k_norm_weight && k_norm_bias)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: k_norm_bias without k_norm_weight");
  if (!(eps >= 0.f)) return fail(INDEXER_FP4_EINVAL, "write_and_score: eps must be >= 0");
  if (k_ld < kHeadDim || k_ld % 8 != 0)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: k_ld=%lld must be >= %d and a multiple of 8", (long long)k_ld,
                kHeadDim);
  if (bt_ld <= 0) return fail(INDEXER_FP4_ENOSPC, "write_and_score: bt_ld=%lld must be positive", (long long)bt_ld);
  if (logits_ld < bt_ld * kPage)
    return fail(INDEXER_FP4_ENOSPC, "write_and_score: logits_ld=%lld < 64*bt_ld=%lld", (long long)logits_ld,
                (long long)(bt_ld * kPage));
  if (!sched || !row_len ||
      (batch > 0 && (!k_bf16 || !slot_mapping || !q_bf16 || !weights || !block_table || !logits || !kv_packed ||
                     !kv_scale)))
    return fail(INDEXER_FP4_EINVAL, "write_and_score: a required pointer is NULL");
  if (batch > 0 && rope_dim > 0 && (!positions || !cos_sin || max_pos <= 0))
    return fail(INDEXER_FP4_EINVAL, "write_and_score: rope_dim=%d needs positions and a cos/sin table", rope_dim);
  if (((uintptr_t)k_bf16 | (uintptr_t)q_bf16 | (uintptr_t)kv_packed | (uintptr_t)kv_scale | (uintptr_t)cos_sin |
       (uintptr_t)k_norm_weight | (uintptr_t)k_norm_bias | (uintptr_t)row_hist) % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "write_and_score: k, q, both planes, cos_sin, k_norm_weight, k_norm_bias and "
                                    "row_hist must be 16-byte aligned");
  const int64_t need = 4 * DecodeSchedLayout(batch, n_units).words;
  if (sched_bytes < need)
    return fail(INDEXER_FP4_ENOSPC, "write_and_score: sched_bytes=%lld < %lld for batch=%d, n_units=%d",
                (long long)sched_bytes, (long long)need, batch, n_units);
  int rc = check_device();
  if (rc) return rc;
  if (batch == 0) return INDEXER_FP4_OK;
  const StepWrite W{(const uint16_t *)k_bf16, k_ld, k_norm_weight, k_norm_bias, eps, positions, cos_sin, max_pos,
                    rope_dim, rope_interleaved != 0, slot_mapping, (const uint16_t *)q_bf16, weights, weight_scale,
                    all_q != 0, kv_packed, kv_scale};
  hipStream_t st = (hipStream_t)stream;
  int32_t *sc = (int32_t *)sched;
  switch (n_heads / 16) {
#define IFP4_CASE(X) \
  case X: rc = launch_decode<FmtFp4, X, 1, true>(st, n_units, nullptr, nullptr, nullptr, n_heads, kv_packed, kv_scale, n_pages, block_table, bt_ld, batch, sc, row_len, logits, logits_ld, row_hist, W); break;
    IFP4_CASE(1) IFP4_CASE(2) IFP4_CASE(3) IFP4_CASE(4) IFP4_CASE(5) IFP4_CASE(6) IFP4_CASE(7) IFP4_CASE(8)
#undef IFP4_CASE
  }
  return rc ? rc : launch_status("write_and_score_decode");
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
