// Internal helpers of the gfx950 FP4 indexer library: error reporting, device checks,
// schedule-buffer layouts, and the block-scaled FP4 MFMA wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "indexer_fp4.h"

namespace ifp4 {

constexpr int kPage = INDEXER_FP4_PAGE;          // tokens per page
constexpr int kHeadDim = INDEXER_FP4_HEAD_DIM;   // elements per key / query head
constexpr int kKeyBytes = kHeadDim / 2;          // packed E2M1 bytes per key (64)
constexpr int kGroups = kHeadDim / 32;           // e8m0 scales per key (4)
constexpr int kPageBytes = kPage * kKeyBytes;    // packed plane bytes per page (4096)
constexpr int kPageScaleBytes = kPage * kGroups; // scale plane bytes per page (256)
constexpr int kKeyBytes8 = kHeadDim;             // MXFP8 (comparator): E4M3 bytes per key (128)
constexpr int kPageBytes8 = kPage * kKeyBytes8;  // its packed plane bytes per page (8192)
constexpr int kRowMultiple = INDEXER_FP4_ROW_MULTIPLE; // prefill rows are padded to a multiple of this

// ---- errors (thread-local message, see indexer_fp4_last_error) -------------------------
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_device();                 // INDEXER_FP4_EARCH unless the current device is gfx950
int launch_status(const char *what);  // INDEXER_FP4_EHIP if the last launch failed

// ---- schedule buffers (int32 words) ------------------------------------------------------
// Decode: [0] magic, [1] error word, [2] batch, [3] next_n, [4] n_units, [5] items,
//         [6..7] 0, then cum_pages[batch+1], unit_begin[n_units+1], unit_seq[n_units],
//         unit_page[n_units], unit_run[n_units]: the sequence holding the unit's first
//         item, that item's page index in it, and how many items from it on stay in that
//         sequence (so a unit finds its first pages without walking cum_pages).
constexpr int32_t kDecodeMagic = 0x34504644;   // "DFP4"
constexpr int32_t kPrefillMagic = 0x34504650;  // "PFP4"
constexpr int kHdrWords = 8;

struct DecodeSchedLayout {
  int64_t cum, unit_begin, unit_seq, unit_page, unit_run, words;
  __host__ __device__ DecodeSchedLayout(int32_t batch, int32_t n_units) {
    cum = kHdrWords;
    unit_begin = cum + (int64_t)batch + 1;
    unit_seq = unit_begin + (int64_t)n_units + 1;
    unit_page = unit_seq + n_units;
    unit_run = unit_page + n_units;
    words = unit_run + n_units;
  }
};

// Prefill: a 16-word header [0] magic, [1] error word, [2] n_req, [3] n_rows_padded,
// [4] n_units, [5] n_tiles, [6] items, [7] tile rows, [8] bt_ld, [9] n_pages (clamped to
// INT32_MAX), then
//   unit records [n_units][16]: {first item, end item, first tile, 0, that tile's record (8
//                words), physical pages of the unit's first four items (-1 past its end)}
//   tiles      [max_tiles][8]: {first row, rows, valid rows, position of the first row,
//                request, pages, first item, 0}
//   cum_items  [max_tiles+1]  first item of each tile (items are (tile, page), tile-major)
//   unit_begin [n_units+1], unit_tile [n_units], req_tile [n_req+1]
//   item_phys  [max_tiles * bt_ld]  physical page of every item, -1 if it cannot be read
// The block table is resolved here, once a step for every layer that shares it, so a scorer
// unit needs one scalar load to start its first page copies.
constexpr int kPrefillTileRows = 16;
constexpr int kPrefillHdrWords = 16;
constexpr int kUnitRecWords = 16;
constexpr int kTileRecWords = 8;
constexpr int kUnitRecPhys = 4;  // first items whose pages a unit record carries

struct PrefillSchedLayout {
  int64_t max_tiles, urec, tiles, cum, unit_begin, unit_tile, req_tile, item_phys, words;
  __host__ __device__ PrefillSchedLayout(int32_t n_req, int32_t n_rows_padded, int32_t n_units, int64_t bt_ld) {
    max_tiles = (int64_t)n_rows_padded / kPrefillTileRows + n_req;
    urec = kPrefillHdrWords;
    tiles = urec + (int64_t)kUnitRecWords * n_units;
    cum = tiles + (int64_t)kTileRecWords * max_tiles;
    unit_begin = cum + max_tiles + 1;
    unit_tile = unit_begin + (int64_t)n_units + 1;
    req_tile = unit_tile + n_units;
    item_phys = req_tile + (int64_t)n_req + 1;
    words = item_phys + max_tiles * bt_ld;
  }
};

// ---- block-scaled FP4 MFMA ----------------------------------------------------------------
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 16x16x128 MXFP4 x MXFP4 -> fp32. Lane l supplies row (A) / column (B) l%16 and the 32
// K-elements [32*(l/16), 32*(l/16)+32) as 16 bytes, element 2i in the low nibble of byte
// i; its scale operand carries that (row, 32-block)'s e8m0 byte in byte SA / SB. The
// result holds C[4*(l/16)+i][l%16] in element i. Only the first four dwords of the A/B
// operands are read for FP4.
template <int SA, int SB>
__device__ __forceinline__ floatx4 mfma_fp4(const uint4 &a, const uint4 &b, floatx4 c, uint32_t sa,
                                            uint32_t sb) {
  intx8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  intx8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SA, (int)sa, SB, (int)sb);
}

// compile-time loop: f(std::integral_constant<int, I>{}) for I = 0..N-1
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), and each
// XCD has its own L2. This maps workgroup b to a work index so that consecutive work indices
// (neighbouring items, which share pages and query rows) run on one XCD: the first n - n % 8
// indices in 8 contiguous blocks, one per XCD, the rest unchanged.
__device__ __forceinline__ int xcd_local_index(int b, int n) {
  constexpr int kXcds = 8;
  const int n8 = n - n % kXcds;
  return b < n8 ? (b % kXcds) * (n8 / kXcds) + b / kXcds : b;
}

// Read-only view in the constant address space: wave-uniform reads through it become scalar
// loads, which do not wait behind the vector-memory queue (the page prefetches). Only for
// memory the kernel does not write.
template <class T>
using const_ptr = const __attribute__((address_space(4))) T *;
template <class T>
__device__ __forceinline__ const_ptr<T> as_const(const T *p) {
  return (const_ptr<T>)p;
}

// Raw buffer view of [base, base + bytes) for range-checked stores: a store at a byte
// offset past `bytes` is dropped by the hardware. Used to mask logits past a row's length
// without a branch (branches around stores make the compiler's memory-wait analysis fall
// back to waiting for every outstanding load). Descriptor word 3 is the gfx9-family raw
// 32-bit buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
#ifndef IFP4_STORE_POLICY
#define IFP4_STORE_POLICY 0
#endif
__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, (int)byte_offset, 0, IFP4_STORE_POLICY);
}
// The same store with the non-temporal hint (cache-policy bit 1 on gfx950): for output that is
// not read again by the kernel and would otherwise push data the kernel does reuse out of L2.
__device__ __forceinline__ void buffer_store_f32_nt(float v, __amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsrc, (int)byte_offset, 0, 2);
}

// Order-preserving 32-bit key of a float (flip the sign bit of non-negative values, invert
// negative ones; -0.0 is folded onto +0.0): a > b as floats iff key(a) > key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histograms of a row's logits on the top 12 key bits (the top-k's first digit), kept in
// device memory by the decode scorer and the top-k: bin b lives at word hist_slot(b), so
// neighbouring bins sit in different 256-byte blocks and device-wide atomics from many
// workgroups on the few occupied bins of a row do not queue on one block.
constexpr int kHistBins = 4096;
__host__ __device__ constexpr uint32_t hist_slot(uint32_t b) { return ((b & 63u) << 6) | (b >> 6); }

// Histogram increment of digit d for lanes with `ok`. A wave whose counted keys all share
// one digit (ties, constant rows) adds them with one atomic instead of 64 conflicting ones.
// Works on LDS and on global memory (through the pointer's address space).
template <class Ptr>
__device__ __forceinline__ void hist_put(Ptr h, uint32_t d, bool ok) {
  const uint64_t act = __ballot(ok);
  if (act == 0) return;
  const int first = __ffsll((unsigned long long)act) - 1;
  const uint32_t d0 = __builtin_amdgcn_readlane(d, first);
  if (__ballot(ok && d != d0) == 0) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&h[d0], (uint32_t)__popcll(act));
  } else if (ok) {
    atomicAdd(&h[d], 1u);
  }
}

}  // namespace ifp4
