// MXFP4 quantization of index keys into the paged two-plane cache, and of queries.
//
// "Score a DSA sparse indexer in FP4" (ROCm/ATOM #2216), commit message: the fused
// writer's FP4 output mode stores each key as packed E2M1 codes plus e8m0 scales in
// the index region's two planes and emits the quantized query with its scales; review
// fixes: rows with a negative slot are skipped. The element and scale rules are the
// OCP MX v1.0 ones (the pages name the format but print no rule): scale exponent
// floor(log2 amax) - 2 clamped to [-127, 127]; elements rounded to the nearest E2M1
// value, ties to the even code, saturating at 6.
//
// One thread encodes one 32-element block: 64 input bytes in, 16 packed bytes and one
// scale byte out. All decisions are made on the bf16 bit patterns in integer
// arithmetic, so the result does not depend on the FP denormal mode.
#include "common.h"

namespace ifp4 {

// E2M1 magnitude code of a bf16 magnitude `mag` (15 bits: exponent << 7 | mantissa) at
// block scale 2^e. With sig the significand (implicit bit included) and ep the
// effective exponent field, |v| = sig * 2^(ep-134) and 4|v|/2^e = sig * 2^sh. The code
// counts the decision points {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} that the scaled
// magnitude passes; at the points with an even code below (0.25, 1.25, 2.5, 5) the
// tie stays below, at the others (0.75, 1.75, 3.5) it goes up.
__device__ __forceinline__ uint32_t e2m1_magnitude_code(uint32_t mag, int e) {
  const uint32_t ex = mag >> 7;
  const uint32_t sig = ex ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu);
  const int ep = ex ? (int)ex : 1;
  const int sh = ep - 134 - e + 2;
  uint32_t c;
  if (sh >= 0) {
    const uint32_t x = sig << (sh < 20 ? sh : 20);  // 4x, saturated well past 20
    c = (x > 1u) + (x >= 3u) + (x > 5u) + (x >= 7u) + (x > 10u) + (x >= 14u) + (x > 20u);
  } else {
    const int n = -sh;  // compare sig against threshold * 2^n
    if (n > 20) return 0u;
    c = (sig > (1u << n)) + (sig >= (3u << n)) + (sig > (5u << n)) + (sig >= (7u << n)) +
        (sig > (10u << n)) + (sig >= (14u << n)) + (sig > (20u << n));
  }
  return c;
}

// 32 bf16 (as 4 x uint4) -> 16 packed bytes (element 2i low nibble of byte i) + scale
__device__ __forceinline__ void encode_block32(const uint4 in[4], uint4 &packed, uint32_t &scale) {
  uint32_t amag = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t w[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
#pragma unroll
    for (int h = 0; h < 4; h++) {
      amag = max(amag, w[h] & 0x7FFFu);
      amag = max(amag, (w[h] >> 16) & 0x7FFFu);
    }
  }
  int e = -127;
  if (amag != 0) {
    const uint32_t ex = amag >> 7;
    const uint32_t sig = ex ? (0x80u | (amag & 0x7Fu)) : (amag & 0x7Fu);
    const int ep = ex ? (int)ex : 1;
    const int fl = (31 - __builtin_clz(sig)) + ep - 134;  // floor(log2 amax)
    e = fl - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  scale = (uint32_t)(e + 127);
  uint32_t out[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t w[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
    uint32_t d = 0;
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const uint32_t lo = w[h] & 0xFFFFu, hi = w[h] >> 16;
      const uint32_t clo = e2m1_magnitude_code(lo & 0x7FFFu, e) | ((lo >> 12) & 8u);
      const uint32_t chi = e2m1_magnitude_code(hi & 0x7FFFu, e) | ((hi >> 12) & 8u);
      d |= (clo | (chi << 4)) << (8 * h);
    }
    out[j] = d;
  }
  packed = make_uint4(out[0], out[1], out[2], out[3]);
}

__global__ __launch_bounds__(256) void quant_cache_kernel(
    const uint16_t *__restrict__ k, int64_t n_tok, int64_t k_ld, const int64_t *__restrict__ slots,
    uint8_t *__restrict__ kv_packed, uint8_t *__restrict__ kv_scale, int64_t n_pages,
    const uint16_t *__restrict__ q, int64_t n_q_vec, uint8_t *__restrict__ q_packed,
    uint8_t *__restrict__ q_scale) {
  const int64_t total = (n_tok + n_q_vec) * kGroups;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t v = i >> 2;
    const int g = (int)(i & 3);
    uint4 in[4];
    uint4 packed;
    uint32_t sc;
    if (v < n_tok) {
      const int64_t slot = slots[v];
      if (slot < 0 || slot >= n_pages * kPage) continue;
      const uint4 *src = reinterpret_cast<const uint4 *>(k + v * k_ld + 32 * g);
#pragma unroll
      for (int j = 0; j < 4; j++) in[j] = src[j];
      encode_block32(in, packed, sc);
      const int64_t page = slot / kPage;
      const int pos = (int)(slot % kPage);
      *reinterpret_cast<uint4 *>(kv_packed + (page * kPage + pos) * kKeyBytes + 16 * g) = packed;
      // scale plane: the 64-row axis is stored as a 16x4 transpose
      kv_scale[(page * kGroups + g) * kPage + (pos % 16) * 4 + pos / 16] = (uint8_t)sc;
    } else {
      const int64_t vq = v - n_tok;
      const uint4 *src = reinterpret_cast<const uint4 *>(q + vq * kHeadDim + 32 * g);
#pragma unroll
      for (int j = 0; j < 4; j++) in[j] = src[j];
      encode_block32(in, packed, sc);
      *reinterpret_cast<uint4 *>(q_packed + vq * kKeyBytes + 16 * g) = packed;
      q_scale[vq * kGroups + g] = (uint8_t)sc;
    }
  }
}

}  // namespace ifp4

using namespace ifp4;

extern "C" int indexer_fp4_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                           const int64_t *slot_mapping, uint8_t *kv_packed,
                                           uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
                                           int64_t n_q_rows, int32_t n_heads, uint8_t *q_packed,
                                           uint8_t *q_scale, void *stream) {
  clear_error();
  if (n_tok < 0 || n_pages < 0 || n_q_rows < 0)
    return fail(INDEXER_FP4_EINVAL, "negative size: n_tok=%lld n_pages=%lld n_q_rows=%lld",
                (long long)n_tok, (long long)n_pages, (long long)n_q_rows);
  if (n_tok > 0) {
    if (!k_bf16 || !slot_mapping || !kv_packed || !kv_scale)
      return fail(INDEXER_FP4_EINVAL, "key arm with n_tok=%lld needs k, slot_mapping and both planes",
                  (long long)n_tok);
    if (k_ld < kHeadDim || k_ld % 8 != 0)
      return fail(INDEXER_FP4_EINVAL, "k_ld=%lld must be >= %d and a multiple of 8", (long long)k_ld, kHeadDim);
    if (((uintptr_t)k_bf16 | (uintptr_t)kv_packed) % 16 != 0)
      return fail(INDEXER_FP4_EINVAL, "k and kv_packed must be 16-byte aligned");
  }
  const bool q_arm = q_bf16 != nullptr && n_q_rows > 0;
  if (q_arm) {
    if (n_heads <= 0) return fail(INDEXER_FP4_EINVAL, "n_heads=%d must be positive", n_heads);
    if (!q_packed || !q_scale) return fail(INDEXER_FP4_EINVAL, "query arm needs q_packed and q_scale");
    if (((uintptr_t)q_bf16 | (uintptr_t)q_packed) % 16 != 0)
      return fail(INDEXER_FP4_EINVAL, "q and q_packed must be 16-byte aligned");
  }
  int rc = check_device();
  if (rc) return rc;
  const int64_t n_q_vec = q_arm ? n_q_rows * (int64_t)n_heads : 0;
  const int64_t total = (n_tok + n_q_vec) * kGroups;
  if (total == 0) return INDEXER_FP4_OK;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quant_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                     (const uint16_t *)k_bf16, n_tok, k_ld, slot_mapping, kv_packed, kv_scale, n_pages,
                     (const uint16_t *)q_bf16, n_q_vec, q_packed, q_scale);
  return launch_status("quant_and_cache");
}
