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
// Four lanes encode one 32-element block (eight elements, one 16-byte load and one 4-byte
// store each), sixteen lanes one 128-element vector: the block maximum is a two-step
// cross-lane reduction. All decisions are made on the bf16 bit patterns in integer
// arithmetic, so the result does not depend on the FP denormal mode.
#include "quant_common.h"

namespace ifp4 {

__global__ __launch_bounds__(256) void quant_cache_kernel(
    const uint16_t *__restrict__ k, int64_t n_tok, int64_t k_ld, const int64_t *__restrict__ slots,
    uint8_t *__restrict__ kv_packed, uint8_t *__restrict__ kv_scale, int64_t n_pages,
    const uint16_t *__restrict__ q, int64_t n_q_vec, uint8_t *__restrict__ q_packed,
    uint8_t *__restrict__ q_scale) {
  // every 16-lane group walks whole vectors, so the four lanes of a block stay together
  const int64_t total = (n_tok + n_q_vec) * kLanesPerVec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t v = i / kLanesPerVec;
    const int l = (int)(i % kLanesPerVec);  // elements 8l .. 8l+7 of the vector
    const int g = l >> 2;                   // its 32-element block
    uint32_t sc;
    if (v < n_tok) {
      const int64_t slot = slots[v];
      if (slot < 0 || slot >= n_pages * kPage) continue;  // uniform over the vector's lanes
      const uint4 in = *reinterpret_cast<const uint4 *>(k + v * k_ld + 8 * l);
      const uint32_t d = encode_lane8(in, sc);
      const int64_t page = slot / kPage;
      const int pos = (int)(slot % kPage);
      *reinterpret_cast<uint32_t *>(kv_packed + (page * kPage + pos) * kKeyBytes + 4 * l) = d;
      // scale plane: the 64-row axis is stored as a 16x4 transpose
      if ((l & 3) == 0) kv_scale[(page * kGroups + g) * kPage + (pos % 16) * 4 + pos / 16] = (uint8_t)sc;
    } else {
      const int64_t vq = v - n_tok;
      const uint4 in = *reinterpret_cast<const uint4 *>(q + vq * kHeadDim + 8 * l);
      const uint32_t d = encode_lane8(in, sc);
      *reinterpret_cast<uint32_t *>(q_packed + vq * kKeyBytes + 4 * l) = d;
      if ((l & 3) == 0) q_scale[vq * kGroups + g] = (uint8_t)sc;
    }
  }
}

// ---------------------------------------------------------------------------------------
// MXFP8 writer for the FP8 comparator (the pages compare the FP4 indexer with an FP8 one
// but give no FP8 format; this is OCP MXFP8): E4M3 elements (bias 7, largest 448, no
// infinities) with one e8m0 scale per 32, scale exponent floor(log2 amax) - 8 clamped to
// [-127, 127], elements rounded to nearest with ties to even and saturated at 448. Same
// lanes as the FP4 writer; element d of a vector is byte d, scales in the FP4 scale plane.

// floor(log2 amax) - 8, clamped; -127 for an all-zero block.
__device__ __forceinline__ int block_exponent8(uint32_t amag) {
  if (amag == 0) return -127;
  const uint32_t ex = amag >> 7;
  const uint32_t sig = ex ? (0x80u | (amag & 0x7Fu)) : (amag & 0x7Fu);
  const int ep = ex ? (int)ex : 1;
  const int e = (31 - __builtin_clz(sig)) + ep - 134 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E4M3 code of bf16 bits b divided by 2^e. The magnitude is M * 2^(E - 7) with M the 8-bit
// significand (no hidden bit for bf16 subnormals); its E4M3 step is 2^(max(L, -6) - 3) for
// leading exponent L, so the code's significand is M shifted right by the difference,
// rounded to nearest even; a carry into the exponent field is the correct next code.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t b, int e) {
  const uint32_t sign = (b >> 8) & 0x80u;
  const uint32_t mag = b & 0x7FFFu;
  if (mag == 0) return sign;
  const uint32_t ex = mag >> 7;
  const int M = (int)(ex ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu));
  const int Ep = (ex ? (int)ex - 127 : -126) - e;          // value = M * 2^(Ep - 7)
  const int L = Ep - 7 + (31 - __builtin_clz((uint32_t)M));  // floor(log2 value)
  const int qe = (L > -6 ? L : -6) - 3;                     // log2 of the E4M3 step there
  const int sh = qe - (Ep - 7);
  int n;
  if (sh <= 0) {
    n = M << (-sh);  // exact (fewer significant bits than the step allows)
  } else if (sh > 9) {
    n = 0;           // below half the smallest step
  } else {
    n = M >> sh;
    const int rem = M & ((1 << sh) - 1), half = 1 << (sh - 1);
    n += (rem > half || (rem == half && (n & 1))) ? 1 : 0;
  }
  uint32_t code = qe == -9 ? (uint32_t)n : (uint32_t)(((qe + 10) << 3) + (n - 8));
  if (code > 0x7Eu) code = 0x7Eu;  // saturate at 448 (0x7F is NaN)
  return code | sign;
}

// This lane's eight bf16 -> eight E4M3 bytes (element i in byte i) and the block's scale.
__device__ __forceinline__ uint2 encode8_lane8(uint4 in, uint32_t &scale) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t amag = 0;
#pragma unroll
  for (int h = 0; h < 4; h++) amag = max(amag, max(w[h] & 0x7FFFu, (w[h] >> 16) & 0x7FFFu));
  amag = max(amag, (uint32_t)__shfl_xor((int)amag, 1, 64));
  amag = max(amag, (uint32_t)__shfl_xor((int)amag, 2, 64));
  const int e = block_exponent8(amag);
  scale = (uint32_t)(e + 127);
  uint32_t o[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 4; h++)
    o[h >> 1] |= (e4m3_code(w[h] & 0xFFFFu, e) | (e4m3_code(w[h] >> 16, e) << 8)) << (16 * (h & 1));
  return make_uint2(o[0], o[1]);
}

__global__ __launch_bounds__(256) void quant8_cache_kernel(
    const uint16_t *__restrict__ k, int64_t n_tok, int64_t k_ld, const int64_t *__restrict__ slots,
    uint8_t *__restrict__ kv_packed, uint8_t *__restrict__ kv_scale, int64_t n_pages,
    const uint16_t *__restrict__ q, int64_t n_q_vec, uint8_t *__restrict__ q_packed,
    uint8_t *__restrict__ q_scale) {
  const int64_t total = (n_tok + n_q_vec) * kLanesPerVec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t v = i / kLanesPerVec;
    const int l = (int)(i % kLanesPerVec);
    const int g = l >> 2;
    uint32_t sc;
    if (v < n_tok) {
      const int64_t slot = slots[v];
      if (slot < 0 || slot >= n_pages * kPage) continue;
      const uint2 d = encode8_lane8(*reinterpret_cast<const uint4 *>(k + v * k_ld + 8 * l), sc);
      const int64_t page = slot / kPage;
      const int pos = (int)(slot % kPage);
      *reinterpret_cast<uint2 *>(kv_packed + (page * kPage + pos) * kKeyBytes8 + 8 * l) = d;
      if ((l & 3) == 0) kv_scale[(page * kGroups + g) * kPage + (pos % 16) * 4 + pos / 16] = (uint8_t)sc;
    } else {
      const int64_t vq = v - n_tok;
      const uint2 d = encode8_lane8(*reinterpret_cast<const uint4 *>(q + vq * kHeadDim + 8 * l), sc);
      *reinterpret_cast<uint2 *>(q_packed + vq * kKeyBytes8 + 8 * l) = d;
      if ((l & 3) == 0) q_scale[vq * kGroups + g] = (uint8_t)sc;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Fused writer: key LayerNorm (k_norm), RoPE on keys and query heads, then the MXFP4 write
// above, plus the scorer's per-head weights ("Score a DSA sparse indexer in FP4", commit
// message: the widened writer emits the quantized query and weights_mqa, and k_norm runs
// before the quantizer; review fixes: slot < 0 rows are skipped and their weights_mqa must
// be zero). The pages give no formulas; the kernel takes these readings: LayerNorm over the
// key's 128 elements with the biased variance, (x - mean) / sqrt(var + eps) * gamma + beta;
// RoPE pairs (i, i + rope_dim/2) or (2i, 2i + 1) of the first rope_dim elements, pair i
// turned by the angle whose cos and sin are entries i and rope_dim/2 + i of the position's
// table row; the result rounded once to bf16 (nearest, ties to even) and quantized like
// plain bf16 input; weights_mqa = weight_scale * weights.
//
// Same lane split as the plain writer: 16 lanes per 128-element vector, 8 elements per
// lane, so the LayerNorm sums are 4-step butterflies inside the 16-lane group and a
// half-split rotation partner sits rope_dim/16 lanes away (rope_dim is a multiple of 16).

__global__ __launch_bounds__(256) void norm_rope_quant_cache_kernel(
    const uint16_t *__restrict__ k, int64_t n_tok, int64_t k_ld, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, const int64_t *__restrict__ positions, const float *__restrict__ cos_sin,
    int64_t max_pos, int rope_dim, bool interleaved, const int64_t *__restrict__ slots, uint8_t *__restrict__ kv_packed,
    uint8_t *__restrict__ kv_scale, int64_t n_pages, const uint16_t *__restrict__ q, int n_heads,
    uint8_t *__restrict__ q_packed, uint8_t *__restrict__ q_scale, const float *__restrict__ weights,
    float weight_scale, float *__restrict__ weights_mqa, bool all_q, int32_t *__restrict__ err) {
  const int64_t n_q_vec = q ? n_tok * (int64_t)n_heads : 0;
  const int64_t total = (n_tok + n_q_vec) * kLanesPerVec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t v = i / kLanesPerVec;
    const int l = (int)(i % kLanesPerVec);
    const int g = l >> 2;
    const bool is_key = v < n_tok;
    const int64_t vq = v - n_tok;
    const int64_t t = is_key ? v : vq / n_heads;  // token
    // Every load that needs only (token, lane) goes out first, in one round; only the angle
    // table row waits for the position. Decisions are uniform over the vector's 16 lanes.
    const int64_t pos_raw = rope_dim > 0 ? positions[t] : 0;
    const int64_t slot = slots[t];
    const uint4 raw = *reinterpret_cast<const uint4 *>(is_key ? k + t * k_ld + 8 * l : q + vq * kHeadDim + 8 * l);
    float gm[8], bt[8];
    const bool norm = is_key && gamma;
    if (norm) {
      const float4 g0 = *reinterpret_cast<const float4 *>(gamma + 8 * l), g1 = *reinterpret_cast<const float4 *>(gamma + 8 * l + 4);
      gm[0] = g0.x, gm[1] = g0.y, gm[2] = g0.z, gm[3] = g0.w, gm[4] = g1.x, gm[5] = g1.y, gm[6] = g1.z, gm[7] = g1.w;
      if (beta) {
        const float4 b0 = *reinterpret_cast<const float4 *>(beta + 8 * l), b1 = *reinterpret_cast<const float4 *>(beta + 8 * l + 4);
        bt[0] = b0.x, bt[1] = b0.y, bt[2] = b0.z, bt[3] = b0.w, bt[4] = b1.x, bt[5] = b1.y, bt[6] = b1.z, bt[7] = b1.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; j++) bt[j] = 0.f;
      }
    }
    const float wv = !is_key && l == 0 ? weights[vq] : 0.f;
    const bool bad_pos = rope_dim > 0 && (pos_raw < 0 || pos_raw >= max_pos);
    float c[8], sn[8];
    if (rope_dim > 0 && 8 * l < rope_dim)
      rope_angles(cos_sin + (bad_pos ? 0 : pos_raw) * rope_dim, l, rope_dim, interleaved, c, sn);
    uint32_t sc;
    if (is_key) {
      const bool in_pool = slot >= 0 && slot < n_pages * kPage;
      if (err && l == 0 && (bad_pos || (slot >= 0 && !in_pool)))
        atomicOr(err, (bad_pos ? INDEXER_FP4_DEV_BAD_POSITION : 0) |
                          (slot >= 0 && !in_pool ? INDEXER_FP4_DEV_SLOT_OUT_OF_POOL : 0));
      if (bad_pos || !in_pool) continue;
      const uint32_t d = norm_rope_encode(raw, l, norm, gm, bt, eps, rope_dim, interleaved, c, sn, sc);
      const int64_t page = slot / kPage;
      const int p = (int)(slot % kPage);
      *reinterpret_cast<uint32_t *>(kv_packed + (page * kPage + p) * kKeyBytes + 4 * l) = d;
      if ((l & 3) == 0) kv_scale[(page * kGroups + g) * kPage + (p % 16) * 4 + p / 16] = (uint8_t)sc;
    } else {
      const bool live = !bad_pos && (slot >= 0 || all_q);
      uint32_t d = 0;
      sc = 0;  // a skipped row stores the quantization of a zero vector and weight 0
      if (live) d = norm_rope_encode(raw, l, false, gm, bt, eps, rope_dim, interleaved, c, sn, sc);
      *reinterpret_cast<uint32_t *>(q_packed + vq * kKeyBytes + 4 * l) = d;
      if ((l & 3) == 0) q_scale[vq * kGroups + g] = (uint8_t)sc;
      if (l == 0) weights_mqa[vq] = live ? weight_scale * wv : 0.f;
    }
  }
}

}  // namespace ifp4

using namespace ifp4;

static int quant_and_cache(bool fp8, const void *k_bf16, int64_t n_tok, int64_t k_ld, const int64_t *slot_mapping,
                           uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
                           int64_t n_q_rows, int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale, void *stream) {
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
  const int64_t total = (n_tok + n_q_vec) * kLanesPerVec;
  if (total == 0) return INDEXER_FP4_OK;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fp8 ? quant8_cache_kernel : quant_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, (const uint16_t *)k_bf16, n_tok, k_ld, slot_mapping, kv_packed, kv_scale,
                     n_pages, (const uint16_t *)q_bf16, n_q_vec, q_packed, q_scale);
  return launch_status(fp8 ? "fp8_quant_and_cache" : "quant_and_cache");
}

extern "C" int indexer_fp4_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                           const int64_t *slot_mapping, uint8_t *kv_packed,
                                           uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
                                           int64_t n_q_rows, int32_t n_heads, uint8_t *q_packed,
                                           uint8_t *q_scale, void *stream) {
  return quant_and_cache(false, k_bf16, n_tok, k_ld, slot_mapping, kv_packed, kv_scale, n_pages, q_bf16, n_q_rows,
                         n_heads, q_packed, q_scale, stream);
}

extern "C" int indexer_fp8_quant_and_cache(const void *k_bf16, int64_t n_tok, int64_t k_ld,
                                           const int64_t *slot_mapping, uint8_t *kv_packed,
                                           uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
                                           int64_t n_q_rows, int32_t n_heads, uint8_t *q_packed,
                                           uint8_t *q_scale, void *stream) {
  return quant_and_cache(true, k_bf16, n_tok, k_ld, slot_mapping, kv_packed, kv_scale, n_pages, q_bf16, n_q_rows,
                         n_heads, q_packed, q_scale, stream);
}

extern "C" int indexer_fp4_norm_rope_quant_and_cache(
    const void *k_bf16, int64_t n_tok, int64_t k_ld, const float *k_norm_weight, const float *k_norm_bias, float eps,
    const int64_t *positions, const float *cos_sin, int64_t max_pos, int32_t rope_dim, int32_t rope_interleaved,
    const int64_t *slot_mapping, uint8_t *kv_packed, uint8_t *kv_scale, int64_t n_pages, const void *q_bf16,
    int32_t n_heads, uint8_t *q_packed, uint8_t *q_scale, const float *weights, float weight_scale,
    float *weights_mqa, int32_t all_q, int32_t *err, void *stream) {
  clear_error();
  if (n_tok < 0 || n_pages < 0)
    return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: negative size: n_tok=%lld n_pages=%lld", (long long)n_tok,
                (long long)n_pages);
  if (rope_dim < 0 || rope_dim > kHeadDim || rope_dim % 16 != 0)
    return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: rope_dim=%d must be a multiple of 16 in 0..%d", rope_dim,
                kHeadDim);
  if (!k_norm_weight && k_norm_bias)
    return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: k_norm_bias without k_norm_weight");
  if (!(eps >= 0.f)) return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: eps must be >= 0");
  if (n_tok > 0) {
    if (!k_bf16 || !slot_mapping || !kv_packed || !kv_scale)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: n_tok=%lld needs k, slot_mapping and both planes",
                  (long long)n_tok);
    if (k_ld < kHeadDim || k_ld % 8 != 0)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: k_ld=%lld must be >= %d and a multiple of 8",
                  (long long)k_ld, kHeadDim);
    if (((uintptr_t)k_bf16 | (uintptr_t)kv_packed) % 16 != 0)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: k and kv_packed must be 16-byte aligned");
    if (rope_dim > 0 && (!positions || !cos_sin || max_pos <= 0))
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: rope_dim=%d needs positions and a cos/sin table", rope_dim);
    if (((uintptr_t)cos_sin | (uintptr_t)k_norm_weight | (uintptr_t)k_norm_bias) % 16 != 0)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: cos_sin, k_norm_weight and k_norm_bias must be 16-byte aligned");
  }
  const bool q_arm = q_bf16 != nullptr && n_tok > 0;
  if (q_arm) {
    if (n_heads <= 0) return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: n_heads=%d must be positive", n_heads);
    if (!q_packed || !q_scale || !weights || !weights_mqa)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: the query arm needs q_packed, q_scale, weights and weights_mqa");
    if (((uintptr_t)q_bf16 | (uintptr_t)q_packed) % 16 != 0)
      return fail(INDEXER_FP4_EINVAL, "norm_rope_quant: q and q_packed must be 16-byte aligned");
  }
  int rc = check_device();
  if (rc) return rc;
  const int64_t total = (n_tok + (q_arm ? n_tok * (int64_t)n_heads : 0)) * kLanesPerVec;
  if (total == 0) return INDEXER_FP4_OK;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(norm_rope_quant_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                     (const uint16_t *)k_bf16, n_tok, k_ld, k_norm_weight, k_norm_bias, eps, positions, cos_sin,
                     max_pos, rope_dim, rope_interleaved != 0, slot_mapping, kv_packed, kv_scale, n_pages,
                     q_arm ? (const uint16_t *)q_bf16 : nullptr, n_heads, q_packed, q_scale, weights, weight_scale,
                     weights_mqa, all_q != 0, err);
  return launch_status("norm_rope_quant_and_cache");
}
