// MXFP4 encoding of bf16 vectors and the fused writer's LayerNorm / RoPE steps, shared by the
// cache writers and the decode scorer that writes its step's key and queries itself.
//
// The element and scale rules are the OCP MX v1.0 ones ("Score a DSA sparse indexer in FP4"
// names the format but prints no rule): scale exponent floor(log2 amax) - 2 clamped to
// [-127, 127]; elements rounded to the nearest E2M1 value, ties to the even code, saturating
// at 6. Four lanes encode one 32-element block (eight elements each), sixteen lanes one
// 128-element vector; the sixteen lanes of a vector are an aligned group of a wave.
#pragma once
#include "common.h"

namespace ifp4 {

constexpr int kLanesPerVec = kHeadDim / 8;  // 16

// Cross-lane moves inside a vector's 16 lanes (one DPP row) with DPP, no LDS round trip:
// the value of lane l ^ 1 or l ^ 2 (quad permutes), and of lane l + n or l - n (row shifts;
// lanes shifted in from outside the row read 0). A DPP move reads lanes that are switched
// off as 0 too, so every move runs with the whole row active and a select follows it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppRowShl = 0x100;  // + n: lane l reads lane l + n
constexpr int kDppRowShr = 0x110;  // + n: lane l reads lane l - n

// Sum over the lanes of the 16-lane row, the same butterfly (and so the same rounding) as
// adding the values of lanes l ^ 1, l ^ 2, l ^ 4, l ^ 8 in turn.
__device__ __forceinline__ float row16_sum(float v) {
  const int l = threadIdx.x & 15;
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  const float dn4 = dpp_f32<kDppRowShr + 4>(v), up4 = dpp_f32<kDppRowShl + 4>(v);
  v += (l & 4) ? dn4 : up4;
  const float dn8 = dpp_f32<kDppRowShr + 8>(v), up8 = dpp_f32<kDppRowShl + 8>(v);
  v += (l & 8) ? dn8 : up8;
  return v;
}

// bf16 bit pattern of the exact value m * 2^p (m in {1, 3, 5, 7}, m * 2^p >= 2^-133; the
// callers keep it below the largest finite bf16).
__device__ __forceinline__ uint32_t bf16_pattern(uint32_t m, int p) {
  const int lm = m >= 4 ? 2 : (m >= 2 ? 1 : 0);  // floor(log2 m)
  const int E = p + lm;
  if (E >= -126) return ((uint32_t)(E + 127) << 7) | ((m << (7 - lm)) & 0x7Fu);
  return m << (p + 133);  // subnormal: the last mantissa bit is 2^-133
}

// The decision points of rounding a magnitude to E2M1 at block scale 2^e, as bf16 bit
// patterns: {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} * 2^e. Bit patterns of non-negative
// bf16 values order like the values, so a magnitude's code is the number of points it
// passes: at the points with an even code below (0.25, 1.25, 2.5, 5) a tie stays below,
// at the others (0.75, 1.75, 3.5) it goes up.
struct E2M1Points {
  uint32_t t[7];
  __device__ __forceinline__ explicit E2M1Points(int e) {
    t[0] = bf16_pattern(1, e - 2);
    t[1] = bf16_pattern(3, e - 2);
    t[2] = bf16_pattern(5, e - 2);
    t[3] = bf16_pattern(7, e - 2);
    t[4] = bf16_pattern(5, e - 1);
    t[5] = bf16_pattern(7, e - 1);
    t[6] = bf16_pattern(5, e);
  }
  __device__ __forceinline__ uint32_t code(uint32_t bits) const {  // bf16 bits -> 4-bit code
    const uint32_t mag = bits & 0x7FFFu;
    const uint32_t c = (mag > t[0]) + (mag >= t[1]) + (mag > t[2]) + (mag >= t[3]) + (mag > t[4]) + (mag >= t[5]) +
                       (mag > t[6]);
    return c | ((bits >> 12) & 8u);
  }
};

// Scale exponent of a block from its largest magnitude (15-bit bf16 pattern):
// floor(log2 amax) - 2, clamped to [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int block_exponent(uint32_t amag) {
  if (amag == 0) return -127;
  const uint32_t ex = amag >> 7;
  const uint32_t sig = ex ? (0x80u | (amag & 0x7Fu)) : (amag & 0x7Fu);
  const int ep = ex ? (int)ex : 1;
  const int e = (31 - __builtin_clz(sig)) + ep - 134 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// This lane's eight bf16 (one uint4) -> four packed bytes (element 2i in the low nibble of
// byte i) and the block's scale byte; the four lanes of a block must be active together.
//
// The codes come from gfx950's scaled conversion (two bf16 -> two E2M1 codes of v / scale
// per instruction, the first in the low nibble). Probed on the device against the threshold
// encoder above for every finite bf16 value at block exponents -10..10, it rounds the same
// way (nearest, ties to the even code, saturating at 6, sign kept), and the exhaustive writer
// test checks it through the library, at the extreme exponents too. Blocks with e <= -124
// (largest magnitude below 2^-121) take the threshold encoder: there a bf16 subnormal could
// reach a nonzero code, and at e = -127 the scale itself is not a normal float.
__device__ __forceinline__ uint32_t encode_lane8(uint4 in, uint32_t &scale) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t amag = 0;
#pragma unroll
  for (int h = 0; h < 4; h++) amag = max(amag, max(w[h] & 0x7FFFu, (w[h] >> 16) & 0x7FFFu));
  amag = max(amag, dpp_u32<kDppXor1>(amag));
  amag = max(amag, dpp_u32<kDppXor2>(amag));
  const int e = block_exponent(amag);
  scale = (uint32_t)(e + 127);
  uint32_t d = 0;
  if (e > -124) {
    const float s = __uint_as_float(scale << 23);  // 2^e, a normal float
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[0]), s, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[1]), s, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[2]), s, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d, __builtin_bit_cast(bf16x2, w[3]), s, 3);
  } else {
    const E2M1Points pts(e);
#pragma unroll
    for (int h = 0; h < 4; h++) d |= (pts.code(w[h] & 0xFFFFu) | (pts.code(w[h] >> 16) << 4)) << (8 * h);
  }
  return d;
}

// ---------------------------------------------------------------------------------------
// Fused-writer steps ("Score a DSA sparse indexer in FP4", commit message: k_norm runs before
// the quantizer; the readings: LayerNorm over the key's 128 elements with the biased
// variance, (x - mean) / sqrt(var + eps) * gamma + beta; RoPE pairs (i, i + rope_dim/2) or
// (2i, 2i + 1) of the first rope_dim elements, pair i turned by the angle whose cos and sin
// are entries i and rope_dim/2 + i of the position's table row; the result rounded once to
// bf16, nearest, ties to even). The LayerNorm sums are 4-step butterflies inside the 16-lane
// group and a half-split rotation partner sits rope_dim/16 lanes away (rope_dim is a
// multiple of 16).

__device__ __forceinline__ float bf16_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, nearest, ties to even (finite input).
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float group16_sum(float v) { return row16_sum(v); }

// x[j] of lane l + h for the lanes l < h, and of lane l - h for the others (the half-split
// rotation partner, h = rope_dim / 16 lanes away).
template <int H>
__device__ __forceinline__ void rope_partner(const float x[8], float part[8], int l) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const float up = dpp_f32<kDppRowShl + H>(x[j]), dn = dpp_f32<kDppRowShr + H>(x[j]);
    part[j] = l < H ? up : dn;
  }
}

__device__ __forceinline__ void unpack8(uint4 in, float x[8]) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
  for (int h = 0; h < 4; h++) {
    x[2 * h] = bf16_to_float(w[h] & 0xFFFFu);
    x[2 * h + 1] = bf16_to_float(w[h] >> 16);
  }
}

__device__ __forceinline__ uint4 pack8(const float x[8]) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 4; h++) w[h] = float_to_bf16(x[2 * h]) | (float_to_bf16(x[2 * h + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// This lane's angle-table entries: element 8l + j of a rotated vector uses cos c[j] and sin
// sn[j] (entries m and rope_dim/2 + m of the row, m its pair index). All 16 B loads: rope_dim
// is a multiple of 16 and the table 16-byte aligned.
__device__ __forceinline__ void rope_angles(const float *__restrict__ row, int l, int rope_dim, bool interleaved,
                                            float c[8], float sn[8]) {
  const int half = rope_dim >> 1;
  if (interleaved) {  // pairs (2m, 2m+1): m = 4l .. 4l+3, each used twice
    const float4 c4 = *reinterpret_cast<const float4 *>(row + 4 * l);
    const float4 s4 = *reinterpret_cast<const float4 *>(row + half + 4 * l);
    const float cc[4] = {c4.x, c4.y, c4.z, c4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int j = 0; j < 8; j++) {
      c[j] = cc[j >> 1];
      sn[j] = ss[j >> 1];
    }
  } else {  // pairs (m, m + half): m = (8l mod half) .. +7
    const int m0 = (8 * l) % half;
    const float4 c0 = *reinterpret_cast<const float4 *>(row + m0), c1 = *reinterpret_cast<const float4 *>(row + m0 + 4);
    const float4 s0 = *reinterpret_cast<const float4 *>(row + half + m0);
    const float4 s1 = *reinterpret_cast<const float4 *>(row + half + m0 + 4);
    const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; j++) {
      c[j] = cc[j];
      sn[j] = ss[j];
    }
  }
}

// Rotates this lane's elements 8l .. 8l+7 in place. All 16 lanes of the group call it.
__device__ __forceinline__ void rope8(float x[8], int l, int rope_dim, bool interleaved, const float c[8],
                                      const float sn[8]) {
  const int half = rope_dim >> 1;
  float part[8];
  if (interleaved) {
#pragma unroll
    for (int j = 0; j < 8; j++) part[j] = x[j ^ 1];
  } else {  // partner lane: l +- half/8 inside the group
    switch (half >> 3) {
      case 1: rope_partner<1>(x, part, l); break;
      case 2: rope_partner<2>(x, part, l); break;
      case 3: rope_partner<3>(x, part, l); break;
      case 4: rope_partner<4>(x, part, l); break;
      case 5: rope_partner<5>(x, part, l); break;
      case 6: rope_partner<6>(x, part, l); break;
      case 7: rope_partner<7>(x, part, l); break;
      default: rope_partner<8>(x, part, l); break;
    }
  }
  if (8 * l >= rope_dim) return;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const bool first = interleaved ? (j & 1) == 0 : 8 * l < half;
    // this element a, its partner b: the first of a pair becomes a cos - b sin, the second a cos + b sin
    x[j] = first ? x[j] * c[j] - part[j] * sn[j] : x[j] * c[j] + part[j] * sn[j];
  }
}

// Key lane l: LayerNorm (with gm / bt when norm), RoPE (angles c / sn when rope_dim > 0),
// then MXFP4: the lane's four packed bytes, its block's scale byte in sc. All 16 lanes of
// the vector call it together.
__device__ __forceinline__ uint32_t norm_rope_encode(uint4 raw, int l, bool norm, const float gm[8], const float bt[8],
                                                     float eps, int rope_dim, bool interleaved, const float c[8],
                                                     const float sn[8], uint32_t &sc) {
  float x[8];
  unpack8(raw, x);
  if (norm) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) s += x[j];
    const float mean = group16_sum(s) * (1.0f / kHeadDim);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      x[j] -= mean;
      ss += x[j] * x[j];
    }
    const float inv = 1.0f / sqrtf(group16_sum(ss) * (1.0f / kHeadDim) + eps);
#pragma unroll
    for (int j = 0; j < 8; j++) x[j] = x[j] * inv * gm[j] + bt[j];
  }
  if (rope_dim > 0) rope8(x, l, rope_dim, interleaved, c, sn);
  return encode_lane8(pack8(x), sc);
}

}  // namespace ifp4
