// Register-level building blocks shared by the decode and prefill scorers: a 64-key
// page of the FP4 cache held as MFMA B operands, query rows held as MFMA A operands, and
// the per-page logit (block-scaled FP4 MFMAs, ReLU, head-weighted sum, cross-lane
// reduction). See score_decode.hip for the data movement these registers encode.
#pragma once
#include "common.h"

namespace ifp4 {

struct PageRegs {
  uint4 k[4];  // 4 key tiles x 16 bytes
  uint32_t s;  // scales: byte t = tile t
};

template <int NH16, int NN>
struct RowRegs {
  uint4 qa[NN][NH16];                // query operand per M-tile (16 heads)
  uint32_t qs[NN][(NH16 + 3) / 4];   // query scales, byte m%4 of word m/4
  float4 w[NN][NH16];                // weights of heads 16m + 4(l/16) + i
};

// Row `r` into slot n of R (no wait: the compiler waits where the registers are first used,
// unless the caller waits itself).
template <int NH16, int NN>
__device__ __forceinline__ void load_row_into(RowRegs<NH16, NN> &R, int n, const uint8_t *__restrict__ qp,
                                              const uint8_t *__restrict__ qs, const float *__restrict__ w,
                                              int64_t r, int n_heads, int lane) {
  const int hl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < (NH16 + 3) / 4; j++) R.qs[n][j] = 0;
#pragma unroll
  for (int m = 0; m < NH16; m++) {
    const int64_t v = r * n_heads + 16 * m + hl;
    R.qa[n][m] = *reinterpret_cast<const uint4 *>(qp + v * kKeyBytes + 16 * g);
    R.qs[n][m / 4] |= (uint32_t)qs[v * kGroups + g] << (8 * (m % 4));
    R.w[n][m] = *reinterpret_cast<const float4 *>(w + r * n_heads + 16 * m + 4 * g);
  }
}

template <int NH16, int NN, bool Wait = true>
__device__ __forceinline__ void load_rows(RowRegs<NH16, NN> &R, const uint8_t *__restrict__ qp,
                                          const uint8_t *__restrict__ qs, const float *__restrict__ w,
                                          int64_t row0, int n_valid, int n_heads, int lane) {
  const int hl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int n = 0; n < NN; n++) {
    if (n >= n_valid) break;  // rows past the tile are never read
    const int64_t r = row0 + n;
#pragma unroll
    for (int j = 0; j < (NH16 + 3) / 4; j++) R.qs[n][j] = 0;
#pragma unroll
    for (int m = 0; m < NH16; m++) {
      const int64_t v = r * n_heads + 16 * m + hl;
      R.qa[n][m] = *reinterpret_cast<const uint4 *>(qp + v * kKeyBytes + 16 * g);
      R.qs[n][m / 4] |= (uint32_t)qs[v * kGroups + g] << (8 * (m % 4));
      R.w[n][m] = *reinterpret_cast<const float4 *>(w + r * n_heads + 16 * m + 4 * g);
    }
  }
  // Wait for the query loads here (vmcnt 0; expcnt and lgkmcnt left free). Rows are
  // reloaded only when a wave moves to another sequence or tile; without this wait the
  // compiler would have to assume at every page that the query loads are the youngest in
  // flight and drain the whole page prefetch ring before each page's MFMAs. (Without Wait
  // the caller lets the compiler wait where the registers are first used.)
  if constexpr (Wait) __builtin_amdgcn_s_waitcnt(0x0F70);
}

// One page as B operands. Key bytes are read with the non-temporal hint: each is used once
// per step, and streaming them past the caches measured ~10 % faster than default loads.
__device__ __forceinline__ void load_page(PageRegs &P, const uint8_t *__restrict__ kvp,
                                          const uint8_t *__restrict__ kvs, int64_t phys, int lane) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const uint8_t *base = kvp + phys * kPageBytes + (lane & 15) * kKeyBytes + (lane >> 4) * 16;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + 1024 * t));
    P.k[t] = make_uint4(v.x, v.y, v.z, v.w);
  }
#ifdef IFP4_NT_SCALES
  P.s = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(kvs + phys * kPageScaleBytes + 4 * lane));
#else
  P.s = *reinterpret_cast<const uint32_t *>(kvs + phys * kPageScaleBytes + 4 * lane);
#endif
}

// One page as B operands with default (cached) loads: for pages that other waves or units read
// again soon (prefill: every tile of a request reads the request's pages).
__device__ __forceinline__ void load_page_cached(PageRegs &P, const uint8_t *__restrict__ kvp,
                                                 const uint8_t *__restrict__ kvs, int64_t phys, int lane) {
  const uint8_t *base = kvp + phys * kPageBytes + (lane & 15) * kKeyBytes + (lane >> 4) * 16;
#pragma unroll
  for (int t = 0; t < 4; t++) P.k[t] = *reinterpret_cast<const uint4 *>(base + 1024 * t);
  P.s = *reinterpret_cast<const uint32_t *>(kvs + phys * kPageScaleBytes + 4 * lane);
}

// ReLU on the float's bits: a negative float is a negative int32, so an integer max with 0
// maps it to +0.0 and leaves non-negative values unchanged (one VALU op, and no input
// canonicalization as an IEEE float max would need).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Cross-lane sum of a page's per-tile partial sums: lane 16G + j holds acc[t] = its head
// group G's part of key 16t + j's logit; afterwards lane 16G + j holds key 16G + j's full sum.
// gfx950's lane-swap moves do it in VALU (no LDS round trip): a 32-lane swap of acc[0] with
// acc[2] leaves every lane its own and its partner's (lane ^ 32) sum of the tile it keeps
// (0 or 1 in the low half, 2 or 3 in the high half), likewise acc[1] with acc[3]; a 16-lane
// swap of the two results then pairs lane groups G and G ^ 1. Each addition adds a lane's own
// term and its partner's, so the result is the same whichever operand the swap returns first.
__device__ __forceinline__ float reduce_tiles(const float (&acc)[4]) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0]), __float_as_uint(acc[2]), false, false);
  const float kx = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[1]), __float_as_uint(acc[3]), false, false);
  const float ky = __uint_as_float(y[0]) + __uint_as_float(y[1]);
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(kx), __float_as_uint(ky), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// Logit of key `lane` of the page for row n: sum over heads of w * ReLU(q . k).
// With DB the MFMAs of key tile t+1 are issued into a second set of accumulators before the
// ReLU/weight epilogue of tile t, so the matrix unit works while the VALU reduces; without
// it one set is reused (16 NH16 fewer registers).
template <int NH16, int NN, int N, bool DB = true>
__device__ __forceinline__ float page_logit(const PageRegs &P, const RowRegs<NH16, NN> &R, int lane) {
  float acc[4];
  constexpr int NB = DB ? 2 : 1;
  floatx4 c[NB][NH16];
  auto mfmas = [&](auto tt) {
    constexpr int T = decltype(tt)::value;
    static_for<NH16>([&](auto mm) {
      constexpr int M = decltype(mm)::value;
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      c[T % NB][M] = mfma_fp4<M % 4, T>(R.qa[N][M], P.k[T], zero, R.qs[N][M / 4], P.s);
    });
  };
  auto epilogue = [&](auto tt) {
    constexpr int T = decltype(tt)::value;
    float a = 0.f;
    static_for<NH16>([&](auto mm) {
      constexpr int M = decltype(mm)::value;
      a += R.w[N][M].x * relu(c[T % NB][M][0]);
      a += R.w[N][M].y * relu(c[T % NB][M][1]);
      a += R.w[N][M].z * relu(c[T % NB][M][2]);
      a += R.w[N][M].w * relu(c[T % NB][M][3]);
    });
    acc[T] = a;
  };
  if constexpr (DB) {
    mfmas(std::integral_constant<int, 0>{});
    static_for<4>([&](auto tt) {
      constexpr int T = decltype(tt)::value;
      if constexpr (T + 1 < 4) mfmas(std::integral_constant<int, T + 1>{});
      epilogue(tt);
    });
  } else {
    static_for<4>([&](auto tt) {
      mfmas(tt);
      epilogue(tt);
    });
  }
  // lanes 16G..16G+15 hold, for every tile, partial sums over their heads; reduce across
  // the four lane groups so that lane 16G+j ends with tile G's full sum for key j
  return reduce_tiles(acc);
}

// ---------------------------------------------------------------------------------------
// The same building blocks over MXFP8 (E4M3) queries and keys, for the FP8 comparator. The
// 16x16x128 scaled MFMA takes 32 FP8 bytes per lane; probed on the device, lane group g
// (lanes 16g .. 16g+15) carries K elements [16g, 16g+16) in its first 16 bytes and
// [64+16g, 64+16g+16) in its last 16, while its scale operand applies to the 32-element
// block g, exactly as for FP4. So a lane loads its key's bytes 16g and 64+16g (16 each),
// and the scale plane and its dword per lane are the FP4 ones.

template <int SA, int SB>
__device__ __forceinline__ floatx4 mfma_fp8(const uint4 (&a)[2], const uint4 (&b)[2], floatx4 c, uint32_t sa,
                                            uint32_t sb) {
  intx8 av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w, (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
  intx8 bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w, (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, SA, (int)sa, SB, (int)sb);
}

struct PageRegs8 {
  uint4 k[4][2];  // 4 key tiles x (bytes 16g.., bytes 64+16g..)
  uint32_t s;
};

template <int NH16, int NN>
struct RowRegs8 {
  uint4 qa[NN][NH16][2];
  uint32_t qs[NN][(NH16 + 3) / 4];
  float4 w[NN][NH16];
};

template <int NH16, int NN>
__device__ __forceinline__ void load_rows8(RowRegs8<NH16, NN> &R, const uint8_t *__restrict__ qp,
                                           const uint8_t *__restrict__ qs, const float *__restrict__ w,
                                           int64_t row0, int n_valid, int n_heads, int lane) {
  const int hl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int n = 0; n < NN; n++) {
    if (n >= n_valid) break;
    const int64_t r = row0 + n;
#pragma unroll
    for (int j = 0; j < (NH16 + 3) / 4; j++) R.qs[n][j] = 0;
#pragma unroll
    for (int m = 0; m < NH16; m++) {
      const int64_t v = r * n_heads + 16 * m + hl;
      R.qa[n][m][0] = *reinterpret_cast<const uint4 *>(qp + v * kKeyBytes8 + 16 * g);
      R.qa[n][m][1] = *reinterpret_cast<const uint4 *>(qp + v * kKeyBytes8 + 64 + 16 * g);
      R.qs[n][m / 4] |= (uint32_t)qs[v * kGroups + g] << (8 * (m % 4));
      R.w[n][m] = *reinterpret_cast<const float4 *>(w + r * n_heads + 16 * m + 4 * g);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the query loads, as in load_rows
}

__device__ __forceinline__ void load_page8(PageRegs8 &P, const uint8_t *__restrict__ kvp,
                                           const uint8_t *__restrict__ kvs, int64_t phys, int lane) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const uint8_t *base = kvp + phys * kPageBytes8 + (lane & 15) * kKeyBytes8 + (lane >> 4) * 16;
#pragma unroll
  for (int t = 0; t < 4; t++) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + 2048 * t + 64 * h));
      P.k[t][h] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  P.s = *reinterpret_cast<const uint32_t *>(kvs + phys * kPageScaleBytes + 4 * lane);
}

template <int NH16, int NN, int N>
__device__ __forceinline__ float page_logit8(const PageRegs8 &P, const RowRegs8<NH16, NN> &R, int lane) {
  float acc[4];
  floatx4 c[2][NH16];
  auto mfmas = [&](auto tt) {
    constexpr int T = decltype(tt)::value;
    static_for<NH16>([&](auto mm) {
      constexpr int M = decltype(mm)::value;
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
      c[T & 1][M] = mfma_fp8<M % 4, T>(R.qa[N][M], P.k[T], zero, R.qs[N][M / 4], P.s);
    });
  };
  auto epilogue = [&](auto tt) {
    constexpr int T = decltype(tt)::value;
    float a = 0.f;
    static_for<NH16>([&](auto mm) {
      constexpr int M = decltype(mm)::value;
      a += R.w[N][M].x * relu(c[T & 1][M][0]);
      a += R.w[N][M].y * relu(c[T & 1][M][1]);
      a += R.w[N][M].z * relu(c[T & 1][M][2]);
      a += R.w[N][M].w * relu(c[T & 1][M][3]);
    });
    acc[T] = a;
  };
  mfmas(std::integral_constant<int, 0>{});
  static_for<4>([&](auto tt) {
    constexpr int T = decltype(tt)::value;
    if constexpr (T + 1 < 4) mfmas(std::integral_constant<int, T + 1>{});
    epilogue(tt);
  });
  return reduce_tiles(acc);
}

// Element-format policies of the decode scorer.
struct FmtFp4 {
  using Page = PageRegs;
  template <int NH16, int NN>
  using Rows = RowRegs<NH16, NN>;
  static __device__ __forceinline__ void page(Page &P, const uint8_t *kvp, const uint8_t *kvs, int64_t phys, int lane) {
    load_page(P, kvp, kvs, phys, lane);
  }
  template <int NH16, int NN>
  static __device__ __forceinline__ void rows(Rows<NH16, NN> &R, const uint8_t *qp, const uint8_t *qs, const float *w,
                                              int64_t row0, int n_valid, int n_heads, int lane) {
    load_rows<NH16, NN>(R, qp, qs, w, row0, n_valid, n_heads, lane);
  }
  template <int NH16, int NN, int N>
  static __device__ __forceinline__ float logit(const Page &P, const Rows<NH16, NN> &R, int lane) {
    return page_logit<NH16, NN, N>(P, R, lane);
  }
};

struct FmtFp8 {
  using Page = PageRegs8;
  template <int NH16, int NN>
  using Rows = RowRegs8<NH16, NN>;
  static __device__ __forceinline__ void page(Page &P, const uint8_t *kvp, const uint8_t *kvs, int64_t phys, int lane) {
    load_page8(P, kvp, kvs, phys, lane);
  }
  template <int NH16, int NN>
  static __device__ __forceinline__ void rows(Rows<NH16, NN> &R, const uint8_t *qp, const uint8_t *qs, const float *w,
                                              int64_t row0, int n_valid, int n_heads, int lane) {
    load_rows8<NH16, NN>(R, qp, qs, w, row0, n_valid, n_heads, lane);
  }
  template <int NH16, int NN, int N>
  static __device__ __forceinline__ float logit(const Page &P, const Rows<NH16, NN> &R, int lane) {
    return page_logit8<NH16, NN, N>(P, R, lane);
  }
};

}  // namespace ifp4
