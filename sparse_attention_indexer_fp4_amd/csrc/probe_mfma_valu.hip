// Throughput probe of the scorers' instruction mix; a measurement kernel, not part of the
// scoring path (built into its own library and run only by bench.py --mfma-valu-probe).
//
// The prefill scorer's page work is 16 block-scaled FP4 MFMAs (16x16x128) per row and an
// epilogue of two fp32 VALU operations per (head, key): a ReLU as an integer max and a fused
// multiply-add into the weighted sum, 128 operations a lane. This kernel runs exactly that
// mix with the operands held in registers (no memory traffic in the timed loop), in waves with
// set roles, so the rate of each kind of work alone and next to the other can be read from
// per-wave clocks and from the SQ counters of each launch:
//   mode 0  two MFMA-only waves a SIMD        mode 3  two waves a SIMD doing both
//   mode 1  two VALU-only waves a SIMD        mode 4  one MFMA-only wave a SIMD
//   mode 2  one MFMA-only and one VALU-only   mode 5  one VALU-only wave a SIMD
// One 512-thread workgroup (8 waves, wave w on SIMD w % 4) per CU -- each reserves 96 KiB of
// LDS it does not use, so no CU takes two -- and a wave's iteration is 16 MFMAs and/or 128 VALU
// operations.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// role of wave w: 0 MFMA, 1 VALU, 2 both, 3 idle
template <int MODE>
__device__ __forceinline__ int role_of(int w) {
  if (MODE == 0) return 0;
  if (MODE == 1) return 1;
  if (MODE == 2) return w < 4 ? 0 : 1;
  if (MODE == 3) return 2;
  if (MODE == 4) return w < 4 ? 0 : 3;
  return w < 4 ? 1 : 3;
}

template <int MODE>
__global__ __launch_bounds__(512) void mfma_valu_probe(const int *__restrict__ in, float *__restrict__ out, int iters,
                                                       long long *__restrict__ cyc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int role = role_of<MODE>(w);
  intx8 a, b;
  for (int i = 0; i < 8; i++) {
    a[i] = in[(lane * 8 + i) & 1023];
    b[i] = in[((lane * 8 + i) & 1023) + 1024];
  }
  // e8m0 scales of 2^-1 or 2^0 (never the NaN code)
  const int sa = (in[lane] & 0x01010101) | 0x7e7e7e7e, sb = (in[lane + 64] & 0x01010101) | 0x7e7e7e7e;
  floatx4 c[16];
  for (int i = 0; i < 16; i++) c[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float v[64], acc[8];
  for (int i = 0; i < 64; i++) v[i] = (float)(in[2048 + ((lane + i) & 1023)] & 0xffff) * 1e-3f - 30.f;
  for (int i = 0; i < 8; i++) acc[i] = 0.f;
  const float wt = (float)(in[3] & 0xff) * 1e-3f;
  const long long r0 = wall_clock64(), t0 = clock64();
  for (int it = 0; it < iters; it++) {
    if (role == 0 || role == 2) {
#pragma unroll
      for (int m = 0; m < 16; m++)
        c[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[m], 4, 4, 0, sa, 0, sb);
    }
    if (role == 1 || role == 2) {
#pragma unroll
      for (int k = 0; k < 64; k++) asm volatile("" : "+v"(v[k]));  // no instruction: the values are new each time
#pragma unroll
      for (int k = 0; k < 64; k++)
        acc[k & 7] = __builtin_fmaf(wt, __int_as_float(max(__float_as_int(v[k]), 0)), acc[k & 7]);
    }
  }
  const long long t1 = clock64(), r1 = wall_clock64();
  float s = 0.f;
  for (int i = 0; i < 16; i++) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  for (int i = 0; i < 8; i++) s += acc[i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
  if (lane == 0) {
    const int g = blockIdx.x * 8 + w;
    cyc[2 * g] = t1 - t0;      // shader clocks
    cyc[2 * g + 1] = r1 - r0;  // 100 MHz wall clock
  }
}

}  // namespace

// in: 4096 ints; out: n_blocks * 512 floats; cyc: n_blocks * 16 int64 (per wave: shader clocks,
// wall-clock ticks). Returns 0, -1 for a mode or size out of range, -2 if the LDS reservation is
// refused, or the HIP error code.
extern "C" int indexer_fp4_probe_mfma_valu(int mode, int iters, int n_blocks, const int *in, float *out,
                                           long long *cyc, void *stream) {
  if (mode < 0 || mode > 5 || iters <= 0 || n_blocks <= 0 || !in || !out || !cyc) return -1;
  hipStream_t st = (hipStream_t)stream;
  constexpr int kLds = 96 * 1024;
  switch (mode) {
#define IFP4_PROBE_CASE(M)                                                                                     \
  case M:                                                                                                      \
    if (hipFuncSetAttribute((const void *)mfma_valu_probe<M>, hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != \
        hipSuccess)                                                                                            \
      return -2;                                                                                               \
    hipLaunchKernelGGL(mfma_valu_probe<M>, dim3(n_blocks), dim3(512), kLds, st, in, out, iters, cyc);         \
    break;
    IFP4_PROBE_CASE(0) IFP4_PROBE_CASE(1) IFP4_PROBE_CASE(2) IFP4_PROBE_CASE(3) IFP4_PROBE_CASE(4) IFP4_PROBE_CASE(5)
#undef IFP4_PROBE_CASE
  }
  return (int)hipGetLastError();
}
