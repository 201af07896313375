// Register-only MFMA rate probe, for benchmarks: how fast this GPU issues
// bf16 MFMAs when nothing else runs, as a function of the operand data.  It is
// not part of the method; it measures the ceiling that the contractions of
// the learner head are compared against.
//
// Each block has 4 waves (one per SIMD).  Each wave keeps 16 independent
// 32x32 fp32 accumulators (256 registers) and multiplies register-resident
// 32x32x16 bf16 fragments in a loop: 16 v_mfma_f32_32x32x16_bf16 per
// iteration, 32768 flops each.  The operands are built in registers from a
// hash of the thread index:
//   mode 0: zeros;
//   mode 1: random signs and mantissas, exponents spread over 2^-3 .. 2^2
//           (the range of normal(0, 1) data);
//   mode 2: the same with exponents 2^-9 .. 2^-4 and 2^-11 .. 2^-6 for the
//           two operands (the magnitudes of LM-head weights and of e).
// The probe reads no memory.  Each thread writes the sum of its accumulators
// to out[blockIdx * 256 + threadIdx], so the results cannot be optimised away.
#include "rz.h"
#include "rz_internal.h"

namespace rz {
namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8_p __attribute__((ext_vector_type(8)));

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// A finite bf16 with random sign and mantissa and a biased exponent in
// [lo, lo + span).
__device__ inline unsigned short random_bf16(uint32_t h, uint32_t lo, uint32_t span) {
  const uint32_t sign = h >> 31;
  const uint32_t e = lo + (h >> 7) % span;
  return static_cast<unsigned short>((sign << 15) | (e << 7) | (h & 0x7Fu));
}

__global__ __launch_bounds__(256) void k_probe_mfma(float* __restrict__ out, int iters, int mode) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  bf16x8_p a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u16x8_p ua, ub;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ha = mix32(tid * 97u + uint32_t(i * 8 + k));
      const uint32_t hb = mix32(tid * 89u + uint32_t(i * 8 + k) + 0x9e3779b9u);
      if (mode == 0) {
        ua[k] = 0;
        ub[k] = 0;
      } else if (mode == 1) {
        ua[k] = random_bf16(ha, 124, 6);
        ub[k] = random_bf16(hb, 124, 6);
      } else {
        ua[k] = random_bf16(ha, 118, 6);
        ub[k] = random_bf16(hb, 116, 6);
      }
    }
    a[i] = __builtin_bit_cast(bf16x8_p, ua);
    b[i] = __builtin_bit_cast(bf16x8_p, ub);
  }
  f32x16_p acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[tid] = s;
}

}  // namespace
}  // namespace rz

extern "C" {

int rz_probe_mfma_peak(float* out, int32_t grid, int32_t iters, int32_t mode, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u)) return RZ_EINVAL;
  if (grid < 1 || grid > 65536 || iters < 1 || iters > 100000000 || mode < 0 || mode > 2)
    return RZ_EINVAL;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return RZ_ENODEV;
  }
  hipLaunchKernelGGL(rz::k_probe_mfma, dim3(uint32_t(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, int(iters), int(mode));
  return hipGetLastError() == hipSuccess ? RZ_OK : RZ_EHIP;
}

}  // extern "C"
