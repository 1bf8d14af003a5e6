// Calibration probe for the rooflines this library reports: the rate at
// which the matrix cores retire bf16 MFMAs when nothing else limits them.
// Every wave keeps 8 independent 32x32x16 accumulators in registers and
// issues `iters` rounds of 8 MFMAs on operands that never leave registers;
// one store per wave keeps the work alive.  Dense flops per MFMA:
// 2 * 32 * 32 * 16.
#include "dev.h"
#include "kernels.h"
#include "../../include/ds4g.h"

namespace ds4g {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short probe_bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float probe_f32x16;

__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* out) {
  probe_f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const int lane = threadIdx.x & 63;
  probe_bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (short)(0x3F80 + ((lane + e) & 7));   // bf16 values near 1
    b[e] = (short)(0x3C00 + ((lane * 3 + e) & 7));
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][lane & 15];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace ds4g

extern "C" int ds4g_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return DS4G_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ds4g::mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     iters, out);
  return hipGetLastError() == hipSuccess ? DS4G_OK : DS4G_ERR_HIP;
}
