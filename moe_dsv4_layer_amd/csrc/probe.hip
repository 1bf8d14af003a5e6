// Calibration probes for the rooflines and launch costs this library
// reports.
//  * mfma_loop_kernel: the rate at which the matrix cores retire bf16 MFMAs
//    when nothing else limits them.  Every wave keeps 8 independent
//    32x32x16 accumulators in registers and issues `iters` rounds of 8 MFMAs
//    on operands that never leave registers; one store per wave keeps the
//    work alive.  Dense flops per MFMA: 2 * 32 * 32 * 16.
//  * mfma_random_kernel: the same loop on operands with random signs and
//    mantissas (exponent fixed, |v| in [0.5, 1)): 8 operand sets per wave
//    rotate so every MFMA sees new bits, as a GEMM on random data does.
//  * read_probe_kernel: the HBM read rate of a given access shape (a
//    contiguous stream, or the walk of an MFMA GEMM over a weight panel).
//  * chain_probe_kernel: the cost of one more launch in a stream or graph,
//    with or without a read of the previous launch's output.
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

__device__ __forceinline__ unsigned probe_mix(unsigned x) {   // xorshift32
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

__global__ void __launch_bounds__(256) mfma_random_kernel(int iters, unsigned seed, float* out) {
  probe_f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  unsigned x = probe_mix(seed ^ (blockIdx.x * 256u + threadIdx.x) * 2654435761u) | 1u;
  u32x4_t a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x = probe_mix(x);
      a[j][e] = (x & 0x807F807Fu) | 0x3F003F00u;   // two bf16: random sign, mantissa
      x = probe_mix(x);
      b[j][e] = (x & 0x807F807Fu) | 0x3F003F00u;
    }
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(probe_bf16x8, a[(j + r) & 7]),
            __builtin_bit_cast(probe_bf16x8, b[(j + 3 * r) & 7]), acc[j], 0, 0, 0);
  }
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][lane & 15];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// The source is rows of `row_stride` bytes, of which the first 8192 are
// read.  A unit is `step_rows` consecutive rows, read in steps of 32 KB: step
// s takes bytes [s*C, (s+1)*C) of every row of the unit, C = 32768 /
// step_rows, as an MFMA GEMM's K loop walks a weight panel.  step_rows = 4 is
// a contiguous stream (one step covers 4 whole rows).  Block b reads a
// contiguous range of units, its steps in order, three steps (96 KB) per
// batch with every load issued before any is used; each thread loads
// 8 x 16 bytes per step and xors them into one word.
__global__ void __launch_bounds__(256) read_probe_kernel(const char* __restrict__ src,
                                                         long n_units, int step_rows,
                                                         long row_stride,
                                                         unsigned* __restrict__ out) {
  const int cpr = 2048 / step_rows;            // 16-byte chunks of a row per step
  const long spu = step_rows / 4;               // steps per unit
  const long u0 = n_units * blockIdx.x / gridDim.x;
  const long u1 = n_units * (blockIdx.x + 1) / gridDim.x;
  const long f1 = u1 * spu;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (long f = u0 * spu; f < f1; f += 3) {
    u32x4_t v[3][8];
#pragma unroll
    for (int j3 = 0; j3 < 3; ++j3) {
      const long ff = f + j3;
      const long u = ff / spu, st = ff - u * spu;
      const char* base = src + u * step_rows * row_stride + st * cpr * 16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = threadIdx.x + 256 * j;
        const int r = idx / cpr, c = idx - r * cpr;
        v[j3][j] = ff < f1 ? *reinterpret_cast<const u32x4_t*>(base + r * row_stride + c * 16)
                           : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j3 = 0; j3 < 3; ++j3)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc ^= v[j3][j];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// One launch of a chain: chained, every thread reads the word the previous
// launch wrote (in[0]) and thread 0 writes in[0] + 1 to out[0]; otherwise
// thread 0 only writes 1.
__global__ void __launch_bounds__(256) chain_probe_kernel(const unsigned* in, unsigned* out,
                                                          int chained) {
  unsigned v = 1u;
  if (chained) v = __builtin_nontemporal_load(in) + 1u;
  if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = v;
}

}  // namespace ds4g

extern "C" int ds4g_probe_read(const void* src, int64_t src_bytes, int32_t step_rows,
                               int64_t row_stride, int64_t read_bytes, int32_t blocks,
                               uint32_t* out, void* stream) {
  if (!src || !out || blocks <= 0 || step_rows < 4 || step_rows > 2048 ||
      (step_rows & (step_rows - 1)) != 0 || row_stride < 8192 || row_stride % 16 != 0 ||
      read_bytes <= 0 || read_bytes % ((int64_t)step_rows * 8192) != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return DS4G_ERR_INVALID_ARG;
  const int64_t n_units = read_bytes / ((int64_t)step_rows * 8192);
  // the last unit's last row ends 8192 bytes into it
  if (((n_units * step_rows - 1) * row_stride + 8192) > src_bytes) return DS4G_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ds4g::read_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const char*>(src), (long)n_units, (int)step_rows,
                     (long)row_stride, reinterpret_cast<unsigned*>(out));
  return hipGetLastError() == hipSuccess ? DS4G_OK : DS4G_ERR_HIP;
}

extern "C" int ds4g_probe_chain(int32_t blocks, int32_t n_kernels, int32_t chained,
                                uint32_t* buf, void* stream) {
  if (blocks <= 0 || n_kernels <= 0 || !buf) return DS4G_ERR_INVALID_ARG;
  (void)hipGetLastError();
  unsigned* w = reinterpret_cast<unsigned*>(buf);
  for (int i = 0; i < n_kernels; ++i)
    hipLaunchKernelGGL(ds4g::chain_probe_kernel, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, w + (i & 1), w + ((i + 1) & 1), (int)chained);
  return hipGetLastError() == hipSuccess ? DS4G_OK : DS4G_ERR_HIP;
}

extern "C" int ds4g_probe_mfma_random(int32_t blocks, int32_t iters, uint32_t seed, float* out,
                                      void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return DS4G_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ds4g::mfma_random_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     iters, seed, out);
  return hipGetLastError() == hipSuccess ? DS4G_OK : DS4G_ERR_HIP;
}

extern "C" int ds4g_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return DS4G_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(ds4g::mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     iters, out);
  return hipGetLastError() == hipSuccess ? DS4G_OK : DS4G_ERR_HIP;
}
