// Device helpers shared by the ds4g HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4g {

constexpr int kWave = 64;

// ----------------------------------------------------------- bf16 <-> fp32
// bf16 is the upper half of an fp32: widening is a shift.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round to nearest even (inputs are finite here)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf16_round(float f) {
  return bf16_to_f32(f32_to_bf16(f));
}

// Load a stored scalar of either weight type as float.
__device__ __forceinline__ float ldw(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldw(const float* p, long i) { return p[i]; }

// 8 consecutive weights (16 B of bf16 or 32 B of fp32) widened to fp32.
struct W8 { float v[8]; };
__device__ __forceinline__ void unpack8(const uint4& q, float* f) {
  f[0] = __uint_as_float(q.x << 16); f[1] = __uint_as_float(q.x & 0xFFFF0000u);
  f[2] = __uint_as_float(q.y << 16); f[3] = __uint_as_float(q.y & 0xFFFF0000u);
  f[4] = __uint_as_float(q.z << 16); f[5] = __uint_as_float(q.z & 0xFFFF0000u);
  f[6] = __uint_as_float(q.w << 16); f[7] = __uint_as_float(q.w & 0xFFFF0000u);
}

// 16-byte streaming load (non-temporal: weights are read once per call)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// raw 8-element chunk holder for either type
template <typename WT> struct Chunk8;
template <> struct Chunk8<uint16_t> {
  uint4 q;
  __device__ __forceinline__ void load(const uint16_t* p) {
    q = ldg_nt16(p);
  }
  __device__ __forceinline__ void widen(float* f) const { unpack8(q, f); }
};
template <> struct Chunk8<float> {
  uint4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = ldg_nt16(p);
    b = ldg_nt16(p + 4);
  }
  __device__ __forceinline__ void widen(float* f) const {
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
    f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
    f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
  }
};

// ----------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// (value, index) max with the lower index winning ties
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// Block-wide sum (blockDim.x a multiple of 64, <= 1024); every thread gets it.
__device__ __forceinline__ float block_sum(float v, float* red /*[16]*/) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Make this wave's LDS writes visible to its own lanes (no block barrier):
// waits for outstanding LDS operations; a wave runs its lanes in lockstep.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// RoPE angle of pair i (of rd rotated dims) at position p: theta =
// p * base^(-2i/rd).  The angle is formed and reduced modulo 2*pi in fp64
// (positions reach 1e4..1e6), then sin/cos are taken in fp32 of the reduced
// angle.  Shared by the prefill and decode kernels so both rotate alike.
__device__ __forceinline__ void rope_cs(long p, int i, int rd, float base, float* c, float* s) {
  const double inv = exp2(-(2.0 * (double)i / (double)rd) * log2((double)base));
  const double th = (double)p * inv;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = th - two_pi * rint(th / two_pi);
  sincosf((float)red, s, c);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace ds4g
