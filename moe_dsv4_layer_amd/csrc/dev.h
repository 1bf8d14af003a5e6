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
// two values rounded to nearest even in one v_cvt_pk_bf16_f32 (a in the low
// half); the same result as f32_to_bf16 on each for finite inputs
typedef float ds4g_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 ds4g_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(ds4g_f32x2{a, b}, ds4g_bf16x2));
}

// ----------------------------------------------------------- fp16 <-> fp32
// The attention path of a prefill (normalised input, low-rank code, q, k, v,
// probabilities, attention output) and the KV ring carry IEEE binary16: three
// more significand bits than bf16 at the same MFMA rate.  Conversions round
// to nearest even.
typedef _Float16 ds4g_f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(ds4g_f32x2{a, b}, ds4g_f16x2));
}
// 8 fp16 values (16 bytes) widened to fp32
__device__ __forceinline__ void unpack8_f16(const uint4& q, float* f) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const ds4g_f16x2 h = __builtin_bit_cast(ds4g_f16x2, w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
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

// Buffer resource for raw buffer loads from base: no stride, no range check
// (num_records = -1: the caller bounds every offset, 32-bit bytes).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r.z = -1;
  r.w = 0x00020000;         // raw dword access
  return r;
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
// Wave-wide reductions on the DPP lane network (row_shr 1/2/4/8 inside each
// 16-lane row, then row_bcast 15/31 across rows; the total ends in lane 63
// and is read back as a wave-uniform value).  No LDS round trips: about a
// third of the latency of the same butterfly through ds_bpermute, which is
// what every GEMV row result and the router's top-k wait on.
#define DS4G_DPP_F(old, v, ctrl, rm, bc)                                                   \
  __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), ctrl, \
                                             rm, 0xF, bc))
__device__ __forceinline__ float wave_sum(float v) {
  v += DS4G_DPP_F(0.f, v, 0x111, 0xF, true);    // row_shr:1, zero fill
  v += DS4G_DPP_F(0.f, v, 0x112, 0xF, true);    // row_shr:2
  v += DS4G_DPP_F(0.f, v, 0x114, 0xF, true);    // row_shr:4
  v += DS4G_DPP_F(0.f, v, 0x118, 0xF, true);    // row_shr:8 -> lane 15 of each row
  v += DS4G_DPP_F(0.f, v, 0x142, 0xA, false);   // row_bcast:15 into rows 1, 3
  v += DS4G_DPP_F(0.f, v, 0x143, 0xC, false);   // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x111, 0xF, false));
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x112, 0xF, false));
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x114, 0xF, false));
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x118, 0xF, false));
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x142, 0xA, false));
  v = fmaxf(v, DS4G_DPP_F(-INFINITY, v, 0x143, 0xC, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_min(int v) {
#define DS4G_DPP_MIN(ctrl, rm) v = min(v, __builtin_amdgcn_update_dpp(0x7fffffff, v, ctrl, rm, 0xF, false))
  DS4G_DPP_MIN(0x111, 0xF); DS4G_DPP_MIN(0x112, 0xF); DS4G_DPP_MIN(0x114, 0xF);
  DS4G_DPP_MIN(0x118, 0xF); DS4G_DPP_MIN(0x142, 0xA); DS4G_DPP_MIN(0x143, 0xC);
#undef DS4G_DPP_MIN
  return __builtin_amdgcn_readlane(v, 63);
}
// (value, index) max with the lower index winning ties; every lane gets it
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#define DS4G_DPP_ARG(ctrl, rm)                                                   \
  {                                                                              \
    const float ov = DS4G_DPP_F(-INFINITY, v, ctrl, rm, false);                  \
    const int oi = __builtin_amdgcn_update_dpp(0x7fffffff, i, ctrl, rm, 0xF, false); \
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }                       \
  }
  DS4G_DPP_ARG(0x111, 0xF) DS4G_DPP_ARG(0x112, 0xF) DS4G_DPP_ARG(0x114, 0xF)
  DS4G_DPP_ARG(0x118, 0xF) DS4G_DPP_ARG(0x142, 0xA) DS4G_DPP_ARG(0x143, 0xC)
#undef DS4G_DPP_ARG
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// All-reduce inside each 16-lane row (every lane of the row gets the row's
// result): quad_perm swaps for lane distance 1 and 2, then row rotations by
// 4 and 8.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, DS4G_DPP_F(v, v, 0xB1, 0xF, false));    // quad_perm [1,0,3,2]
  v = fmaxf(v, DS4G_DPP_F(v, v, 0x4E, 0xF, false));    // quad_perm [2,3,0,1]
  v = fmaxf(v, DS4G_DPP_F(v, v, 0x124, 0xF, false));   // row_ror:4
  v = fmaxf(v, DS4G_DPP_F(v, v, 0x128, 0xF, false));   // row_ror:8
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += DS4G_DPP_F(v, v, 0xB1, 0xF, false);
  v += DS4G_DPP_F(v, v, 0x4E, 0xF, false);
  v += DS4G_DPP_F(v, v, 0x124, 0xF, false);
  v += DS4G_DPP_F(v, v, 0x128, 0xF, false);
  return v;
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

// ----------------------------------------------------------- routing
// Order-preserving map of a float to an unsigned key (larger float, larger
// key; -0 < +0) and back.
__device__ __forceinline__ unsigned order_key(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_val(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#define DS4G_DPP_MAXU(ctrl, rm) v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, rm, 0xF, false))
  DS4G_DPP_MAXU(0x111, 0xF); DS4G_DPP_MAXU(0x112, 0xF); DS4G_DPP_MAXU(0x114, 0xF);
  DS4G_DPP_MAXU(0x118, 0xF); DS4G_DPP_MAXU(0x142, 0xA); DS4G_DPP_MAXU(0x143, 0xC);
#undef DS4G_DPP_MAXU
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// Router selection: top-k of the E <= 64 NV logits (descending, ties to the
// lower index) and the softmax probabilities of the chosen ones, by one wave
// with the logits in registers (element lane + 64 i, i < NV).  Each lane
// sorts its NV elements by (key descending, index ascending); a round takes
// the wave max of the lanes' heads, then the lowest index among the heads
// that hold it, and the lane that owns it drops its head: two DPP reductions
// and a register shift per round.  A NaN logit ranks as -inf.  Lane r < k
// keeps the r-th choice and writes it to sel[r] / wsel[r] (LDS or global).
template <int NV>
__device__ __forceinline__ void route_topk(const float (&lg)[8], int E, int k, int* sel,
                                           float* wsel) {
  const int lane = threadIdx.x & 63;
  unsigned key[NV];
  int idx[NV];
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    const float x = lg[i];
    v[i] = x == x ? x : -INFINITY;
    key[i] = e < E ? order_key(v[i]) : 0u;   // every valid key is above 0
    idx[i] = e;
  }
  // odd-even transposition sort of the lane's NV entries
#pragma unroll
  for (int pass = 0; pass < NV; ++pass)
#pragma unroll
    for (int a = pass & 1; a + 1 < NV; a += 2) {
      const bool sw = key[a + 1] > key[a] || (key[a + 1] == key[a] && idx[a + 1] < idx[a]);
      const unsigned tk = sw ? key[a + 1] : key[a];
      const int ti = sw ? idx[a + 1] : idx[a];
      key[a + 1] = sw ? key[a] : key[a + 1];
      idx[a + 1] = sw ? idx[a] : idx[a + 1];
      key[a] = tk;
      idx[a] = ti;
    }
  const unsigned m0 = wave_max_u32(key[0]);
  const float m = order_val(m0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) s += (lane + 64 * i < E) ? expf(v[i] - m) : 0.f;
  s = wave_sum(s);
  float mytop = 0.f;
  int myidx = 0;
#pragma unroll 1
  for (int r = 0; r < k; ++r) {
    const unsigned top = (r == 0) ? m0 : wave_max_u32(key[0]);
    const int w = min(wave_min(key[0] == top ? idx[0] : 0x7fffffff), E - 1);
    if (lane == r) { mytop = order_val(top); myidx = w; }
    if (idx[0] == w) {   // the owner drops its head
#pragma unroll
      for (int i = 0; i + 1 < NV; ++i) { key[i] = key[i + 1]; idx[i] = idx[i + 1]; }
      key[NV - 1] = 0u;
    }
  }
  if (lane < k) { sel[lane] = myidx; wsel[lane] = expf(mytop - m) / s; }
}
__device__ __forceinline__ void route_wave(const float (&lg)[8], int E, int k, int* sel,
                                           float* wsel) {
  if (E <= 64) route_topk<1>(lg, E, k, sel, wsel);
  else if (E <= 128) route_topk<2>(lg, E, k, sel, wsel);
  else if (E <= 256) route_topk<4>(lg, E, k, sel, wsel);
  else route_topk<8>(lg, E, k, sel, wsel);
  wave_lds_sync();
}

// RoPE angle of pair i (of rd rotated dims) at position p: theta =
// p * base^(-2i/rd).  The angle is formed and reduced modulo 2*pi in fp64
// (positions reach 1e4..1e6), then sin/cos are taken in fp32 of the reduced
// angle.  Shared by the prefill and decode kernels so both rotate alike.
__device__ __forceinline__ double rope_inv(int i, int rd, float base) {
  return exp2(-(2.0 * (double)i / (double)rd) * log2((double)base));
}
__device__ __forceinline__ void rope_cs_inv(long p, double inv, float* c, float* s) {
  const double th = (double)p * inv;
  const double two_pi = 6.283185307179586476925286766559;
  const double red = th - two_pi * rint(th / two_pi);
  sincosf((float)red, s, c);
}
__device__ __forceinline__ void rope_cs(long p, int i, int rd, float base, float* c, float* s) {
  rope_cs_inv(p, rope_inv(i, rd, base), c, s);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace ds4g
