// Single-token (decode) kernels: every weight byte is read once, so these are
// HBM-bound GEMVs.  Weights stream with 16-byte non-temporal loads; the
// activation vector lives in registers (each wave holds the K-slice it needs),
// dot products reduce with wave shuffles.  RMSNorm is fused into the GEMV that
// consumes it; the MoE gate/up kernel picks its experts itself from the router
// logits, so routing costs no extra launch.
//
// Follows the layer of ds4-learning 端到端推理流程, 阶段四 4.2 单层前向.
#include "dev.h"
#include "kernels.h"

namespace ds4g {

// ---------------------------------------------------------------------------
// Generic GEMV: out[n] (=|+=) sum_k W[n, k] * xs[k],  xs = x (optionally
// RMSNorm(x) * gamma).  A block is 4 waves; the waves split K in KSPLIT parts
// and the rows of the block in 4/KSPLIT groups.  Each wave handles RB rows at
// a time with CPL 8-element chunks per lane per row (K <= KSPLIT*CPL*512).
// Blocks stride over row groups so the x slice is loaded once per wave.
template <typename WT, int KSPLIT, int CPL, int RB>
__global__ void __launch_bounds__(256)
gemv_kernel(const WT* __restrict__ W, int N, int K, const float* __restrict__ x,
            const WT* __restrict__ gamma, float eps, float* __restrict__ out,
            int accumulate, int64_t* pos_inc) {
  constexpr int RSPLIT = 4 / KSPLIT;
  __shared__ float red[4][RB];
  __shared__ float ssq[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int kpart = wid % KSPLIT, rgroup = wid / KSPLIT;
  const int nchunk = K >> 3;

  if (pos_inc && blockIdx.x == 0 && threadIdx.x == 0) *pos_inc += 1;

  // x slice in registers
  float xv[CPL][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = (kpart * CPL + i) * 64 + lane;
    if (c < nchunk) {
      const float4 a = reinterpret_cast<const float4*>(x)[2 * c];
      const float4 b = reinterpret_cast<const float4*>(x)[2 * c + 1];
      xv[i][0] = a.x; xv[i][1] = a.y; xv[i][2] = a.z; xv[i][3] = a.w;
      xv[i][4] = b.x; xv[i][5] = b.y; xv[i][6] = b.z; xv[i][7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xv[i][e] * xv[i][e];
  }
  if (gamma) {
    ss = wave_sum(ss);
    if (lane == 0) ssq[wid] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int p = 0; p < KSPLIT; ++p) tot += ssq[rgroup * KSPLIT + p];
    const float rs = rsqrtf(tot / (float)K + eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (kpart * CPL + i) * 64 + lane;
      if (c < nchunk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] = xv[i][e] * rs * ldw(gamma, c * 8 + e);
      }
    }
  }

  const int rows_per_block = RB * RSPLIT;
  for (int r0 = blockIdx.x * rows_per_block; r0 < N; r0 += gridDim.x * rows_per_block) {
    const int rbase = r0 + rgroup * RB;
    Chunk8<WT> ch[RB][CPL];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (kpart * CPL + i) * 64 + lane;
        if (rbase + r < N && c < nchunk) ch[r][i].load(W + (long)(rbase + r) * K + c * 8);
      }
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      acc[r] = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (kpart * CPL + i) * 64 + lane;
        if (rbase + r < N && c < nchunk) {
          float f[8];
          ch[r][i].widen(f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r] += f[e] * xv[i][e];
        }
      }
      acc[r] = wave_sum(acc[r]);
    }
    if (KSPLIT == 1) {
      if (lane < RB && rbase + lane < N) {
        float a = acc[0];
#pragma unroll
        for (int r = 1; r < RB; ++r) if (lane == r) a = acc[r];
        out[rbase + lane] = accumulate ? out[rbase + lane] + a : a;
      }
    } else {
      __syncthreads();
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) red[wid][r] = acc[r];
      }
      __syncthreads();
      if (kpart == 0 && lane < RB && rbase + lane < N) {
        float a = 0.f;
#pragma unroll
        for (int p = 0; p < KSPLIT; ++p) a += red[rgroup * KSPLIT + p][lane];
        out[rbase + lane] = accumulate ? out[rbase + lane] + a : a;
      }
    }
  }
}

template <typename WT>
int launch_gemv(const WT* W, int N, int K, const float* x, const WT* gamma, float eps,
                float* out, int accumulate, int64_t* pos_inc, hipStream_t st) {
  const int nchunk = K / 8;
  int grid;
#define DS4G_GEMV(KS, C, R)                                                      \
  {                                                                              \
    const int rpb = R * (4 / KS);                                                \
    grid = (N + rpb - 1) / rpb;                                                  \
    if (grid > 4096) grid = 4096;                                                \
    hipLaunchKernelGGL((gemv_kernel<WT, KS, C, R>), dim3(grid), dim3(256), 0, st, \
                       W, N, K, x, gamma, eps, out, accumulate, pos_inc);        \
    return 0;                                                                    \
  }
  if (nchunk <= 64) DS4G_GEMV(1, 1, 2)          // K <= 512
  if (nchunk <= 128) DS4G_GEMV(1, 2, 2)         // K <= 1024
  if (nchunk <= 256) DS4G_GEMV(4, 1, 2)         // K <= 2048
  if (nchunk <= 512) DS4G_GEMV(4, 2, 2)         // K <= 4096
  if (nchunk <= 1024) DS4G_GEMV(4, 4, 2)        // K <= 8192
  if (nchunk <= 2048) DS4G_GEMV(4, 8, 1)        // K <= 16384
#undef DS4G_GEMV
  return -1;
}
template int launch_gemv<uint16_t>(const uint16_t*, int, int, const float*, const uint16_t*,
                                   float, float*, int, int64_t*, hipStream_t);
template int launch_gemv<float>(const float*, int, int, const float*, const float*, float,
                                float*, int, int64_t*, hipStream_t);

// ---------------------------------------------------------------------------
// Router selection shared by the decode MoE kernels: top-k of E logits
// (descending, ties to the lower index) and softmax probabilities of the
// chosen ones.  Run by one wave; results in sel[]/wsel[].
__device__ void route_one(const float* __restrict__ logits, int E, int k, int* sel,
                          float* wsel) {
  const int lane = threadIdx.x & 63;
  float v[8];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? logits[e] : -INFINITY;
    m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (lane + 64 * i < E) s += expf(v[i] - m);
  s = wave_sum(s);
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
    wave_argmax(bv, bi);
    if (lane == 0) { sel[r] = bi; wsel[r] = expf(bv - m) / s; }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (lane + 64 * i == bi) v[i] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// MoE gate/up for one token: for each chosen expert slot s (k routed + the
// shared expert in slot k) and inner row i:  z[s, i] = silu(G y) * (U y)
// with y = RMSNorm(h2) * g2.  A block = 4 waves splitting K = hidden; each
// wave does RB (gate, up) row pairs.  Every block routes for itself; block 0
// publishes the routing (sel/wsel to the workspace, optional outputs).


template <typename WT, int CPL, int RB>
__global__ void __launch_bounds__(256)
moe_gateup_decode(MoeDecodeArgs a) {
  __shared__ int sel[9];
  __shared__ float wsel[9];
  __shared__ float ssq[4];
  __shared__ float red[4][RB][2];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nchunk = a.d >> 3;
  if (wid == 0) route_one(a.logits, a.E, a.k, sel, wsel);

  // y slice: wave w holds chunks [w*CPL*64, (w+1)*CPL*64)
  float yv[CPL][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = (wid * CPL + i) * 64 + lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      yv[i][e] = (c < nchunk) ? a.h2[c * 8 + e] : 0.f;
      ss += yv[i][e] * yv[i][e];
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) ssq[wid] = ss;
  __syncthreads();
  const float rs = rsqrtf((ssq[0] + ssq[1] + ssq[2] + ssq[3]) / (float)a.d + a.eps);
  const WT* g2 = static_cast<const WT*>(a.ffn_norm);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = (wid * CPL + i) * 64 + lane;
    if (c < nchunk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[i][e] = yv[i][e] * rs * ldw(g2, c * 8 + e);
    }
  }

  if (blockIdx.x == 0) {
    // publish routing (one token: perm lists the k entries by expert)
    if (threadIdx.x < a.k) {
      a.sel[threadIdx.x] = sel[threadIdx.x];
      a.wsel[threadIdx.x] = wsel[threadIdx.x];
      if (a.topk_idx) a.topk_idx[threadIdx.x] = sel[threadIdx.x];
      if (a.topk_w) a.topk_w[threadIdx.x] = wsel[threadIdx.x];
      if (a.perm) {
        int r = 0;
        for (int j = 0; j < a.k; ++j) r += sel[j] < sel[threadIdx.x];
        a.perm[r] = threadIdx.x;
      }
    }
    if (a.count || a.offset) {
      for (int e = threadIdx.x; e <= a.E; e += blockDim.x) {
        int c = 0, o = 0;
        for (int j = 0; j < a.k; ++j) { c += sel[j] == e; o += sel[j] < e; }
        if (a.count && e < a.E) a.count[e] = c;
        if (a.offset) a.offset[e] = o;
      }
    }
    if (a.router_in) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (wid * CPL + i) * 64 + lane;
        if (c < nchunk)
#pragma unroll
          for (int e = 0; e < 8; ++e) a.router_in[c * 8 + e] = yv[i][e];
      }
    }
  }

  const int ntask = a.k * a.I + a.Is;
  for (int t0 = blockIdx.x * RB; t0 < ntask; t0 += gridDim.x * RB) {
    Chunk8<WT> cg[RB][CPL], cu[RB][CPL];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      if (t >= ntask) continue;
      const WT *G, *U;
      if (t < a.k * a.I) {
        const int s = t / a.I, i = t - s * a.I;
        const long base = ((long)sel[s] * a.I + i) * a.d;
        G = static_cast<const WT*>(a.gate) + base;
        U = static_cast<const WT*>(a.up) + base;
      } else {
        const long base = (long)(t - a.k * a.I) * a.d;
        G = static_cast<const WT*>(a.sh_gate) + base;
        U = static_cast<const WT*>(a.sh_up) + base;
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (wid * CPL + i) * 64 + lane;
        if (c < nchunk) { cg[r][i].load(G + c * 8); cu[r][i].load(U + c * 8); }
      }
    }
    float ag[RB], au[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      ag[r] = 0.f; au[r] = 0.f;
      if (t0 + r < ntask) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = (wid * CPL + i) * 64 + lane;
          if (c < nchunk) {
            float f[8], g[8];
            cg[r][i].widen(f);
            cu[r][i].widen(g);
#pragma unroll
            for (int e = 0; e < 8; ++e) { ag[r] += f[e] * yv[i][e]; au[r] += g[e] * yv[i][e]; }
          }
        }
      }
      ag[r] = wave_sum(ag[r]);
      au[r] = wave_sum(au[r]);
    }
    __syncthreads();
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) { red[wid][r][0] = ag[r]; red[wid][r][1] = au[r]; }
    }
    __syncthreads();
    if (wid == 0 && lane < RB && t0 + lane < ntask) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) { g += red[p][lane][0]; u += red[p][lane][1]; }
      a.z[t0 + lane] = silu(g) * u;
    }
  }
}

// MoE down + combine + residual for one token:
//   x[n] = h2[n] + sum_s w_s (D_{e_s} z_s)[n] + (D_sh z_sh)[n]
// One wave per RB output rows; K = I per expert; the sum over slots runs in
// slot order, then the shared expert, then the residual (fixed order).
template <typename WT, int CPL, int RB>
__global__ void __launch_bounds__(256)
moe_down_decode(MoeDecodeArgs a, float* x) {
  extern __shared__ float zs[];   // [k*I + Is]
  __shared__ int sel[9];
  __shared__ float wsel[9];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nz = a.k * a.I + a.Is;
  for (int i = threadIdx.x; i < nz; i += blockDim.x) zs[i] = a.z[i];
  if (threadIdx.x < a.k) { sel[threadIdx.x] = a.sel[threadIdx.x]; wsel[threadIdx.x] = a.wsel[threadIdx.x]; }
  __syncthreads();

  const int nwaves = gridDim.x * 4;
  for (int n0 = (blockIdx.x * 4 + wid) * RB; n0 < a.d; n0 += nwaves * RB) {
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;
    for (int s = 0; s <= a.k; ++s) {
      const int Ks = (s < a.k) ? a.I : a.Is;
      const WT* D = (s < a.k) ? static_cast<const WT*>(a.down) + (long)sel[s] * a.d * a.I
                              : static_cast<const WT*>(a.sh_down);
      const float* zz = zs + s * a.I;
      const float wgt = (s < a.k) ? wsel[s] : 1.0f;
      Chunk8<WT> ch[RB][CPL];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = i * 64 + lane;
          if (n0 + r < a.d && c * 8 < Ks) ch[r][i].load(D + (long)(n0 + r) * Ks + c * 8);
        }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = i * 64 + lane;
          if (n0 + r < a.d && c * 8 < Ks) {
            float f[8];
            ch[r][i].widen(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) p += f[e] * zz[c * 8 + e];
          }
        }
        acc[r] += wgt * wave_sum(p);
      }
    }
    if (lane < RB && n0 + lane < a.d) {
      float v = acc[0];
#pragma unroll
      for (int r = 1; r < RB; ++r) if (lane == r) v = acc[r];
      x[n0 + lane] = a.h2[n0 + lane] + v;
    }
  }
}

template <typename WT>
int launch_moe_decode(const MoeDecodeArgs& a, float* x, hipStream_t st) {
  // gate/up: K = d split over 4 waves
  const int nchunk = a.d / 8;
  const int ntask = a.k * a.I + a.Is;
  int cpl = (nchunk + 255) / 256;
  constexpr int RB = 2;
  int grid = (ntask + RB - 1) / RB;
  if (grid > 4096) grid = 4096;
  if (cpl <= 1)
    hipLaunchKernelGGL((moe_gateup_decode<WT, 1, RB>), dim3(grid), dim3(256), 0, st, a);
  else if (cpl <= 2)
    hipLaunchKernelGGL((moe_gateup_decode<WT, 2, RB>), dim3(grid), dim3(256), 0, st, a);
  else if (cpl <= 4)
    hipLaunchKernelGGL((moe_gateup_decode<WT, 4, RB>), dim3(grid), dim3(256), 0, st, a);
  else
    return -1;
  // down: K = I (or Is) per slot, whole rows per wave
  const int kmax = a.I > a.Is ? a.I : a.Is;
  const int cpl2 = (kmax / 8 + 63) / 64;
  const size_t lds = (size_t)ntask * sizeof(float);
  int grid2 = (a.d + 4 * 2 - 1) / (4 * 2);
  if (cpl2 <= 1)
    hipLaunchKernelGGL((moe_down_decode<WT, 1, 2>), dim3(grid2), dim3(256), lds, st, a, x);
  else if (cpl2 <= 2)
    hipLaunchKernelGGL((moe_down_decode<WT, 2, 2>), dim3(grid2), dim3(256), lds, st, a, x);
  else if (cpl2 <= 4)
    hipLaunchKernelGGL((moe_down_decode<WT, 4, 2>), dim3(grid2), dim3(256), lds, st, a, x);
  else
    return -1;
  return 0;
}
template int launch_moe_decode<uint16_t>(const MoeDecodeArgs&, float*, hipStream_t);
template int launch_moe_decode<float>(const MoeDecodeArgs&, float*, hipStream_t);

}  // namespace ds4g
