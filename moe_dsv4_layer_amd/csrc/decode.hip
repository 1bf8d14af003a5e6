// Single-token (decode) kernels.  One decode token reads every weight it
// needs exactly once, so these are HBM-bound GEMVs: weights stream with
// 16-byte non-temporal loads that are issued before anything else a block
// does (norm prologues, routing reads), the activation vector lives in
// registers, dot products reduce with wave shuffles.  RMSNorm is fused into
// the GEMV that consumes it.  Every MoE gate/up block picks the top-k from
// the router logits itself (a few hundred logits from L2): cheaper than any
// cross-block hand-off, which on this chip needs a full L2 write-back.
//
// Follows the layer of ds4-learning 端到端推理流程, 阶段四 4.2 单层前向.
#include "dev.h"
#include "kernels.h"

#include <algorithm>

// Launch shapes (rows in flight per block, grid caps); measured choices.
#ifndef DS4G_GEMV_GRID_MAX
#define DS4G_GEMV_GRID_MAX 2048
#endif
#ifndef DS4G_GEMV_RB_K8K
#define DS4G_GEMV_RB_K8K 4
#endif
#ifndef DS4G_GATEUP_RB
#define DS4G_GATEUP_RB 4
#endif
#ifndef DS4G_GATEUP_GRID_MAX
#define DS4G_GATEUP_GRID_MAX 896
#endif
#ifndef DS4G_DOWN_RB
#define DS4G_DOWN_RB 16
#endif
#ifndef DS4G_ROUTER_SHARED_RB
#define DS4G_ROUTER_SHARED_RB 2
#endif
#ifndef DS4G_SHGU_GRID_MAX   // blocks of the gate/up launch that compute the shared gate/up
#define DS4G_SHGU_GRID_MAX 128
#endif

namespace ds4g {

// ---------------------------------------------------------------------------
// GEMV.  A block is 4 waves that split K in KSPLIT parts and the block's rows
// in 4/KSPLIT groups; each wave handles RB rows at a time with CPL 8-element
// chunks per lane per row (K <= KSPLIT*CPL*512).  Blocks stride over row
// groups; the next group's loads are issued before the current group's
// reductions.
template <typename WT, int KSPLIT, int CPL, int RB>
__global__ void __launch_bounds__(256)
gemv_kernel(GemvArgs a) {
  constexpr int RSPLIT = 4 / KSPLIT;
  __shared__ float red[4][RB];
  __shared__ float ssq[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int kpart = wid % KSPLIT, rgroup = wid / KSPLIT;
  const int N = a.N, K = a.K, nchunk = K >> 3;
  const WT* W = static_cast<const WT*>(a.W);
  const int rows_per_block = RB * RSPLIT;
  const int stride = gridDim.x * rows_per_block;

  Chunk8<WT> ch[RB][CPL];
  auto load_rows = [&](int r0) {
    const int rbase = r0 + rgroup * RB;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (kpart * CPL + i) * 64 + lane;
        if (rbase + r < N && c < nchunk) ch[r][i].load(W + (long)(rbase + r) * K + c * 8);
      }
  };
  int r0 = blockIdx.x * rows_per_block;
  if (r0 < N) load_rows(r0);
  if (a.zero)
    for (int i = blockIdx.x * 256 + threadIdx.x; i < a.zero_words; i += gridDim.x * 256)
      a.zero[i] = 0u;

  // x slice in registers, optionally normalised
  float xv[CPL][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = (kpart * CPL + i) * 64 + lane;
    if (c < nchunk) {
      const float4 p = reinterpret_cast<const float4*>(a.x)[2 * c];
      const float4 q = reinterpret_cast<const float4*>(a.x)[2 * c + 1];
      xv[i][0] = p.x; xv[i][1] = p.y; xv[i][2] = p.z; xv[i][3] = p.w;
      xv[i][4] = q.x; xv[i][5] = q.y; xv[i][6] = q.z; xv[i][7] = q.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[i][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xv[i][e] * xv[i][e];
  }
  if (a.gamma) {
    const WT* gamma = static_cast<const WT*>(a.gamma);
    ss = wave_sum(ss);
    if (lane == 0) ssq[wid] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int p = 0; p < KSPLIT; ++p) tot += ssq[rgroup * KSPLIT + p];
    const float rs = rsqrtf(tot / (float)K + a.eps);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (kpart * CPL + i) * 64 + lane;
      if (c < nchunk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[i][e] = xv[i][e] * rs * ldw(gamma, c * 8 + e);
      }
    }
  }
  if (a.router_in && blockIdx.x == 0 && rgroup == 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (kpart * CPL + i) * 64 + lane;
      if (c < nchunk)
#pragma unroll
        for (int e = 0; e < 8; ++e) a.router_in[c * 8 + e] = xv[i][e];
    }
  }

  // largest output this thread wrote and its row (rows ascend, so the first
  // of equal values is the lowest row)
  float bm = -INFINITY;
  int bi = 0x7fffffff;
  for (; r0 < N; r0 += stride) {
    const int rbase = r0 + rgroup * RB;
    // the residual of the rows this thread writes goes out with the weights,
    // not after the reductions
    const bool writer = (KSPLIT == 1 || kpart == 0) && lane < RB && rbase + lane < N;
    const float res = (a.accumulate && writer) ? a.out[rbase + lane] : 0.f;
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
    }
    if (r0 + stride < N) load_rows(r0 + stride);
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = wave_sum(acc[r]);
    if (KSPLIT == 1) {
      if (lane < RB && rbase + lane < N) {
        float v = acc[0];
#pragma unroll
        for (int r = 1; r < RB; ++r) if (lane == r) v = acc[r];
        v = a.accumulate ? res + v : v;
        a.out[rbase + lane] = v;
        if (v > bm) { bm = v; bi = rbase + lane; }
      }
    } else {
      __syncthreads();
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) red[wid][r] = acc[r];
      }
      __syncthreads();
      if (kpart == 0 && lane < RB && rbase + lane < N) {
        float v = 0.f;
#pragma unroll
        for (int p = 0; p < KSPLIT; ++p) v += red[rgroup * KSPLIT + p][lane];
        v = a.accumulate ? res + v : v;
        a.out[rbase + lane] = v;
        if (v > bm) { bm = v; bi = rbase + lane; }
      }
    }
  }
  if (a.blockmax) {
    __shared__ float wm[4];
    __shared__ int wi[4];
    wave_argmax(bm, bi);
    if (lane == 0) { wm[wid] = bm; wi[wid] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int k = 1; k < 4; ++k)
        if (wm[k] > bm || (wm[k] == bm && wi[k] < bi)) { bm = wm[k]; bi = wi[k]; }
      a.blockmax[blockIdx.x] = bm;
      a.blockarg[blockIdx.x] = bi;
    }
  }
}

// The GEMV instance for K: (KSPLIT, CPL, RB) by the number of 8-element
// chunks of a row.
#define DS4G_GEMV_SHAPES(X)                                          \
  if (nchunk <= 64) X(1, 1, 2)          /* K <= 512 */               \
  if (nchunk <= 128) X(1, 2, 2)         /* K <= 1024 */              \
  if (nchunk <= 256) X(4, 1, 2)         /* K <= 2048 */              \
  if (nchunk <= 512) X(4, 2, 2)         /* K <= 4096 */              \
  if (nchunk <= 1024) X(4, 4, DS4G_GEMV_RB_K8K)   /* K <= 8192 */    \
  if (nchunk <= 2048) X(4, 8, 1)        /* K <= 16384 */
#define DS4G_GEMV_GRID(KS, R)                                        \
  const int rpb = R * (4 / KS);                                      \
  int grid = (N + rpb - 1) / rpb;                                    \
  if (grid > DS4G_GEMV_GRID_MAX) grid = DS4G_GEMV_GRID_MAX;

int gemv_grid(int N, int K) {
  const int nchunk = K / 8;
#define DS4G_GEMV(KS, C, R) { DS4G_GEMV_GRID(KS, R) return grid; }
  DS4G_GEMV_SHAPES(DS4G_GEMV)
#undef DS4G_GEMV
  return 0;
}

template <typename WT>
int launch_gemv(const GemvArgs& a, Exec st) {
  const int nchunk = a.K / 8;
  const int N = a.N;
#define DS4G_GEMV(KS, C, R)                                                    \
  {                                                                            \
    DS4G_GEMV_GRID(KS, R)                                                      \
    DS4G_LAUNCH((gemv_kernel<WT, KS, C, R>), dim3(grid), dim3(256), 0, st, a); \
    return 0;                                                                  \
  }
  DS4G_GEMV_SHAPES(DS4G_GEMV)
#undef DS4G_GEMV
  return -1;
}
template int launch_gemv<uint16_t>(const GemvArgs&, Exec);
template int launch_gemv<float>(const GemvArgs&, Exec);

// ---------------------------------------------------------------------------
// Multi-row GEMV: the dense projections of a batched decode call (M <= 8
// rows).  Each weight row is streamed once for all M rows.  The block layout
// is gemv_kernel's: 4 waves split K in KSPLIT parts and the block's rows in
// 4/KSPLIT groups; a wave keeps its K slice of all M activation rows in
// registers (bf16 or fp16 (XF16), MR x CPL chunks of 8) and streams RB bf16
// weight rows at a time, issuing the next rows' loads before the current
// rows' reductions.
template <int MR, int KSPLIT, int CPL, int RB, bool DUAL, bool XF16>
__global__ void __launch_bounds__(256)
gemv_rows_kernel(GemvRowsArgs a) {
  constexpr int RSPLIT = 4 / KSPLIT;
  constexpr int NV = DUAL ? 2 : 1;
  __shared__ float red[4][RB][MR][NV];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int kpart = wid % KSPLIT, rgroup = wid / KSPLIT;
  const int N = a.N, K = a.K, nchunk = K >> 3;
  const int rows_per_block = RB * RSPLIT;
  const int stride = gridDim.x * rows_per_block;

  uint4 xr[MR][CPL];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (kpart * CPL + i) * 64 + lane;
      xr[m][i] = (m < a.M && c < nchunk)
                     ? *reinterpret_cast<const uint4*>(a.X + (long)m * a.lda + c * 8)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
  Chunk8<uint16_t> cw[RB][CPL], cu[DUAL ? RB : 1][CPL];
  auto load_rows = [&](int r0) __attribute__((always_inline)) {
    const int rbase = r0 + rgroup * RB;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (kpart * CPL + i) * 64 + lane;
        if (rbase + r < N && c < nchunk) {
          cw[r][i].load(a.W + (long)(rbase + r) * K + c * 8);
          if (DUAL) cu[DUAL ? r : 0][i].load(a.W2 + (long)(rbase + r) * K + c * 8);
        }
      }
  };
  int r0 = blockIdx.x * rows_per_block;
  if (r0 < N) load_rows(r0);
  for (; r0 < N; r0 += stride) {
    const int rbase = r0 + rgroup * RB;
    float acc[RB][MR][NV];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][m][v] = 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (kpart * CPL + i) * 64 + lane;
        if (rbase + r < N && c < nchunk) {
          float w[8], u[8];
          cw[r][i].widen(w);
          if (DUAL) cu[DUAL ? r : 0][i].widen(u);
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            float x[8];
            if constexpr (XF16) unpack8_f16(xr[m][i], x);
            else unpack8(xr[m][i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              acc[r][m][0] += w[e] * x[e];
              if (DUAL) acc[r][m][NV - 1] += u[e] * x[e];
            }
          }
        }
      }
    if (r0 + stride < N) load_rows(r0 + stride);
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[r][m][v] = wave_sum(acc[r][m][v]);
    __syncthreads();   // the previous row group's sums have been read
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int v = 0; v < NV; ++v) red[wid][r][m][v] = acc[r][m][v];
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < RSPLIT * RB * MR) {
      const int rg = t / (RB * MR), r = (t / MR) % RB, m = t % MR;
      const int n = r0 + rg * RB + r;
      if (n < N && m < a.M) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int p = 0; p < KSPLIT; ++p) {
          g += red[rg * KSPLIT + p][r][m][0];
          if (DUAL) u += red[rg * KSPLIT + p][r][m][NV - 1];
        }
        const long o = (long)m * a.ldc + n;
        if (DUAL) static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(silu(g) * u);
        else if (a.epi == EPI_BF16) static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(g);
        else if (a.epi == EPI_F16) static_cast<uint16_t*>(a.C)[o] = f32_to_f16(g);
        else if (a.epi == EPI_RESID) static_cast<float*>(a.C)[o] += g;
        else static_cast<float*>(a.C)[o] = g;
      }
    }
  }
}

template <int MR, bool DUAL, bool XF16>
int launch_gemv_rows_mr(const GemvRowsArgs& a, Exec st) {
  constexpr int RB = 2;
  auto go = [&](auto kern, int ksplit) {
    const int rpb = RB * (4 / ksplit);
    long grid = (a.N + rpb - 1) / rpb;
    if (grid > DS4G_GEMV_GRID_MAX) grid = DS4G_GEMV_GRID_MAX;
    DS4G_LAUNCH(kern, dim3((unsigned)grid), dim3(256), 0, st, a);
    return 0;
  };
  if (a.K <= 1024) return go(gemv_rows_kernel<MR, 1, 2, RB, DUAL, XF16>, 1);
  return go(gemv_rows_kernel<MR, 4, 2, RB, DUAL, XF16>, 4);
}

template <int MR>
int launch_gemv_rows_m(const GemvRowsArgs& a, Exec st) {
  if (a.epi == EPI_SWIGLU_BF16) return a.x_f16 ? -1 : launch_gemv_rows_mr<MR, true, false>(a, st);
  return a.x_f16 ? launch_gemv_rows_mr<MR, false, true>(a, st)
                 : launch_gemv_rows_mr<MR, false, false>(a, st);
}

int launch_gemv_rows(const GemvRowsArgs& a, Exec st) {
  const bool dual = a.epi == EPI_SWIGLU_BF16;
  // K <= 4096: with 8 rows, a wider K slice per lane (K = 8192, W_o) needs
  // ~330-390 VGPRs, one wave per SIMD, and streamed at half the split-K
  // GEMM's rate (47 against 20 us at B = 8)
  if (a.M < 1 || a.M > 8 || a.K % 8 || a.K > 4096 || a.N < 1 || (dual && !a.W2)) return -1;
  if (!dual && a.epi != EPI_F32 && a.epi != EPI_BF16 && a.epi != EPI_F16 && a.epi != EPI_RESID)
    return -1;
  if (a.lda % 8) return -1;   // 16-byte activation chunks
  if (a.M <= 2) return launch_gemv_rows_m<2>(a, st);
  if (a.M <= 4) return launch_gemv_rows_m<4>(a, st);
  return launch_gemv_rows_m<8>(a, st);
}

// ---------------------------------------------------------------------------
// MoE decode for one token, three kernels:
//   router_shared_decode  logits = W_r y, y = RMSNorm(h2) * g2
//   moe_gateup_decode     its first blocks compute the shared expert's
//                         z_sh = silu(G_sh y) * (U_sh y), whose loads need no
//                         routing and fill HBM while the other blocks route;
//                         those pick the top-k from the logits (every wave for
//                         itself) and compute z_s = silu(G_s y) * (U_s y)
//   moe_down_decode       x = h2 + sum_s w_s D_s z_s + D_sh z_sh, one wave per
//                         routed slot and one for the shared expert
// The router launch reads only W_r, so the routing the gate/up blocks wait
// for is ready early.

// y = RMSNorm(h2) * g2 over the K slice of wave w (chunks [w*CPL*64,
// (w+1)*CPL*64)); h2 is read by every block (L2-resident).
template <typename WT, int CPL>
struct NormSlice {
  float v[CPL][8];
  __device__ __forceinline__ void load(const float* h2, int nchunk) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (wid * CPL + i) * 64 + lane;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = (c < nchunk) ? h2[c * 8 + e] : 0.f;
    }
  }
  // block-wide (4 waves): every thread must call it
  __device__ __forceinline__ void normalize(const void* gamma, float eps, int d, float* ssq) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nchunk = d >> 3;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[i][e] * v[i][e];
    ss = wave_sum(ss);
    if (lane == 0) ssq[wid] = ss;
    __syncthreads();
    const float rs = rsqrtf((ssq[0] + ssq[1] + ssq[2] + ssq[3]) / (float)d + eps);
    const WT* g = static_cast<const WT*>(gamma);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (wid * CPL + i) * 64 + lane;
      if (c < nchunk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = v[i][e] * rs * ldw(g, c * 8 + e);
      }
    }
  }
};

// Router logits and the shared expert's gate/up.  Task groups: the first
// ceil(E/RB) are RB router rows each (one weight row -> one logit), the rest
// RB shared (gate, up) row pairs each.  Blocks (4 waves splitting K = hidden)
// stride over groups; the next group's loads go out before the reductions.
// Groups [g0, g1) of that list, taken by block blk of nblk; every thread of
// the block calls it.
template <typename WT, int CPL, int RB>
__device__ __forceinline__ void router_shared_groups(const MoeDecodeArgs& a, int g0, int g1,
                                                     int blk, int nblk) {
  __shared__ float ssq[4];
  __shared__ float red[4][RB][2];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nchunk = a.d >> 3;
  const int ngr = (a.E + RB - 1) / RB, ng = g1;
  Chunk8<WT> cg[RB][CPL], cu[RB][CPL];
  auto load_group = [&](int g) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const WT *G, *U = nullptr;
      if (g < ngr) {
        const int e = g * RB + r;
        if (e >= a.E) continue;
        G = static_cast<const WT*>(a.router) + (long)e * a.d;
      } else {
        const int t = (g - ngr) * RB + r;
        if (t >= a.Is) continue;
        G = static_cast<const WT*>(a.sh_gate) + (long)t * a.d;
        U = static_cast<const WT*>(a.sh_up) + (long)t * a.d;
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = (wid * CPL + i) * 64 + lane;
        if (c < nchunk) {
          cg[r][i].load(G + c * 8);
          if (U) cu[r][i].load(U + c * 8);
        }
      }
    }
  };
  int g = g0 + blk;
  if (g < ng) load_group(g);
  NormSlice<WT, CPL> y;
  y.load(a.h2, nchunk);
  y.normalize(a.ffn_norm, a.eps, a.d, ssq);
  if (g0 == 0 && blk == 0 && a.router_in) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = (wid * CPL + i) * 64 + lane;
      if (c < nchunk)
#pragma unroll
        for (int e = 0; e < 8; ++e) a.router_in[c * 8 + e] = y.v[i][e];
    }
  }
  for (; g < ng; g += nblk) {
    const bool router = g < ngr;
    float ag[RB], au[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      ag[r] = 0.f; au[r] = 0.f;
      const bool live = router ? g * RB + r < a.E : (g - ngr) * RB + r < a.Is;
      if (live) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = (wid * CPL + i) * 64 + lane;
          if (c < nchunk) {
            float f[8];
            cg[r][i].widen(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) ag[r] += f[e] * y.v[i][e];
            if (!router) {
              cu[r][i].widen(f);
#pragma unroll
              for (int e = 0; e < 8; ++e) au[r] += f[e] * y.v[i][e];
            }
          }
        }
      }
    }
    if (g + nblk < ng) load_group(g + nblk);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      ag[r] = wave_sum(ag[r]);
      if (!router) au[r] = wave_sum(au[r]);
    }
    __syncthreads();
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) { red[wid][r][0] = ag[r]; red[wid][r][1] = au[r]; }
    }
    __syncthreads();
    if (wid == 0 && lane < RB) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) { gs += red[p][lane][0]; us += red[p][lane][1]; }
      if (router) {
        const int e = g * RB + lane;
        if (e < a.E) a.logits_out[e] = gs;
      } else {
        const int t = (g - ngr) * RB + lane;
        if (t < a.Is) a.z[a.k * a.I + t] = silu(gs) * us;   // z layout: routed slots, then shared
      }
    }
  }
}

// The router logits alone (the shared expert's gate/up runs in the first
// blocks of the routed gate/up launch, which need no routing).
template <typename WT, int CPL, int RB>
__global__ void __launch_bounds__(256)
router_shared_decode(MoeDecodeArgs a) {
  router_shared_groups<WT, CPL, RB>(a, 0, (a.E + RB - 1) / RB, blockIdx.x, gridDim.x);
}

// Routed gate/up: blocks [0, a.nsd) compute the shared expert's gate/up rows
// (they need only y, so their loads fill HBM while the routed blocks route);
// the rest stride
// over RB routed (gate, up) row pairs.  Every wave routes for itself from the
// logits in its registers (no block barrier before its routed loads); the
// first routed block publishes the routing for the down kernel and the caller.
template <typename WT, int CPL, int RB>
__global__ void __launch_bounds__(256)
moe_gateup_decode(MoeDecodeArgs a) {
  __shared__ float ssq[4];
  __shared__ float red[4][RB][2];
  __shared__ int wsel_idx[4][8];
  __shared__ float wsel_w[4][8];
  if ((int)blockIdx.x < a.nsd) {   // the shared expert's gate/up rows
    constexpr int RBR = DS4G_ROUTER_SHARED_RB;
    const int ngr = (a.E + RBR - 1) / RBR;
    router_shared_groups<WT, CPL, RBR>(a, ngr, ngr + (a.Is + RBR - 1) / RBR, blockIdx.x, a.nsd);
    return;
  }
  const int bid = blockIdx.x - a.nsd, nblk = gridDim.x - a.nsd;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nchunk = a.d >> 3;
  const int ntask = a.k * a.I;

  // The reads every block needs (router logits, h2) go out first, ahead of
  // any weight traffic: the routed rows cannot be loaded before they return.
  float lg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lg[i] = a.logits[min(lane + 64 * i, a.E - 1)];
  NormSlice<WT, CPL> y;
  y.load(a.h2, nchunk);
  const int* sel = wsel_idx[wid];     // this wave's routing (its own LDS slots)
  const float* wsel = wsel_w[wid];

  Chunk8<WT> cg[RB][CPL], cu[RB][CPL];
  // task t: routed slot s = t / I, row i
  auto load_tasks = [&](int t0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int t = t0 + r;
      if (t >= ntask) continue;
      const int s = t / a.I, i = t - s * a.I;
      const long base = ((long)sel[s] * a.I + i) * a.d;
      const WT* G = static_cast<const WT*>(a.gate) + base;
      const WT* U = static_cast<const WT*>(a.up) + base;
#pragma unroll
      for (int ii = 0; ii < CPL; ++ii) {
        const int c = (wid * CPL + ii) * 64 + lane;
        if (c < nchunk) { cg[r][ii].load(G + c * 8); cu[r][ii].load(U + c * 8); }
      }
    }
  };
  int t0 = bid * RB;
  const int stride = nblk * RB;
  route_wave(lg, a.E, a.k, wsel_idx[wid], wsel_w[wid]);   // every wave routes for itself
  if (t0 < ntask) load_tasks(t0);
  y.normalize(a.ffn_norm, a.eps, a.d, ssq);

  if (bid == 0 && wid == 0 && lane < a.k) {
    // publish the routing (one token: perm lists its k entries by expert)
    const int sj = sel[lane];
    const float wj = wsel[lane];
    a.sel[lane] = sj;
    a.wsel[lane] = wj;
    if (a.topk_idx) a.topk_idx[lane] = sj;
    if (a.topk_w) a.topk_w[lane] = wj;
    if (a.perm) {
      int r = 0;
      for (int q = 0; q < a.k; ++q) r += sel[q] < sj;
      a.perm[r] = lane;
    }
  }
  if (bid == 0 && (a.count || a.offset)) {
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) {
      int c = 0, o = 0;
      for (int q = 0; q < a.k; ++q) { c += sel[q] == e; o += sel[q] < e; }
      if (a.count && e < a.E) a.count[e] = c;
      if (a.offset) a.offset[e] = o;
    }
  }

  for (; t0 < ntask; t0 += stride) {
    float ag[RB], au[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      ag[r] = 0.f; au[r] = 0.f;
      if (t0 + r < ntask) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const int c = (wid * CPL + i) * 64 + lane;
          if (c < nchunk) {
            float f[8], gg[8];
            cg[r][i].widen(f);
            cu[r][i].widen(gg);
#pragma unroll
            for (int e = 0; e < 8; ++e) { ag[r] += f[e] * y.v[i][e]; au[r] += gg[e] * y.v[i][e]; }
          }
        }
      }
    }
    if (t0 + stride < ntask) load_tasks(t0 + stride);
#pragma unroll
    for (int r = 0; r < RB; ++r) { ag[r] = wave_sum(ag[r]); au[r] = wave_sum(au[r]); }
    __syncthreads();
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) { red[wid][r][0] = ag[r]; red[wid][r][1] = au[r]; }
    }
    __syncthreads();
    if (wid == 0 && lane < RB && t0 + lane < ntask) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) { gs += red[p][lane][0]; us += red[p][lane][1]; }
      a.z[t0 + lane] = silu(gs) * us;
    }
  }
}

// MoE down + combine + residual for one token:
//   x[n] = h2[n] + sum_s w_s (D_{e_s} z_s)[n] + (D_sh z_sh)[n]
// A block is k + 1 waves and owns RB output rows; wave s < k handles routed
// slot s and wave k the shared expert, so the weight rows of every slot are
// in flight together.  The sum runs in slot order, then the shared expert,
// then the residual.  Block 0 advances the ring position (the attention
// kernel has read it already).
template <typename WT, int CPL, int RB>
__global__ void __launch_bounds__(576)
moe_down_decode(MoeDecodeArgs a, float* x, int64_t* pos_inc) {
  __shared__ int sel[8];
  __shared__ float wsel[8];
  __shared__ float part[9][RB];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x < a.k) { sel[threadIdx.x] = a.sel[threadIdx.x]; wsel[threadIdx.x] = a.wsel[threadIdx.x]; }
  if (pos_inc && blockIdx.x == 0 && threadIdx.x == 0) *pos_inc += 1;
  const int n0 = blockIdx.x * RB;
  // the residual rows go out before the weights
  const float h2v = (threadIdx.x < RB && n0 + (int)threadIdx.x < a.d) ? a.h2[n0 + threadIdx.x] : 0.f;
  __syncthreads();
  if (wid <= a.k) {
    const int s = wid;
    const bool shared = s == a.k;
    const int Ks = shared ? a.Is : a.I;
    const WT* D = shared ? static_cast<const WT*>(a.sh_down)
                         : static_cast<const WT*>(a.down) + (long)sel[s] * a.d * a.I;
    Chunk8<WT> ch[RB][CPL];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int c = i * 64 + lane;
        if (n0 + r < a.d && c * 8 < Ks) ch[r][i].load(D + (long)(n0 + r) * Ks + c * 8);
      }
    const float* zz = a.z + s * a.I;   // the shared slot follows the k routed ones
    float zv[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane;
#pragma unroll
      for (int e = 0; e < 8; ++e) zv[i][e] = (c * 8 < Ks) ? zz[c * 8 + e] : 0.f;
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
          for (int e = 0; e < 8; ++e) p += f[e] * zv[i][e];
        }
      }
      p = wave_sum(p);
      if (lane == 0) part[s][r] = p;
    }
  }
  __syncthreads();
  if (wid == 0 && lane < RB && n0 + lane < a.d) {
    float v = 0.f;
    for (int s = 0; s < a.k; ++s) v += wsel[s] * part[s][lane];
    v += part[a.k][lane];
    x[n0 + lane] = h2v + v;
  }
}

template <typename WT>
int launch_moe_decode(const MoeDecodeArgs& a0, float* x, int64_t* pos_inc, Exec st) {
  if (a0.k > 8 || a0.E > 512 || a0.d % 8 || a0.I % 8 || a0.Is % 8) return -1;
  const int nchunk = a0.d / 8;
  const int cpl = (nchunk + 255) / 256;      // K = d over 4 waves
  // K = I (routed) or Is (shared) per wave of the down kernel
  const int cpld = (std::max(a0.I, a0.Is) / 8 + 63) / 64;
  if (cpl > 4 || cpld > 4) return -1;
  MoeDecodeArgs a = a0;
  // router logits
  {
    constexpr int RB = DS4G_ROUTER_SHARED_RB;
    const int ng = (a.E + RB - 1) / RB;
#define DS4G_RS(C) DS4G_LAUNCH((router_shared_decode<WT, C, RB>), dim3(ng), dim3(256), 0, st, a)
    if (cpl == 1) DS4G_RS(1); else if (cpl == 2) DS4G_RS(2); else DS4G_RS(4);
#undef DS4G_RS
  }
  // shared gate/up rows + routed gate/up
  {
    constexpr int RB = DS4G_GATEUP_RB;
    a.nsd = (a.Is + DS4G_ROUTER_SHARED_RB - 1) / DS4G_ROUTER_SHARED_RB;   // groups of shared rows
    if (a.nsd > DS4G_SHGU_GRID_MAX) a.nsd = DS4G_SHGU_GRID_MAX;
    const int ntask = a.k * a.I;
    int grid = (ntask + RB - 1) / RB;
    if (grid > DS4G_GATEUP_GRID_MAX) grid = DS4G_GATEUP_GRID_MAX;
    grid += a.nsd;
#define DS4G_GU(C) DS4G_LAUNCH((moe_gateup_decode<WT, C, RB>), dim3(grid), dim3(256), 0, st, a)
    if (cpl == 1) DS4G_GU(1); else if (cpl == 2) DS4G_GU(2); else DS4G_GU(4);
#undef DS4G_GU
  }
  // routed down + shared down + combine + residual: k + 1 waves per block,
  // DS4G_DOWN_RB rows per block where a wave's rows fit its registers
  // (bf16, K <= 1024), else 8
  {
    const int dthreads = 64 * (a.k + 1);
#define DS4G_DN(C, R) DS4G_LAUNCH((moe_down_decode<WT, C, R>), dim3((a.d + R - 1) / R), dim3(dthreads), 0, st, a, x, pos_inc)
    bool done = false;
    if constexpr (sizeof(WT) == 2) {
      if (cpld == 1) { DS4G_DN(1, DS4G_DOWN_RB); done = true; }
      else if (cpld == 2) { DS4G_DN(2, DS4G_DOWN_RB); done = true; }
    }
    if (!done) {
      if (cpld == 1) DS4G_DN(1, 8);
      else if (cpld == 2) DS4G_DN(2, 8);
      else DS4G_DN(4, 8);
    }
#undef DS4G_DN
  }
  return 0;
}
template int launch_moe_decode<uint16_t>(const MoeDecodeArgs&, float*, int64_t*, Exec);
template int launch_moe_decode<float>(const MoeDecodeArgs&, float*, int64_t*, Exec);

}  // namespace ds4g
