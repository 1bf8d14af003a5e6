// RoPE, sliding-window multi-query attention and the KV ring.
//
// ds4-learning 端到端推理流程, 阶段四 4.2 单层前向: q and k are rotated at their
// position, (k, v) is appended to the KV cache, then all 64 query heads attend
// to the same keys (MQA) inside a 128-token window.  The cache is a W-slot
// ring: position p lives in slot p % W, so a token sees exactly the slots
// still in its window.  Keys and values are cached in bf16; every key a query
// sees (its own included) is the cached bf16 value, so prefill and decode see
// identical numbers.
#include "dev.h"
#include "kernels.h"

namespace ds4g {

// ---------------------------------------------------------------------------
// rope_qkv: qkv fp32 [T, H*dh + 2*dh] (raw projection) ->
//   q  [T, H, dh]  rotated (QT = float or bf16)
//   kc [T, dh]     rotated, bf16
//   vc [T, dh]     bf16
// Pair i of the rotated tail turns by (pos0 + t) * base^(-2i/rd); the angle
// and its sine/cosine are formed in fp64 (positions reach 1e4..1e6, where an
// fp32 angle would be off by ~1e-3 rad).  One block per token.
template <typename QT>
__global__ void __launch_bounds__(256)
rope_qkv_kernel(const float* __restrict__ qkv, int T, int H, int dh, int rd, float base,
                const int64_t* __restrict__ pos, QT* __restrict__ q, uint16_t* __restrict__ kc,
                uint16_t* __restrict__ vc) {
  __shared__ float cs[64], sn[64];
  const int t = blockIdx.x;
  const long p = *pos + t;
  const int half = rd / 2, off = dh - rd;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv = pow((double)base, -2.0 * (double)i / (double)rd);
    double s, c;
    sincos((double)p * inv, &s, &c);
    cs[i] = (float)c;
    sn[i] = (float)s;
  }
  __syncthreads();
  const int qd = H * dh;
  const float* row = qkv + (long)t * (qd + 2 * dh);
  // pairs over q heads and k: (H + 1) * dh / 2 pairs
  const int npair = (H + 1) * (dh / 2);
  for (int pi = threadIdx.x; pi < npair; pi += blockDim.x) {
    const int head = pi / (dh / 2), j = pi - head * (dh / 2);   // head == H is k
    const int e0 = 2 * j;
    float a = row[head * dh + e0], b = row[head * dh + e0 + 1];
    if (e0 >= off) {
      const int i = (e0 - off) / 2;
      const float c = cs[i], s = sn[i];
      const float na = a * c - b * s, nb = a * s + b * c;
      a = na; b = nb;
    }
    if (head < H) {
      QT* dst = q + (long)t * qd + head * dh + e0;
      if constexpr (sizeof(QT) == 2) { dst[0] = f32_to_bf16(a); dst[1] = f32_to_bf16(b); }
      else { dst[0] = a; dst[1] = b; }
    } else {
      kc[(long)t * dh + e0] = f32_to_bf16(a);
      kc[(long)t * dh + e0 + 1] = f32_to_bf16(b);
    }
  }
  for (int e = threadIdx.x; e < dh; e += blockDim.x)
    vc[(long)t * dh + e] = f32_to_bf16(row[qd + dh + e]);
}

// ---------------------------------------------------------------------------
// Windowed MQA, SIMT: one block per (token, group of HG heads).  The window's
// keys (transposed) and values are staged in LDS as bf16; a wave takes one
// head at a time: lanes own keys for q.k, lanes own dims for p.v.
// Key of position j < pos0 comes from ring slot j % W, else from kc/vc.
template <typename OT, int DH>
__global__ void __launch_bounds__(256)
attn_window_kernel(const float* __restrict__ q, const uint16_t* __restrict__ kc,
                   const uint16_t* __restrict__ vc, const uint16_t* __restrict__ ring_k,
                   const uint16_t* __restrict__ ring_v, const int64_t* __restrict__ pos,
                   int T, int H, int W, int HG, OT* __restrict__ o) {
  constexpr int WMAX = 128;
  __shared__ uint16_t kT[DH][WMAX + 2];   // +2: spread banks across rows
  __shared__ uint16_t vs[WMAX][DH];
  __shared__ float qs[4][DH];
  __shared__ float ps[4][WMAX];
  const int t = blockIdx.x;
  const int h0 = blockIdx.y * HG;
  const long pos0 = *pos;
  const long p = pos0 + t;
  const long lo = p - W + 1 > 0 ? p - W + 1 : 0;
  const int n = (int)(p - lo + 1);
  const float scale = rsqrtf((float)DH);

  for (int idx = threadIdx.x; idx < n * (DH / 2); idx += blockDim.x) {
    const int jw = idx / (DH / 2), e = (idx - jw * (DH / 2)) * 2;
    const long j = lo + jw;
    const uint16_t *ks, *vsrc;
    if (j < pos0) {
      const long slot = j % W;
      ks = ring_k + slot * DH;
      vsrc = ring_v + slot * DH;
    } else {
      ks = kc + (j - pos0) * DH;
      vsrc = vc + (j - pos0) * DH;
    }
    const uint32_t kk = *reinterpret_cast<const uint32_t*>(ks + e);
    const uint32_t vv = *reinterpret_cast<const uint32_t*>(vsrc + e);
    kT[e][jw] = (uint16_t)(kk & 0xFFFF);
    kT[e + 1][jw] = (uint16_t)(kk >> 16);
    *reinterpret_cast<uint32_t*>(&vs[jw][e]) = vv;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int hh = wid; hh < HG && h0 + hh < H; hh += 4) {
    const int h = h0 + hh;
    const float* qh = q + ((long)t * H + h) * DH;
    for (int e = lane; e < DH; e += 64) qs[wid][e] = qh[e];
    wave_lds_sync();
    float s0 = -INFINITY, s1 = -INFINITY;
    {
      float a0 = 0.f, a1 = 0.f;
      for (int e = 0; e < DH; ++e) {
        const float qe = qs[wid][e];
        a0 += qe * bf16_to_f32(kT[e][lane]);
        a1 += qe * bf16_to_f32(kT[e][lane + 64]);
      }
      if (lane < n) s0 = a0 * scale;
      if (lane + 64 < n) s1 = a1 * scale;
    }
    const float m = wave_max(fmaxf(s0, s1));
    const float e0 = (lane < n) ? expf(s0 - m) : 0.f;
    const float e1 = (lane + 64 < n) ? expf(s1 - m) : 0.f;
    const float sum = wave_sum(e0 + e1);
    const float inv = 1.0f / sum;
    ps[wid][lane] = e0 * inv;
    ps[wid][lane + 64] = e1 * inv;
    wave_lds_sync();
    float o0 = 0.f, o1 = 0.f;
    for (int j = 0; j < n; ++j) {
      const float pj = ps[wid][j];
      o0 += pj * bf16_to_f32(vs[j][lane]);
      if (DH > 64) o1 += pj * bf16_to_f32(vs[j][lane + 64]);
    }
    OT* dst = o + ((long)t * H + h) * DH;
    if constexpr (sizeof(OT) == 2) {
      dst[lane] = f32_to_bf16(o0);
      if (DH > 64) dst[lane + 64] = f32_to_bf16(o1);
    } else {
      dst[lane] = o0;
      if (DH > 64) dst[lane + 64] = o1;
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// ring_commit: copy the cached (k, v) of the last min(T, W) tokens into their
// ring slots, then advance *pos by T.  One block; runs after every reader of
// the old ring contents and of *pos.
__global__ void __launch_bounds__(256)
ring_commit_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int T,
                   int W, int dh, uint16_t* __restrict__ ring_k, uint16_t* __restrict__ ring_v,
                   int64_t* pos) {
  const long pos0 = *pos;
  const int first = T > W ? T - W : 0;
  const int cnt = T - first;
  for (int idx = threadIdx.x; idx < cnt * dh; idx += blockDim.x) {
    const int r = idx / dh, e = idx - r * dh;
    const int t = first + r;
    const long slot = (pos0 + t) % W;
    ring_k[slot * dh + e] = kc[(long)t * dh + e];
    ring_v[slot * dh + e] = vc[(long)t * dh + e];
  }
  __syncthreads();
  if (threadIdx.x == 0) *pos = pos0 + T;
}

int launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.q_bf16)
    hipLaunchKernelGGL((rope_qkv_kernel<uint16_t>), dim3(a.T), dim3(256), 0, st, a.qkv, a.T, a.H,
                       a.dh, a.rd, a.base, a.pos, (uint16_t*)a.q, a.kc, a.vc);
  else
    hipLaunchKernelGGL((rope_qkv_kernel<float>), dim3(a.T), dim3(256), 0, st, a.qkv, a.T, a.H,
                       a.dh, a.rd, a.base, a.pos, (float*)a.q, a.kc, a.vc);
  const int HG = a.heads_per_block;
  dim3 grid(a.T, (a.H + HG - 1) / HG);
#define DS4G_ATT(OT, DH)                                                                      \
  hipLaunchKernelGGL((attn_window_kernel<OT, DH>), grid, dim3(256), 0, st, (const float*)a.q, \
                     a.kc, a.vc, a.ring_k, a.ring_v, a.pos, a.T, a.H, a.W, HG, (OT*)a.o)
  if (a.dh == 128) {
    if (a.o_bf16) DS4G_ATT(uint16_t, 128); else DS4G_ATT(float, 128);
  } else if (a.dh == 64) {
    if (a.o_bf16) DS4G_ATT(uint16_t, 64); else DS4G_ATT(float, 64);
  } else {
    return -1;
  }
#undef DS4G_ATT
  hipLaunchKernelGGL(ring_commit_kernel, dim3(1), dim3(256), 0, st, a.kc, a.vc, a.T, a.W, a.dh,
                     a.ring_k, a.ring_v, a.pos);
  return 0;
}

}  // namespace ds4g
