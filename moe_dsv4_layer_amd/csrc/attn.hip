// RoPE, sliding-window multi-query attention and the KV ring.
//
// ds4-learning 端到端推理流程, 阶段四 4.2 单层前向: q and k are rotated at their
// position, (k, v) is appended to the KV cache, then all 64 query heads attend
// to the same keys (MQA) inside a 128-token window.  The cache is a W-slot
// ring: position p lives in slot p % W, so a token sees exactly the slots
// still in its window.  Keys and values are cached in fp16 (IEEE binary16);
// every key a query sees (its own included) is the cached fp16 value, so
// prefill and decode see identical numbers.
#include "dev.h"
#include "kernels.h"

namespace ds4g {

// ---------------------------------------------------------------------------
// rope_qkv: qkv fp32 [T, H*dh + 2*dh] (raw projection) ->
//   q  [T, H, dh]  rotated (QT = float or fp16)
//   kc [T, dh]     rotated, fp16
//   vc [T, dh]     fp16
// Pair i of the rotated tail turns by (pos0 + t) * base^(-2i/rd) (angle in
// fp64, see rope_cs).  One block per token.
template <typename QT>
__global__ void __launch_bounds__(256)
rope_qkv_kernel(const float* __restrict__ qkv, int T, int H, int dh, int rd, float base,
                const int64_t* __restrict__ pos, QT* __restrict__ q, uint16_t* __restrict__ kc,
                uint16_t* __restrict__ vc) {
  __shared__ float cs[64], sn[64];
  const int t = blockIdx.x;
  const long p = *pos + t;
  const int half = rd / 2, off = dh - rd;
  for (int i = threadIdx.x; i < half; i += blockDim.x) rope_cs(p, i, rd, base, &cs[i], &sn[i]);
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
      if constexpr (sizeof(QT) == 2) { dst[0] = f32_to_f16(a); dst[1] = f32_to_f16(b); }
      else { dst[0] = a; dst[1] = b; }
    } else {
      kc[(long)t * dh + e0] = f32_to_f16(a);
      kc[(long)t * dh + e0 + 1] = f32_to_f16(b);
    }
  }
  for (int e = threadIdx.x; e < dh; e += blockDim.x)
    vc[(long)t * dh + e] = f32_to_f16(row[qd + dh + e]);
}

// ---------------------------------------------------------------------------
// Windowed MQA, SIMT: one block per (token, group of HG heads).  The window's
// keys (transposed) and values are staged in LDS as fp16; a wave takes one
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
        a0 += qe * f16_to_f32(kT[e][lane]);
        a1 += qe * f16_to_f32(kT[e][lane + 64]);
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
      o0 += pj * f16_to_f32(vs[j][lane]);
      if (DH > 64) o1 += pj * f16_to_f32(vs[j][lane + 64]);
    }
    OT* dst = o + ((long)t * H + h) * DH;
    if constexpr (sizeof(OT) == 2) {
      dst[lane] = f32_to_f16(o0);
      if (DH > 64) dst[lane + 64] = f32_to_f16(o1);
    } else {
      dst[lane] = o0;
      if (DH > 64) dst[lane + 64] = o1;
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// ring_commit: copy the cached (k, v) of the last min(T, W) tokens into their
// ring slots, then advance *pos by T.  One block: every thread reads *pos
// before the barrier, thread 0 advances it after (so no reader sees the new
// value); 16-byte copies, at most W rows of dh fp16 for k and for v.  Runs
// after every reader of the old ring contents.
__global__ void __launch_bounds__(1024)
ring_commit_kernel(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int T,
                   int W, int dh, uint16_t* __restrict__ ring_k, uint16_t* __restrict__ ring_v,
                   int64_t* __restrict__ pos) {
  const int64_t p = *pos;
  const int first = T > W ? T - W : 0;
  const int cnt = T - first, cpr = dh / 8;   // rows, 16-byte chunks per row
  for (int u = threadIdx.x; u < cnt * cpr; u += blockDim.x) {
    const int t = first + u / cpr, c = u % cpr;
    const int slot = (int)((p + t) % W);
    reinterpret_cast<uint4*>(ring_k + (long)slot * dh)[c] =
        reinterpret_cast<const uint4*>(kc + (long)t * dh)[c];
    reinterpret_cast<uint4*>(ring_v + (long)slot * dh)[c] =
        reinterpret_cast<const uint4*>(vc + (long)t * dh)[c];
  }
  __syncthreads();
  if (threadIdx.x == 0) *pos = p + T;
}

static void ring_commit(const AttnArgs& a, Exec st) {
  DS4G_LAUNCH(ring_commit_kernel, dim3(1), dim3(1024), 0, st, a.kc, a.vc, a.T, a.W, a.dh,
              a.ring_k, a.ring_v, a.pos);
}

int launch_attention(const AttnArgs& a, Exec st) {
  if (a.q_f16)
    DS4G_LAUNCH((rope_qkv_kernel<uint16_t>), dim3(a.T), dim3(256), 0, st, a.qkv, a.T, a.H,
                       a.dh, a.rd, a.base, a.pos, (uint16_t*)a.q, a.kc, a.vc);
  else
    DS4G_LAUNCH((rope_qkv_kernel<float>), dim3(a.T), dim3(256), 0, st, a.qkv, a.T, a.H,
                       a.dh, a.rd, a.base, a.pos, (float*)a.q, a.kc, a.vc);
  const int HG = a.heads_per_block;
  dim3 grid(a.T, (a.H + HG - 1) / HG);
#define DS4G_ATT(OT, DH)                                                                      \
  DS4G_LAUNCH((attn_window_kernel<OT, DH>), grid, dim3(256), 0, st, (const float*)a.q, \
                     a.kc, a.vc, a.ring_k, a.ring_v, a.pos, a.T, a.H, a.W, HG, (OT*)a.o)
  if (a.dh == 128) {
    if (a.o_f16) DS4G_ATT(uint16_t, 128); else DS4G_ATT(float, 128);
  } else if (a.dh == 64) {
    if (a.o_f16) DS4G_ATT(uint16_t, 64); else DS4G_ATT(float, 64);
  } else {
    return -1;
  }
#undef DS4G_ATT
  ring_commit(a, st);
  return 0;
}

// ---------------------------------------------------------------------------
// Decode attention (one token at position p = *pos): RoPE of the token's q
// heads and k, write (k, v) into ring slot p % W, softmax over the window
// [max(0, p-W+1), p] of q.k/sqrt(dh), o = sum p_j v_j.
//
// One block (256 threads) per head.  The work per head is tiny (2 x 128 x dh
// multiply-adds), so the kernel is latency-bound: every thread issues all of
// its K and V loads (straight from the ring into registers) at once, by ring
// slot, without waiting for *pos, and the RoPE frequencies are formed while
// *pos is in flight; the position only masks slots and picks the angle.
//   scores: thread t owns half of slot s = t/2 (dh/2 dims), halves meet by
//           a lane shuffle;
//   p.v:    thread t owns 8 dims (group t % DG) of KPG slots (group t / DG),
//           slot groups meet in LDS.
// Slot s holds key j = (s - lo) mod W of the window [lo, p]; slot p % W
// holds position p - W, outside the window: its load is replaced by the
// token's own k, v, and block 0 may overwrite it while the other blocks read.
// *pos is advanced by a later kernel.  Batched decode: blockIdx.y is the sequence b, with its own qkv row
// (stride qkv_stride), ring (b * W * DH), position pos[b] and o row (H * DH);
// o is fp32 or fp16 (OT).
template <int DH, typename OT>
__global__ void __launch_bounds__(256)
attn_decode_kernel(const float* __restrict__ qkv, long qkv_stride, int H, int W, int rd,
                   float base, const int64_t* __restrict__ pos, uint16_t* __restrict__ ring_k,
                   uint16_t* __restrict__ ring_v, OT* __restrict__ o) {
  {
    const int b = blockIdx.y;
    qkv += b * qkv_stride;
    pos += b;
    ring_k += (long)b * W * DH;
    ring_v += (long)b * W * DH;
    o += (long)b * H * DH;
  }
  constexpr int KC = DH / 16;            // 16-byte K chunks per thread (half a row)
  constexpr int DG = DH / 8;             // p.v dim groups of 8
  constexpr int KG = 256 / DG;           // p.v key groups
  constexpr int KPG = 128 / KG;          // keys per group
  __shared__ float cs[64], sn[64];
  __shared__ __align__(16) float qs[DH];
  __shared__ __align__(16) uint16_t kself[DH];
  __shared__ __align__(16) uint16_t vself[DH];
  __shared__ float pr[128];
  __shared__ float wred[4];
  __shared__ float red[KG][DH];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = blockIdx.x;
  const int qd = H * DH;
  // the token's q (this head), k and v need no position: load them first
  // (pairs: tid < DH/2 -> q, DH/2 <= tid < DH -> k, DH <= tid < 2 DH -> v)
  float ta = 0.f, tb = 0.f;
  if (tid < DH) {
    const bool isq = tid < DH / 2;
    const int e0 = 2 * (isq ? tid : tid - DH / 2);
    const float* src = isq ? qkv + (long)h * DH : qkv + qd;
    ta = src[e0];
    tb = src[e0 + 1];
  } else if (tid < 2 * DH) {
    ta = qkv[qd + DH + (tid - DH)];
  }
  const long p = *pos;
  // ---- issue every ring load now, by slot (slots past W read slot 0)
  const int jk = tid >> 1, hk = tid & 1;
  uint4 kreg[KC];
  {
    const long at = (jk < W) ? (long)jk * DH + hk * (DH / 2) : 0;
#pragma unroll
    for (int c = 0; c < KC; ++c) kreg[c] = *reinterpret_cast<const uint4*>(ring_k + at + c * 8);
  }
  const int dg = tid % DG, kg = tid / DG;
  uint4 vreg[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const int sl = kg * KPG + u;
    const long at = (sl < W) ? (long)sl * DH + dg * 8 : 0;
    vreg[u] = *reinterpret_cast<const uint4*>(ring_v + at);
  }
  // RoPE frequencies need no position
  double rinv = 0.0;
  if (tid < rd / 2) rinv = rope_inv(tid, rd, base);
  // the window [lo, p]: slot s holds key (s - lo) mod W, the token is key n-1
  const long lo = p - W + 1 > 0 ? p - W + 1 : 0;
  const int n = (int)(p - lo + 1);
  const int s0 = (int)(lo % W);
  auto key_of = [&](int sl) { const int j = sl - s0; return j < 0 ? j + W : j; };
  // ---- RoPE of q (this head) and k; the token's k, v in fp16 like the ring
  const int off = DH - rd;
  if (tid < rd / 2) rope_cs_inv(p, rinv, &cs[tid], &sn[tid]);
  __syncthreads();
  if (tid < DH) {   // pairs: tid < DH/2 -> q, else -> k
    const bool isq = tid < DH / 2;
    const int e0 = 2 * (isq ? tid : tid - DH / 2);
    float a = ta, b = tb;
    if (e0 >= off) {
      const int i = (e0 - off) / 2;
      const float c = cs[i], s = sn[i];
      const float na = a * c - b * s, nb = a * s + b * c;
      a = na; b = nb;
    }
    if (isq) { qs[e0] = a; qs[e0 + 1] = b; }
    else { kself[e0] = f32_to_f16(a); kself[e0 + 1] = f32_to_f16(b); }
  } else if (tid < 2 * DH) {
    vself[tid - DH] = f32_to_f16(ta);
  }
  __syncthreads();
  if (h == 0) {
    const long slot = p % W;
    if (tid < DH) ring_k[slot * DH + tid] = kself[tid];
    else if (tid < 2 * DH) ring_v[slot * DH + tid - DH] = vself[tid - DH];
  }
  // ---- scores (slot jk, key kj)
  const int kj = jk < W ? key_of(jk) : W;
  float sj;
  {
    if (kj == n - 1) {
#pragma unroll
      for (int c = 0; c < KC; ++c)
        kreg[c] = *reinterpret_cast<const uint4*>(kself + hk * (DH / 2) + c * 8);
    }
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float f[8];
      unpack8_f16(kreg[c], f);
      const float4 q0 = *reinterpret_cast<const float4*>(&qs[hk * (DH / 2) + c * 8]);
      const float4 q1 = *reinterpret_cast<const float4*>(&qs[hk * (DH / 2) + c * 8 + 4]);
      acc += q0.x * f[0] + q0.y * f[1] + q0.z * f[2] + q0.w * f[3] +
             q1.x * f[4] + q1.y * f[5] + q1.z * f[6] + q1.w * f[7];
    }
    acc += __shfl_xor(acc, 1, 64);
    sj = (kj < n) ? acc * rsqrtf((float)DH) : -INFINITY;
  }
  // softmax over the window: block max and sum (each key counted by its even lane)
  const float m = wave_max(sj);
  if (lane == 0) wred[wid] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
  const float ej = (kj < n) ? expf(sj - mx) : 0.f;
  const float es = wave_sum(hk == 0 ? ej : 0.f);
  __syncthreads();
  if (lane == 0) wred[wid] = es;
  if (hk == 0) pr[jk] = ej;
  __syncthreads();
  const float inv = 1.0f / (wred[0] + wred[1] + wred[2] + wred[3]);
  // ---- p.v
  {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const int sl = kg * KPG + u;
      const int j = sl < W ? key_of(sl) : W;
      if (j < n) {
        uint4 v4 = vreg[u];
        if (j == n - 1) v4 = *reinterpret_cast<const uint4*>(vself + dg * 8);
        float f[8];
        unpack8_f16(v4, f);
        const float pj = pr[sl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += pj * f[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[kg][dg * 8 + e] = acc[e];
  }
  __syncthreads();
  if (tid < DH) {
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < KG; ++g) v += red[g][tid];
    if constexpr (sizeof(OT) == 2) o[(long)h * DH + tid] = f32_to_f16(v * inv);
    else o[(long)h * DH + tid] = v * inv;
  }
}

int launch_attention_decode(const AttnArgs& a, Exec st) {
  const dim3 grid(a.H);
  if (a.dh == 128)
    DS4G_LAUNCH((attn_decode_kernel<128, float>), grid, dim3(256), 0, st, a.qkv, 0L, a.H,
                       a.W, a.rd, a.base, a.pos, a.ring_k, a.ring_v, (float*)a.o);
  else if (a.dh == 64)
    DS4G_LAUNCH((attn_decode_kernel<64, float>), grid, dim3(256), 0, st, a.qkv, 0L, a.H,
                       a.W, a.rd, a.base, a.pos, a.ring_k, a.ring_v, (float*)a.o);
  else
    return -1;
  return 0;
}

int launch_attention_decode_batch(const AttnArgs& a, int B, Exec st) {
  if (B <= 0 || B > 65535) return -1;
  const dim3 grid(a.H, B);
  const long stride = (long)a.H * a.dh + 2L * a.dh;
#define DS4G_AD(DH, OT)                                                                       \
  DS4G_LAUNCH((attn_decode_kernel<DH, OT>), grid, dim3(256), 0, st, a.qkv, stride, a.H, \
                     a.W, a.rd, a.base, a.pos, a.ring_k, a.ring_v, (OT*)a.o)
  if (a.dh == 128) {
    if (a.o_f16) DS4G_AD(128, uint16_t); else DS4G_AD(128, float);
  } else if (a.dh == 64) {
    if (a.o_f16) DS4G_AD(64, uint16_t); else DS4G_AD(64, float);
  } else {
    return -1;
  }
#undef DS4G_AD
  // every block has read pos[b]: advance the positions
  return 0;
}

// ---------------------------------------------------------------------------
// Prefill attention on the matrix cores (fp16 q, K, V, P; fp32 accumulate).
//
// A block takes the tokens of one 16-position-aligned span of absolute
// positions [A, A + 16) and 32 heads.  Block key row j is position
// A - W + 1 + j, so token tl (0..15) of the span sees rows [tl, tl + W - 1].
// The block stages its key rows once (fp16, XOR-swizzled rows) and the values
// transposed (8 consecutive keys of one dim are 16 contiguous bytes) in LDS.
// Aligning spans to absolute positions (not to the batch start) gives every
// token the same key-to-lane placement and reduction order whatever batch it
// arrives in, so a prefill resumed from a ring snapshot reproduces the
// uninterrupted prefill bit for bit.
//
// The unit of work is a 32-column tile: two consecutive tokens x 16 heads
// (MQA: every head of a token sees the same keys).  It is computed
// transposed, keys on the rows, so that the scores never leave registers:
//   S^T = K Q^T   key tiles of 32 rows from the pair's window start rounded
//                 down to 8 (4.5 tiles: the pair needs at most 136 rows), x
//                 dh/16 steps of v_mfma_f32_32x32x16_f16
//   mask, column max / sum: within the lane, then with lane ^ 32
//   O^T = V^T P^T dh/32 output tiles x 9 key steps of 16; the B operand P^T is
//                 the S^T accumulator rounded to fp16 in place
// The accumulator of a 32x32 MFMA gives lane l the column l % 32 and rows
// 8g + 4(l / 32) + i (g, i < 4); the B operand wants 8 consecutive keys
// 8(l / 32) .. + 7 of a 16-key step.  Feeding K row pi(r) to A-operand row r,
// pi(8g + 4h + i) = 16(g / 2) + 8h + 4(g % 2) + i, makes the accumulator rows
// of g = 2s, 2s + 1 exactly the keys of step s, so P^T needs no shuffle.
// Keys before the batch come from the ring (slot pos % W); the batch's own
// keys from kc/vc (already rotated and rounded to fp16).
// 4 waves and 74 KB of LDS per block: two blocks per CU, so one block's
// staging overlaps the other's arithmetic.
typedef _Float16 attn_f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float attn_f32x16;

// K rows are 16-B chunk-swizzled so that the 8 rows {x..x+3, x+8..x+11}
// (x % 4 == 0) that 8 consecutive lanes read hit 8 different bank groups
__device__ __forceinline__ int attn_kswz(int j) { return (j & 3) | (((j >> 3) & 1) << 2); }

template <int DH>
__global__ void __launch_bounds__(256, 2)
attn_prefill_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                  const uint16_t* __restrict__ vc, const uint16_t* __restrict__ ring_k,
                  const uint16_t* __restrict__ ring_v, const int64_t* __restrict__ pos, int T,
                  int H, int W, uint16_t* __restrict__ o) {
  constexpr int BQ = 16;
  constexpr int NK = 144;         // K rows: every key of the span (16 + W - 1 <= 143)
  constexpr int NV = 152;         // V keys: window start (<= 8) + 9 steps of 16
  constexpr int CPR = DH / 8;     // 16-B chunks per row
  constexpr int KSTEP = DH / 16;  // S^T contraction steps
  constexpr int DTILE = DH / 32;  // O^T row tiles
  __shared__ __align__(16) uint16_t Ks[NK * DH];    // [key][dh], chunk-swizzled
  __shared__ __align__(16) uint16_t Vt[DH * NV];    // [dh][key]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const long pos0 = *pos;
  const long P0 = (pos0 / BQ) * BQ + (long)blockIdx.x * BQ;   // span start A
  const long t0 = P0 - pos0;              // batch row of span position 0 (may be < 0)
  if (t0 >= T) return;
  const long kbase = P0 - W + 1;          // position of block key row 0
  const int nkeys = BQ + W - 1;           // <= 143
  auto key_src = [&](int j, bool val) -> const uint16_t* {
    const long kp = kbase + j;
    if (j >= nkeys || kp < 0 || kp >= pos0 + T) return nullptr;   // outside the sequence: 0
    if (kp < pos0) return (val ? ring_v : ring_k) + (kp % W) * DH;
    return (val ? vc : kc) + (kp - pos0) * DH;
  };
  const int lr = lane & 31, hf = lane >> 5;
  // wave w: head group 2 * blockIdx.y + w % 2, token pairs w / 2, w / 2 + 2, ...
  const int hg = 2 * blockIdx.y + (wid & 1);
  const int head = hg * 16 + (lr & 15);
  // Q^T B operand of pair p: column lr is token 2p + lr/16, head lr % 16 of
  // the group; zero outside the batch (branch-free: such lanes load row 0)
  auto load_q = [&](int p, attn_f16x8 (&dst)[DH / 16]) {
    const long t = t0 + 2 * p + ((lr >> 4) & 1);
    const bool ok = p < BQ / 2 && t >= 0 && t < T && head < H;
    const uint16_t* src = ok ? q + (t * H + head) * DH + hf * 8 : q;
#pragma unroll
    for (int ks = 0; ks < DH / 16; ++ks) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + (ok ? ks * 16 : 0));
      dst[ks] = __builtin_bit_cast(attn_f16x8, ok ? v : u32x4_t{0, 0, 0, 0});
    }
  };
  // the first pair's q goes out ahead of the staging loads
  attn_f16x8 qf[DH / 16];
  load_q(wid >> 1, qf);
  // every load of a thread goes out before its first LDS store (one wait, not
  // one round trip per chunk)
  constexpr int KIT = (NK * CPR + 255) / 256, VIT = (NV * CPR + 255) / 256;
  u32x4_t kbuf[KIT], vbuf[VIT];
  // branch-free: rows outside the sequence load row 0 of the batch and are
  // zeroed after the load
  const u32x4_t zero = {0, 0, 0, 0};
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + 256 * it, j = idx / CPR, c = idx - j * CPR;
    const uint16_t* src = idx < NK * CPR ? key_src(j, false) : nullptr;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>((src ? src : kc) + c * 8);
    kbuf[it] = src ? v : zero;
  }
  // V: consecutive lanes take consecutive keys of one 8-dim chunk, so each
  // 2-byte store row is contiguous across the wave
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int idx = tid + 256 * it, c = idx / NV, j = idx - c * NV;
    const uint16_t* src = idx < NV * CPR ? key_src(j, true) : nullptr;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>((src ? src : vc) + (idx < NV * CPR ? c * 8 : 0));
    vbuf[it] = src ? v : zero;
  }
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int idx = tid + 256 * it, j = idx / CPR, c = idx - j * CPR;
    if (idx < NK * CPR)
      *reinterpret_cast<u32x4_t*>(Ks + j * DH + ((c ^ attn_kswz(j)) * 8)) = kbuf[it];
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int idx = tid + 256 * it, c = idx / NV, j = idx - c * NV;
    if (idx < NV * CPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(c * 8 + e) * NV + j] = (uint16_t)(vbuf[it][e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();
  // exp(x * scale) = exp2(x * scale * log2(e))
  const float sl2 = rsqrtf((float)DH) * 1.4426950408889634f;
  const int pr = 16 * ((lr >> 3) >> 1) + 8 * ((lr >> 2) & 1) + 4 * ((lr >> 3) & 1) + (lr & 3);
  if (hg * 16 >= H) return;
  const long kmin = kbase < 0 ? -kbase : 0;       // first key row inside the sequence
  for (int p = wid >> 1; p < BQ / 2; p += 2) {
    // the next pair's q goes out before this pair's math
    attn_f16x8 qn[KSTEP];
    load_q(p + 2, qn);
    const int tl = 2 * p;
    const int tc = tl + ((lr >> 4) & 1);             // this lane's column token
    const long t = t0 + tc;
    const bool col_ok = t >= 0 && t < T && head < H;
    const int j0 = tl & ~7;
    if (t0 + tl + 1 >= 0 && t0 + tl < T) {           // a token of the pair is in the batch
    // ---- S^T = K Q^T; tile 4 keeps only its first 16 rows (g < 2), its
    // other rows are clamped to the last staged row and never used
    attn_f32x16 sacc[5];
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      sacc[m] = attn_f32x16{};
      const int j = min(j0 + 32 * m + pr, NK - 1);
      const uint16_t* krow = Ks + j * DH;
      const int sw = attn_kswz(j);
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(krow + (((2 * ks + hf) ^ sw) * 8));
        sacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            *reinterpret_cast<const attn_f16x8*>(&v), qf[ks], sacc[m], 0, 0, 0);
      }
    }
    // ---- mask to the window [tc, tc + W - 1] and the sequence start where a
    // tile crosses either edge for either token (wave-uniform test); then the
    // column max.  Accumulator (m, g, i) is key j0 + 32m + 16(g/2) + 8hf + 4(g%2) + i
    const int lo = max(tc, (int)kmin), hi = tc + W - 1;
    const int lo_pair = max(tl + 1, (int)kmin), hi_pair = tl + W - 1;
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      const int ng = m < 4 ? 4 : 2;
      const int jt = j0 + 32 * m;
      if (jt >= lo_pair && jt + 16 * (ng / 2) - 1 <= hi_pair) {
#pragma unroll
        for (int g = 0; g < ng; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[m][4 * g + i]);
      } else {
#pragma unroll
        for (int g = 0; g < ng; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = jt + 16 * (g >> 1) + 8 * hf + 4 * (g & 1) + i;
            const float v = (j >= lo && j <= hi) ? sacc[m][4 * g + i] : -INFINITY;
            sacc[m][4 * g + i] = v;
            mx = fmaxf(mx, v);
          }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mo = -mx * sl2;
    float sm = 0.f;
    attn_f16x8 pf[9];
#pragma unroll
    for (int m = 0; m < 5; ++m)
#pragma unroll
      for (int s = 0; s < (m < 4 ? 2 : 1); ++s) {
        float e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          e[k] = __builtin_amdgcn_exp2f(fmaf(sacc[m][8 * s + k], sl2, mo));   // masked: 0
          sm += e[k];
        }
        const u32x4_t pk = {pack_f16x2(e[0], e[1]), pack_f16x2(e[2], e[3]),
                            pack_f16x2(e[4], e[5]), pack_f16x2(e[6], e[7])};
        pf[2 * m + s] = __builtin_bit_cast(attn_f16x8, pk);
      }
    sm += __shfl_xor(sm, 32, kWave);
    // ---- O^T = V^T P^T
    attn_f32x16 oacc[DTILE];
#pragma unroll
    for (int dt = 0; dt < DTILE; ++dt) {
      oacc[dt] = attn_f32x16{};
      const uint16_t* vrow = Vt + (dt * 32 + lr) * NV + j0 + 8 * hf;
#pragma unroll
      for (int st = 0; st < 9; ++st) {
        const uint4 v = *reinterpret_cast<const uint4*>(vrow + 16 * st);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            *reinterpret_cast<const attn_f16x8*>(&v), pf[st], oacc[dt], 0, 0, 0);
      }
    }
    // lane holds dims dt*32 + 8g + 4hf + (0..3) of its column;
    // lane ^ 32 holds the other 4 dims of each 8-dim group: swap halves so
    // that every lane stores whole 16-byte groups (two per output tile)
    {
      const float inv = 1.f / sm;
#pragma unroll
      for (int dt = 0; dt < DTILE; ++dt) {
        unsigned pk[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          pk[g][0] = pack_f16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
          pk[g][1] = pack_f16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        }
        const int ga = hf ? 0 : 1, gb = hf ? 2 : 3;
        const unsigned r0 = __shfl_xor((int)pk[ga][0], 32, kWave), r1 = __shfl_xor((int)pk[ga][1], 32, kWave);
        const unsigned r2 = __shfl_xor((int)pk[gb][0], 32, kWave), r3 = __shfl_xor((int)pk[gb][1], 32, kWave);
        if (col_ok) {
          uint16_t* orow = o + (t * H + head) * DH;
          const int g0 = hf ? 1 : 0, g1 = hf ? 3 : 2;
          const u32x4_t w0 = hf ? u32x4_t{r0, r1, pk[1][0], pk[1][1]} : u32x4_t{pk[0][0], pk[0][1], r0, r1};
          const u32x4_t w1 = hf ? u32x4_t{r2, r3, pk[3][0], pk[3][1]} : u32x4_t{pk[2][0], pk[2][1], r2, r3};
          *reinterpret_cast<u32x4_t*>(orow + dt * 32 + 8 * g0) = w0;
          *reinterpret_cast<u32x4_t*>(orow + dt * 32 + 8 * g1) = w1;
        }
      }
    }
    }
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) qf[ks] = qn[ks];
  }
}

// cos / sin of every (pair i, row t) of a prefill, for the RoPE epilogue of
// the QKV GEMM (angle as in rope_cs: fp64, reduced mod 2 pi)
__global__ void __launch_bounds__(256)
rope_table_kernel(const int64_t* __restrict__ pos, int T, int ld, int rd, float base,
                  float* __restrict__ c, float* __restrict__ s) {
  const int t = blockIdx.x * 256 + threadIdx.x, i = blockIdx.y;
  if (t >= ld) return;
  float cv = 1.f, sv = 0.f;
  if (t < T) rope_cs(*pos + t, i, rd, base, &cv, &sv);
  c[(long)i * ld + t] = cv;
  s[(long)i * ld + t] = sv;
}

int launch_rope_table(const int64_t* pos, int T, int ld, int rd, float base, float* c, float* s,
                      Exec st) {
  if (ld < T || ld % 4 || rd < 2) return -1;
  DS4G_LAUNCH(rope_table_kernel, dim3((ld + 255) / 256, rd / 2), dim3(256), 0, st, pos, T,
                     ld, rd, base, c, s);
  return 0;
}

int launch_attention_prefill_mfma(const AttnArgs& a, Exec st) {
  if (a.W > 128 || !a.q_f16 || !a.o_f16) return -1;
  if (!a.rope_done)   // else the QKV GEMM's epilogue wrote rotated q, kc, vc
    DS4G_LAUNCH((rope_qkv_kernel<uint16_t>), dim3(a.T), dim3(256), 0, st, a.qkv, a.T, a.H,
                       a.dh, a.rd, a.base, a.pos, (uint16_t*)a.q, a.kc, a.vc);
  // spans are aligned to absolute positions: one extra span covers the
  // unknown (device-side) offset of the first position within its span
  const dim3 grid((a.T + 15) / 16 + 1, (a.H + 31) / 32);
  if (a.dh == 128)
    DS4G_LAUNCH((attn_prefill_mfma<128>), grid, dim3(256), 0, st, (const uint16_t*)a.q,
                       a.kc, a.vc, a.ring_k, a.ring_v, a.pos, a.T, a.H, a.W, (uint16_t*)a.o);
  else if (a.dh == 64)
    DS4G_LAUNCH((attn_prefill_mfma<64>), grid, dim3(256), 0, st, (const uint16_t*)a.q,
                       a.kc, a.vc, a.ring_k, a.ring_v, a.pos, a.T, a.H, a.W, (uint16_t*)a.o);
  else
    return -1;
  ring_commit(a, st);
  return 0;
}

}  // namespace ds4g
