// Prefill helpers: row RMSNorm, router top-k, and the token -> expert grouping
// that feeds the grouped expert GEMMs.
//
// ds4-learning 端到端推理流程, 阶段四 4.2 单层前向: x_norm = RMSNorm(x);
// scores = x_norm @ W_router (256 experts); top6 = TopK(scores, 6).  The
// grouping is this library's layout for running each expert once over all of its
// tokens (阶段三 逐层批处理): entries t*k + j, grouped by expert, in token order
// inside an expert; built with per-expert prefix sums, so it is deterministic
// (no atomics decide an order).
#include "dev.h"
#include "kernels.h"

namespace ds4g {

// ------------------------------------------------------------ RMSNorm rows
// y = RMSNorm(x[t]) * gamma per row; outputs (each optional): fp32 of, bf16
// ob, fp16 oh, and os3 = the exact three-term bf16 split [y1 | y2 | y3] (row stride
// 3d): y1 = bf16(y), y2 = bf16(y - y1), y3 = bf16(y - y1 - y2).  Products of
// the terms with bf16 weights are exact in fp32 and y - y1 - y2 - y3 is below
// 2^-27 |y|, so a bf16 MFMA GEMM over the split gives fp32-quality results.
constexpr int RMS_CHUNKS = 16;   // rows up to 16384 wide
__device__ __forceinline__ void load_gain4(const uint16_t* g, int i, float* o) {
  const uint2 q = *reinterpret_cast<const uint2*>(g + i);
  o[0] = __uint_as_float(q.x << 16); o[1] = __uint_as_float(q.x & 0xFFFF0000u);
  o[2] = __uint_as_float(q.y << 16); o[3] = __uint_as_float(q.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load_gain4(const float* g, int i, float* o) {
  const float4 q = *reinterpret_cast<const float4*>(g + i);
  o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
}

template <typename WT>
__global__ void __launch_bounds__(256)
rmsnorm_rows_kernel(const float* __restrict__ x, int d, const WT* __restrict__ gamma, float eps,
                    float* __restrict__ of, uint16_t* __restrict__ ob, uint16_t* __restrict__ oh,
                    uint16_t* __restrict__ os3) {
  // the row stays in registers between the sum of squares and the scaling
  // (d <= 256 * 4 * RMS_CHUNKS); all of a thread's loads go out together
  __shared__ float red[16];
  const long t = blockIdx.x;
  const float* row = x + t * d;
  float4 xv[RMS_CHUNKS];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c) {
    const int i = threadIdx.x * 4 + c * 1024;
    xv[c] = i < d ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c)
    ss += xv[c].x * xv[c].x + xv[c].y * xv[c].y + xv[c].z * xv[c].z + xv[c].w * xv[c].w;
  ss = block_sum(ss, red);
  const float rs = rsqrtf(ss / (float)d + eps);
#pragma unroll
  for (int c = 0; c < RMS_CHUNKS; ++c) {
    const int i = threadIdx.x * 4 + c * 1024;
    if (i >= d) break;
    const float4 v = xv[c];
    float g[4];
    load_gain4(gamma, i, g);
    float y[4] = {v.x * rs * g[0], v.y * rs * g[1], v.z * rs * g[2], v.w * rs * g[3]};
    if (of) *reinterpret_cast<float4*>(of + t * d + i) = make_float4(y[0], y[1], y[2], y[3]);
    uint16_t b1[4], b2[4], b3[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b1[e] = f32_to_bf16(y[e]);
      const float r1 = y[e] - bf16_to_f32(b1[e]);
      b2[e] = f32_to_bf16(r1);
      b3[e] = f32_to_bf16(r1 - bf16_to_f32(b2[e]));
    }
    auto pack = [](const uint16_t* b) {
      uint2 p;
      p.x = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
      p.y = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
      return p;
    };
    if (ob) *reinterpret_cast<uint2*>(ob + t * d + i) = pack(b1);
    if (oh) {
      uint2 p;
      p.x = pack_f16x2(y[0], y[1]);
      p.y = pack_f16x2(y[2], y[3]);
      *reinterpret_cast<uint2*>(oh + t * d + i) = p;
    }
    if (os3) {
      uint16_t* o = os3 + t * 3 * d + i;
      *reinterpret_cast<uint2*>(o) = pack(b1);
      *reinterpret_cast<uint2*>(o + d) = pack(b2);
      *reinterpret_cast<uint2*>(o + 2 * d) = pack(b3);
    }
  }
}

template <typename WT>
int launch_rmsnorm_rows(const float* x, int T, int d, const WT* gamma, float eps, float* of,
                        uint16_t* ob, uint16_t* oh, uint16_t* os3, Exec st) {
  if (d % 4 || d > 1024 * RMS_CHUNKS) return -1;
  DS4G_LAUNCH((rmsnorm_rows_kernel<WT>), dim3(T), dim3(256), 0, st, x, d, gamma, eps, of,
                     ob, oh, os3);
  return 0;
}
template int launch_rmsnorm_rows<uint16_t>(const float*, int, int, const uint16_t*, float,
                                           float*, uint16_t*, uint16_t*, uint16_t*, Exec);
template int launch_rmsnorm_rows<float>(const float*, int, int, const float*, float, float*,
                                        uint16_t*, uint16_t*, uint16_t*, Exec);

// ------------------------------------------------------------ top-k per token
// One wave per token: the k largest of the E logits (lower index wins ties)
// and the softmax probability of each pick, by route_wave (each lane sorts
// its logits once; a round is two DPP reductions and a register shift), the
// selection decode's gate/up blocks make.
// The logits arrive as nsplit partial sums (split-K GEMM); they are added in
// split order, so the result does not depend on scheduling.  lsum (the
// summed logits) is written only when a caller asked for them.
// NV = E/64 rounded up to a power of two: only the logits a lane holds take
// registers, so more waves fit beside the GEMM blocks of the second stream.
template <int NV>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ logits, int nsplit, float* __restrict__ lsum, int T, int E,
            int k, int* __restrict__ idx, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // the partial sums of all NV experts of a lane, 4 splits at a time, are
  // loaded before any is added; the adds run in split order
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  for (int z0 = 0; z0 < nsplit; z0 += 4) {
    float p[4][NV];
#pragma unroll
    for (int zz = 0; zz < 4; ++zz)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        p[zz][i] = (z0 + zz < nsplit && e < E) ? logits[((long)(z0 + zz) * T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int zz = 0; zz < 4; ++zz)
      if (z0 + zz < nsplit) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += p[zz][i];
      }
  }
  if (lsum) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < E) lsum[(long)t * E + lane + 64 * i] = v[i];
  }
  // route_topk (route_wave's selection at this NV) takes a NaN score as
  // -inf and keeps every index in [0, E)
  route_topk<NV>(v, E, k, idx + (long)t * k, wts + (long)t * k);
}

// ------------------------------------------------------------ block scans
// Exclusive prefix sum of n <= 256*SEG ints in LDS, in place; returns total.
template <int SEG>
__device__ int block_excl_scan(int* a, int n, int* wsum /*[4]*/) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int loc[SEG];
  int s = 0;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int j = tid * SEG + i;
    loc[i] = (j < n) ? a[j] : 0;
    s += loc[i];
  }
  // inclusive wave scan of s
  int inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wid] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  int run = base + inc - s;
#pragma unroll
  for (int i = 0; i < SEG; ++i) {
    const int j = tid * SEG + i;
    if (j < n) a[j] = run;
    run += loc[i];
  }
  __syncthreads();
  return total;
}

// ------------------------------------------------------------ expert ranks
// The permutation orders the T*k entries by (expert, entry index), so the
// rank of entry i inside its expert is the number of earlier entries with
// the same expert.  It is counted per chunk of kRankChunk entries, then the
// chunks are added in chunk order; every count is exact, so the result is
// the same however the blocks run.
//
// Chunk c (one block, one entry per thread): the lanes of a wave holding the
// same expert are found with one ballot per bit of the expert id; an entry's
// rank in the chunk is the count of its expert in earlier waves plus the
// lanes of its group below it.  chunk[c][e] = the chunk's entries of e.
__global__ void __launch_bounds__(kRankChunk)
rank_chunk_kernel(const int* __restrict__ idx, int n, int E, int* __restrict__ rank,
                  int* __restrict__ chunk) {
  constexpr int NW = kRankChunk / 64;
  extern __shared__ int wcs[];   // [NW][E]: sized by the launch, so the block fits beside
                                 // the shared expert's GEMM blocks on the second stream
  auto wc = [&](int w, int x) -> int& { return wcs[w * E + x]; };
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int i = blockIdx.x * kRankChunk + threadIdx.x;
  const int e = (i < n) ? idx[i] : -1;
  for (int j = threadIdx.x; j < NW * E; j += kRankChunk) wcs[j] = 0;
  // lanes whose expert equals this lane's
  uint64_t same = __ballot(e >= 0);
#pragma unroll
  for (int b = 0; b < 9; ++b) {   // E <= 512
    const bool bit = (e >> b) & 1;
    const uint64_t mb = __ballot(bit);
    same &= bit ? mb : ~mb;
  }
  const uint64_t below = same & ((1ull << lane) - 1ull);
  __syncthreads();
  if (e >= 0 && below == 0) wc(wid, e) = __popcll(same);   // the group's lowest lane
  __syncthreads();
  // per expert: exclusive prefix over the waves, and the chunk's total
  for (int x = threadIdx.x; x < E; x += kRankChunk) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = wc(w, x);
      wc(w, x) = run;
      run += t;
    }
    chunk[(long)blockIdx.x * E + x] = run;
  }
  __syncthreads();
  if (e >= 0) rank[i] = wc(wid, e) + __popcll(below);
}

// Per expert: the chunk counts turned into the entries of that expert in
// earlier chunks (added in chunk order), and the expert's total.  A block
// takes EPB experts; thread (expert, group g) takes a contiguous run of the
// chunks, loaded 8 at a time with all 8 in flight (the first 8 stay in
// registers for the second pass, so a run of up to 8 chunks is read once);
// the runs' sums are combined in group order through LDS.
// 256-thread blocks: beside the shared expert's GEMM blocks (8 waves, most
// of a CU's registers) a 16-wave block would wait for an empty CU.
constexpr int kPrefixEPB = 4;
__global__ void __launch_bounds__(256)
rank_prefix_kernel(int* __restrict__ chunk, int nchunk, int E, int* __restrict__ count) {
  __shared__ int gsum[256];
  const int epb = min(E, kPrefixEPB);
  const int G = 256 / epb;                       // groups per expert
  const int el = threadIdx.x % epb, gidx = threadIdx.x / epb;
  const int e = blockIdx.x * epb + el;
  const bool on = gidx < G && e < E;
  const int per = (nchunk + G - 1) / G;
  const int c0 = gidx * per, c1 = min(nchunk, c0 + per);
  int first[8];
  int s = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) first[u] = 0;
  if (on) {
    for (int c = c0; c < c1; c += 8) {   // 8 loads in flight
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (c + u < c1) ? chunk[(long)(c + u) * E + e] : 0;
      if (c == c0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) first[u] = v[u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
  }
  gsum[threadIdx.x] = s;
  __syncthreads();
  if (!on) return;
  int run = 0;
  for (int g = 0; g < gidx; ++g) run += gsum[g * epb + el];
  if (gidx == G - 1) count[e] = run + s;
  for (int c = c0; c < c1; c += 8) {
    int v[8];
    if (c == c0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = first[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = (c + u < c1) ? chunk[(long)(c + u) * E + e] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c + u < c1) {
        chunk[(long)(c + u) * E + e] = run;
        run += v[u];
      }
  }
}

// ------------------------------------------------------------ scatter + tiles
// Every block rebuilds offset[] from count[] (E <= 512) and scatters its
// entries; block 0 also publishes offset[] and the GEMM tile list.
__global__ void __launch_bounds__(256)
route_scatter_kernel(RouteArgs r) {
  __shared__ int off[513];
  __shared__ int tl[513];
  __shared__ int wsum[4];
  const int E = r.E;
  for (int e = threadIdx.x; e < E; e += 256) off[e] = r.count[e];
  __syncthreads();
  const int total = block_excl_scan<2>(off, E, wsum);
  if (threadIdx.x == 0) off[E] = total;
  __syncthreads();
  const int nent = r.T * r.k;
  const int ent = blockIdx.x * 256 + threadIdx.x;
  if (ent < nent) {
    const int e = r.topk_idx[ent];
    const int p = off[e] + r.chunk[(long)(ent / kRankChunk) * E + e] + r.rank[ent];
    r.perm[p] = ent;
    r.gather[p] = ent / r.k;
    r.pos_of[ent] = p;
  }
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= E; e += 256) {
      r.offset[e] = off[e];
      if (r.out_offset) r.out_offset[e] = off[e];
      if (r.out_count && e < E) r.out_count[e] = r.count[e];
    }
    for (int e = threadIdx.x; e < E; e += 256) tl[e] = (r.count[e] + r.tile_m - 1) / r.tile_m;
    __syncthreads();
    const int nt = block_excl_scan<2>(tl, E, wsum);
    for (int e = threadIdx.x; e < E; e += 256) {
      const int n = (r.count[e] + r.tile_m - 1) / r.tile_m;
      for (int m = 0; m < n; ++m) r.tiles[tl[e] + m] = (e << 16) | m;
    }
    if (threadIdx.x == 0) *r.ntiles = nt;
  }
}

int launch_route(const RouteArgs& r, Exec st) {
  if (r.E > 512 || r.k > 8) return -1;
#define DS4G_TOPK(NV)                                                                     \
  DS4G_LAUNCH(topk_kernel<NV>, dim3((r.T + 3) / 4), dim3(256), 0, st, r.logits, r.nsplit, \
              r.logits_sum, r.T, r.E, r.k, r.topk_idx, r.topk_w)
  if (r.E <= 64) DS4G_TOPK(1);
  else if (r.E <= 128) DS4G_TOPK(2);
  else if (r.E <= 256) DS4G_TOPK(4);
  else DS4G_TOPK(8);
#undef DS4G_TOPK
  const int nent = r.T * r.k;
  const int nchunk = (nent + kRankChunk - 1) / kRankChunk;
  DS4G_LAUNCH(rank_chunk_kernel, dim3(nchunk), dim3(kRankChunk),
              (size_t)(kRankChunk / 64) * r.E * sizeof(int), st, r.topk_idx, nent, r.E, r.rank,
              r.chunk);
  DS4G_LAUNCH(rank_prefix_kernel, dim3((r.E + kPrefixEPB - 1) / kPrefixEPB), dim3(256), 0, st,
              r.chunk, nchunk, r.E, r.count);
  DS4G_LAUNCH(route_scatter_kernel, dim3((nent + 255) / 256), dim3(256), 0, st, r);
  return 0;
}

// ------------------------------------------------------------ MoE combine
// x[t] += sum_j w[t, j] * part[pos_of[t*k + j]], j = 0..k-1 in order, where
// x already holds h2 + shared-expert output.  One block per token: the k
// expert-output rows are read whole (contiguous), 4 floats per thread.
// 4 consecutive expert-output values as fp32 (fp32 or bf16 storage)
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

template <typename PT>
__global__ void __launch_bounds__(256)
moe_combine_kernel(float* __restrict__ x, const PT* __restrict__ part,
                   const int* __restrict__ pos_of, const float* __restrict__ w, int d, int k,
                   int64_t* __restrict__ pos_inc) {
  const int t = blockIdx.x;
  if (pos_inc && threadIdx.x == 0) pos_inc[t] += 1;   // batched decode: row t's sequence
  __shared__ int rows[8];
  __shared__ float ws[8];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = pos_of[t * k + threadIdx.x];
    ws[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 a = *reinterpret_cast<const float4*>(x + (long)t * d + c);
    for (int j = 0; j < k; ++j) {
      const float4 p = load4(part + (long)rows[j] * d + c);
      a.x += ws[j] * p.x; a.y += ws[j] * p.y; a.z += ws[j] * p.z; a.w += ws[j] * p.w;
    }
    *reinterpret_cast<float4*>(x + (long)t * d + c) = a;
  }
}

int launch_moe_combine(float* x, const void* part, int part_bf16, const int* pos_of,
                       const float* w, int T, int d, int k, int64_t* pos_inc, Exec st) {
  if (d % 4 || k > 8) return -1;
  if (part_bf16)
    DS4G_LAUNCH(moe_combine_kernel<uint16_t>, dim3(T), dim3(256), 0, st, x,
                       static_cast<const uint16_t*>(part), pos_of, w, d, k, pos_inc);
  else
    DS4G_LAUNCH(moe_combine_kernel<float>, dim3(T), dim3(256), 0, st, x,
                       static_cast<const float*>(part), pos_of, w, d, k, pos_inc);
  return 0;
}

}  // namespace ds4g
