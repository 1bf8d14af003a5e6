// Token sampler over the full vocabulary (ds4-learning 端到端推理流程,
// 阶段四 4.3 采样): divide the logits by the temperature, keep the most
// probable tokens until they hold top_p of the mass (sorted descending), then
// a roulette walk in vocabulary order with r = u * (kept mass); temperature 0
// is argmax (阶段六 温度覆盖).
//
// The page's CPU code sorts and walks 129280 entries one by one.  Here no sort
// is needed: the top-p cut is found by a two-level radix select on the bits of
// the (positive) weights q = exp((l - max)/T) -- first the top 16 bits, then
// the low 16 bits of the crossing bucket -- with bucket masses kept as 64-bit
// fixed-point integers (q * 2^45), so every sum is exact and independent of
// the order atomics land in.  Equal weights at the cut are kept in index
// order.  The roulette is a two-level prefix sum (1024-entry segments, then
// the entries of one segment).  Every step is deterministic.
#include "dev.h"
#include "kernels.h"

namespace ds4g {

namespace {
constexpr int SEG = 1024;          // entries per segment / per block
constexpr int NB1 = 16384;         // level-1 buckets (q <= 1 => key1 <= 0x3F80)
constexpr int NB2 = 65536;         // level-2 buckets
constexpr double FX = 35184372088832.0;   // 2^45
// level-1 keys below KLO (q < 2^-45, exponent field < 82) have no fixed-point
// mass: fx(q) = 0 there, so their histogram entries stay zero
constexpr int KLO = 82 << 7;
constexpr int NKEY = 0x3F80 + 1 - KLO;   // keys KLO..0x3F80 (q <= 1)
constexpr int QSEGS = 4;                 // segments per samp_q block

__device__ __forceinline__ uint64_t fx(float q) { return (uint64_t)((double)q * FX); }

struct SampState {
  float M;              // max logit
  uint32_t b1;          // level-1 crossing bucket
  unsigned long long above1;   // mass of buckets above b1
  double target;        // top_p * total mass
  unsigned long long total;
  uint32_t vstar;       // bits of the cut weight q*
  int m;                // equal-to-q* entries kept (in index order)
  unsigned long long above; // mass strictly above q*
  double u;             // the uniform draw; r = u * (kept mass) is formed in S7
  int all;              // top_p >= 1: keep everything
};

struct SampWs {
  float* bmax; int* barg; float* q;
  unsigned long long* h1; unsigned long long* h2; unsigned int* c2;
  unsigned long long* g2;   // level-2 mass per group of 1024 descending positions
  unsigned long long* seg_gt; int* seg_gtn; int* seg_tie;
  SampState* st;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline SampWs carve(void* base, int V) {
  const int nb = (V + SEG - 1) / SEG;
  char* p = static_cast<char*>(base);
  SampWs w;
  size_t o = 0;
  w.bmax = (float*)(p + o); o = align256(o + nb * sizeof(float));
  w.barg = (int*)(p + o); o = align256(o + nb * sizeof(int));
  w.q = (float*)(p + o); o = align256(o + (size_t)V * sizeof(float));
  w.h1 = (unsigned long long*)(p + o); o = align256(o + NB1 * 8);
  w.h2 = (unsigned long long*)(p + o); o = align256(o + NB2 * 8);
  w.c2 = (unsigned int*)(p + o); o = align256(o + NB2 * 4);
  w.g2 = (unsigned long long*)(p + o); o = align256(o + (NB2 / 1024) * 8);
  w.seg_gt = (unsigned long long*)(p + o); o = align256(o + nb * 8);
  w.seg_gtn = (int*)(p + o); o = align256(o + nb * 4);
  w.seg_tie = (int*)(p + o); o = align256(o + nb * 4);
  w.st = (SampState*)(p + o); o = align256(o + sizeof(SampState));
  return w;
}
size_t carve_bytes(int V) {
  const int nb = (V + SEG - 1) / SEG;
  size_t o = 0;
  o = align256(o + nb * sizeof(float));
  o = align256(o + nb * sizeof(int));
  o = align256(o + (size_t)V * sizeof(float));
  o = align256(o + NB1 * 8);
  o = align256(o + NB2 * 8);
  o = align256(o + NB2 * 4);
  o = align256(o + (NB2 / 1024) * 8);
  o = align256(o + nb * 8);
  o = align256(o + nb * 4);
  o = align256(o + nb * 4);
  o = align256(o + sizeof(SampState));
  return o;
}

// block-wide inclusive scan of one u64 per thread (blockDim 1024)
__device__ unsigned long long block_incl_scan_u64(unsigned long long v, unsigned long long* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  __syncthreads();
  if (lane == 63) red[wid] = v;
  __syncthreads();
  unsigned long long base = 0;
  for (int w = 0; w < wid; ++w) base += red[w];
  (void)nw;
  __syncthreads();
  return v + base;
}
}  // namespace

size_t sample_ws_bytes(int V) { return carve_bytes(V); }

// S1: per-segment max and its first index; clear the histograms.
__global__ void __launch_bounds__(256)
samp_max_kernel(const float* __restrict__ logits, int V, SampWs w) {
  const int nb = gridDim.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __shared__ float bv[4];
  __shared__ int bi[4];
  float m = -INFINITY;
  int mi = blockIdx.x * SEG;   // a segment of NaN / -inf logits still names a token
  for (int i = blockIdx.x * SEG + threadIdx.x; i < min(V, (blockIdx.x + 1) * SEG); i += 256) {
    const float l = logits[i];
    if (l > m) { m = l; mi = i; }
  }
  wave_argmax(m, mi);
  if (lane == 0) { bv[wid] = m; bi[wid] = mi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < 4; ++k)
      if (bv[k] > m || (bv[k] == m && bi[k] < mi)) { m = bv[k]; mi = bi[k]; }
    w.bmax[blockIdx.x] = m;
    w.barg[blockIdx.x] = mi;
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < NB1; i += nb * 256) w.h1[i] = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < NB2; i += nb * 256) { w.h2[i] = 0; w.c2[i] = 0; }
}

// The temperature of a call: a host value, or one read from device memory
// each time (tdev), so that a captured graph can switch between sampling and
// argmax without being captured again.
__device__ __forceinline__ bool sampling(float temperature, const float* tdev) {
  const float t = tdev ? *tdev : temperature;
  return t > 0.f;
}

// argmax over the segment results (temperature <= 0)
__global__ void __launch_bounds__(64)
samp_argmax_kernel(int nb, SampWs w, int* token, float temperature, const float* tdev) {
  if (sampling(temperature, tdev)) return;
  float m = -INFINITY;
  int mi = 0x7fffffff;
  for (int b = threadIdx.x; b < nb; b += 64) {
    const float v = w.bmax[b];
    const int i = w.barg[b];
    if (v > m || (v == m && i < mi)) { m = v; mi = i; }
  }
  wave_argmax(m, mi);
  if (threadIdx.x == 0) *token = mi;
}

// the largest logit, from the segment maxima (block-wide: every thread;
// red holds one float per wave)
__device__ __forceinline__ float global_max(const SampWs& w, int nb, float* red) {
  float m = -INFINITY;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) m = fmaxf(m, w.bmax[b]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

// S2: q = exp((l - M) / T); level-1 histogram of fixed-point mass.  A block
// of 1024 takes QSEGS segments and sums their masses per key in LDS first, so
// that equal keys (a narrow logit spread puts thousands of weights in one
// key) cost one global atomic per block instead of one per entry.
__global__ void __launch_bounds__(1024)
samp_q_kernel(const float* __restrict__ logits, int V, int nb, float temperature,
              const float* tdev, SampWs w) {
  if (!sampling(temperature, tdev)) return;
  if (tdev) temperature = *tdev;
  __shared__ unsigned long long hist[NKEY];
  __shared__ float red[16];
  for (int k = threadIdx.x; k < NKEY; k += blockDim.x) hist[k] = 0;
  const float M = global_max(w, nb, red);   // ends in a barrier: hist is clear
  if (blockIdx.x == 0 && threadIdx.x == 0) w.st->M = M;
  const int lo = blockIdx.x * QSEGS * SEG, hi = min(V, lo + QSEGS * SEG);
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    float q = expf((logits[i] - M) / temperature);
    q = (q == q) ? fminf(q, 1.f) : 0.f;   // a NaN logit weighs nothing; keys stay <= 0x3F80
    w.q[i] = q;
    const int key = (int)(__float_as_uint(q) >> 16) - KLO;
    if (key >= 0) atomicAdd(&hist[key], (unsigned long long)fx(q));
  }
  __syncthreads();
  for (int k = threadIdx.x; k < NKEY; k += blockDim.x) {
    const unsigned long long v = hist[k];
    if (v) atomicAdd(&w.h1[KLO + k], v);
  }
}

// S3 (one block of 1024): total mass, target, and the level-1 bucket where the
// descending cumulative mass reaches the target.
__global__ void __launch_bounds__(1024)
samp_level1_kernel(float top_p, SampWs w, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev)) return;
  __shared__ unsigned long long red[16];
  constexpr int PER = NB1 / 1024;
  // position i in descending bucket order: bucket NB1-1-i
  unsigned long long loc[PER];
  unsigned long long s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    loc[j] = w.h1[NB1 - 1 - (threadIdx.x * PER + j)];
    s += loc[j];
  }
  const unsigned long long inc = block_incl_scan_u64(s, red);
  __shared__ unsigned long long tot;
  if (threadIdx.x == 1023) tot = inc;
  __syncthreads();
  double target = (double)top_p * (double)tot;
  if (target < 0.5) target = 0.5;   // keep at least one token
  const bool all = top_p >= 1.0f;
  if (threadIdx.x == 0) {
    w.st->total = tot;
    w.st->target = target;
    w.st->all = all ? 1 : 0;
  }
  if (all) return;
  unsigned long long run = inc - s;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const unsigned long long nxt = run + loc[j];
    if ((double)run < target && (double)nxt >= target) {
      w.st->b1 = NB1 - 1 - (threadIdx.x * PER + j);
      w.st->above1 = run;
    }
    run = nxt;
  }
}

// S4: level-2 histogram inside bucket b1.
__global__ void __launch_bounds__(256)
samp_hist2_kernel(int V, SampWs w, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev) || w.st->all) return;
  const uint32_t b1 = w.st->b1;
  for (int i = blockIdx.x * SEG + threadIdx.x; i < min(V, (blockIdx.x + 1) * SEG); i += 256) {
    const float q = w.q[i];
    const uint32_t bits = __float_as_uint(q);
    if ((bits >> 16) == b1) {
      atomicAdd(&w.h2[bits & 0xFFFF], (unsigned long long)fx(q));
      atomicAdd(&w.c2[bits & 0xFFFF], 1u);
    }
  }
}

__device__ __forceinline__ uint64_t splitmix64_next(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// min-p: every weight below min(min_p, 1) is dropped (the largest weight
// is exactly 1).  When that threshold lies above the top-p cut q*, it becomes
// the cut and every entry equal to it is kept; otherwise top-p decides.
__device__ __forceinline__ void apply_min_p(SampState* st, float min_p) {
  if (!(min_p > 0.f)) return;
  const float thr = fminf(min_p, 1.f);
  if (thr > __uint_as_float(st->vstar)) {
    st->vstar = __float_as_uint(thr);
    st->m = 0x7fffffff;
  }
}

// S5a: level-2 mass per group of 1024 descending positions (group g: buckets
// NB2-1-1024g down to NB2-1024-1024g, contiguous), one block per group.
__global__ void __launch_bounds__(256)
samp_l2sum_kernel(SampWs w, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev) || w.st->all) return;
  __shared__ unsigned long long ws[4];
  const unsigned long long* hb = w.h2 + (NB2 - 1024 - blockIdx.x * 1024) + threadIdx.x * 4;
  const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(hb);
  const ulonglong2 b = *reinterpret_cast<const ulonglong2*>(hb + 2);
  unsigned long long s = a.x + a.y + b.x + b.y;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) w.g2[blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

// S5 (one block of 1024): exact cut weight q*, how many equal-to-q* entries
// are kept (top-p, then min-p), and the generator draw u.
__global__ void __launch_bounds__(1024)
samp_level2_kernel(SampWs w, uint64_t* rng, float min_p, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev)) return;
  __shared__ unsigned long long red[16];
  SampState* st = w.st;
  if (st->all) {
    if (threadIdx.x == 0) {
      st->vstar = 0u;
      st->m = 0x7fffffff;   // every entry equal to q* = 0 is kept too
      st->above = st->total;
      apply_min_p(st, min_p);
      const uint64_t z = splitmix64_next(rng);
      st->u = (double)(z >> 40) * (1.0 / 16777216.0);
    }
    return;
  }
  const double target = st->target;
  const unsigned long long a1 = st->above1;
  // the group of 1024 positions that holds the crossing (the cumulative mass
  // is non-decreasing and level 1 put the target inside bucket b1): wave 0
  // scans the 64 group sums
  __shared__ int grp;
  __shared__ unsigned long long grun;
  if (threadIdx.x == 0) grp = -1;
  __syncthreads();
  if (threadIdx.x < NB2 / 1024) {
    const int lane = threadIdx.x;
    const unsigned long long gs = w.g2[lane];
    unsigned long long cum = gs;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = __shfl_up(cum, o, 64);
      if (lane >= o) cum += y;
    }
    const unsigned long long run0 = a1 + cum - gs;
    if ((double)run0 < target && (double)(run0 + gs) >= target) {
      grp = lane;
      grun = run0;
    }
  }
  __syncthreads();
  if (grp < 0) return;
  // the group's positions, one per thread (descending), prefix-summed
  const uint32_t b2 = NB2 - 1 - (grp * 1024 + threadIdx.x);
  const unsigned long long hv = w.h2[b2];
  const unsigned long long run = grun + block_incl_scan_u64(hv, red) - hv;   // mass before b2
  if ((double)run < target && (double)(run + hv) >= target) {
    const uint32_t vbits = (st->b1 << 16) | b2;
    const unsigned long long qf = fx(__uint_as_float(vbits));
    const unsigned int cnt = w.c2[b2];
    // smallest m >= 1 with run + m*qf >= target
    long long mm = (long long)ceil((target - (double)run) / (double)qf);
    if (mm < 1) mm = 1;
    if (mm > (long long)cnt) mm = cnt;
    while (mm > 1 && (double)(run + (unsigned long long)(mm - 1) * qf) >= target) --mm;
    while (mm < (long long)cnt && (double)(run + (unsigned long long)mm * qf) < target) ++mm;
    st->vstar = vbits;
    st->m = (int)mm;
    st->above = run;
    apply_min_p(st, min_p);
    const uint64_t z = splitmix64_next(rng);
    st->u = (double)(z >> 40) * (1.0 / 16777216.0);
  }
}

// S6: per segment, mass strictly above q*, how many such entries, and how
// many entries equal q*.
__global__ void __launch_bounds__(256)
samp_segsum_kernel(int V, SampWs w, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev)) return;
  __shared__ unsigned long long ss[4];
  __shared__ int sn[4], st_[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const float qs = __uint_as_float(w.st->vstar);
  unsigned long long s = 0;
  int n = 0, t = 0;
  for (int i = blockIdx.x * SEG + threadIdx.x; i < min(V, (blockIdx.x + 1) * SEG); i += 256) {
    const float q = w.q[i];
    if (q > qs) { s += fx(q); ++n; }
    else if (q == qs) ++t;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o, 64);
    n += __shfl_xor(n, o, 64);
    t += __shfl_xor(t, o, 64);
  }
  if (lane == 0) { ss[wid] = s; sn[wid] = n; st_[wid] = t; }
  __syncthreads();
  if (threadIdx.x == 0) {
    w.seg_gt[blockIdx.x] = ss[0] + ss[1] + ss[2] + ss[3];
    w.seg_gtn[blockIdx.x] = sn[0] + sn[1] + sn[2] + sn[3];
    w.seg_tie[blockIdx.x] = st_[0] + st_[1] + st_[2] + st_[3];
  }
}

// S7 (one block of 1024): the kept mass K (exact, per segment in fixed point),
// r = u * K, then the segment and the entry where the running kept mass
// (vocabulary order) first reaches r.
__global__ void __launch_bounds__(1024)
samp_pick_kernel(int V, int nb, SampWs w, int* token, float temperature, const float* tdev) {
  if (!sampling(temperature, tdev)) return;
  __shared__ unsigned long long red[16];
  __shared__ int tie_base_s, seg_s;
  __shared__ unsigned long long cum_before_s, kept_s;
  __shared__ int wtie[16];
  const SampState& st = *w.st;
  const float qs = __uint_as_float(st.vstar);
  const unsigned long long qf = fx(qs);
  const int m = st.m;
  // level A: segments (nb <= 1024), one per thread
  const int b = threadIdx.x;
  int tie = (b < nb) ? w.seg_tie[b] : 0;
  // exclusive scan of ties
  int tinc = tie;
  {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(tinc, o, 64);
      if (lane >= o) tinc += y;
    }
    if (lane == 63) wtie[wid] = tinc;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wid; ++w2) base += wtie[w2];
    tinc += base;
    __syncthreads();
  }
  const int tie_before = tinc - tie;
  long long kt = (long long)m - tie_before;
  if (kt < 0) kt = 0;
  if (kt > tie) kt = tie;
  const unsigned long long segk = (b < nb) ? w.seg_gt[b] + (unsigned long long)kt * qf : 0ull;
  const int segn = (b < nb) ? w.seg_gtn[b] + (int)kt : 0;
  const unsigned long long cinc = block_incl_scan_u64(segk, red);
  if (b == 0) seg_s = nb - 1;
  if (b == nb - 1) kept_s = cinc;
  __syncthreads();
  const double r = st.u * (double)kept_s;
  // first segment with kept entries whose inclusive cumulative mass >= r
  const bool hit = (b < nb) && segn > 0 && (double)cinc >= r;
  // smallest such b: reduce with atomicMin in LDS
  if (hit) atomicMin(&seg_s, b);
  __syncthreads();
  if (b == seg_s) { cum_before_s = cinc - segk; tie_base_s = tie_before; }
  __syncthreads();
  // level B: entries of the chosen segment, one per thread
  const int sb = seg_s;
  const int i = sb * SEG + threadIdx.x;
  const float q = (i < V) ? w.q[i] : 0.f;
  const int is_tie = (i < V && q == qs) ? 1 : 0;
  // rank of this tie among the segment's ties
  int tr = is_tie;
  {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(tr, o, 64);
      if (lane >= o) tr += y;
    }
    __syncthreads();
    if (lane == 63) wtie[wid] = tr;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wid; ++w2) base += wtie[w2];
    tr += base;
  }
  const int tie_rank = tie_base_s + tr - is_tie;
  const bool kept = (i < V) && ((q > qs) || (is_tie && tie_rank < m));
  const unsigned long long mass = kept ? ((q > qs) ? fx(q) : qf) : 0ull;
  const unsigned long long run = cum_before_s + block_incl_scan_u64(mass, red);
  __shared__ int tok;
  if (threadIdx.x == 0) tok = 0x7fffffff;
  __syncthreads();
  if (kept && (double)run >= r) atomicMin(&tok, i);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (tok == 0x7fffffff) {   // defensive: never leave an out-of-range id
      float bm = -INFINITY;
      int bi = 0;
      for (int k = 0; k < nb; ++k)
        if (w.bmax[k] > bm) { bm = w.bmax[k]; bi = w.barg[k]; }
      tok = bi;
    }
    *token = tok;
  }
}

int launch_sample(const SampleArgs& s, Exec st) {
  const int nb = (s.V + SEG - 1) / SEG;
  if (nb > 1024 || s.V > (1 << 18)) return -1;
  SampWs w = carve(s.ws, s.V);
  const float T = s.temperature;
  const float* td = s.temperature_dev;
  DS4G_LAUNCH(samp_max_kernel, dim3(nb), dim3(256), 0, st, s.logits, s.V, w);
  // a host temperature picks the path here; a device one, inside every kernel
  if (td || !(T > 0.f))
    DS4G_LAUNCH(samp_argmax_kernel, dim3(1), dim3(64), 0, st, nb, w, s.token, T, td);
  if (!td && !(T > 0.f)) return 0;
  DS4G_LAUNCH(samp_q_kernel, dim3((nb + QSEGS - 1) / QSEGS), dim3(1024), 0, st, s.logits,
                     s.V, nb, T, td, w);
  DS4G_LAUNCH(samp_level1_kernel, dim3(1), dim3(1024), 0, st, s.top_p, w, T, td);
  DS4G_LAUNCH(samp_hist2_kernel, dim3(nb), dim3(256), 0, st, s.V, w, T, td);
  DS4G_LAUNCH(samp_l2sum_kernel, dim3(NB2 / 1024), dim3(256), 0, st, w, T, td);
  DS4G_LAUNCH(samp_level2_kernel, dim3(1), dim3(1024), 0, st, w, s.rng, s.min_p, T, td);
  DS4G_LAUNCH(samp_segsum_kernel, dim3(nb), dim3(256), 0, st, s.V, w, T, td);
  DS4G_LAUNCH(samp_pick_kernel, dim3(1), dim3(1024), 0, st, s.V, nb, w, s.token, T, td);
  return 0;
}

// ---------------------------------------------------------------------------
// Token embedding (ds4-learning 端到端推理流程, 阶段四 4.1): row id of the
// table, widened to fp32.  One block per token; ids outside the table give a
// zero row.  `ids` may live on the device only (sampled tokens).
template <typename WT>
__global__ void __launch_bounds__(256)
embed_kernel(const WT* __restrict__ table, const int* __restrict__ ids, int vocab, int hidden,
             float* __restrict__ x) {
  const int t = blockIdx.x;
  const int id = ids[t];
  const bool ok = id >= 0 && id < vocab;
  const WT* row = table + (long)(ok ? id : 0) * hidden;
  float* out = x + (long)t * hidden;
  for (int c = threadIdx.x; c < hidden / 8; c += blockDim.x) {
    Chunk8<WT> ch;
    ch.load(row + c * 8);
    float f[8];
    ch.widen(f);
    float4* o4 = reinterpret_cast<float4*>(out + c * 8);
    o4[0] = ok ? make_float4(f[0], f[1], f[2], f[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
    o4[1] = ok ? make_float4(f[4], f[5], f[6], f[7]) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

int launch_embed(const void* table, int wdtype_bf16, const int* ids, int T, int vocab, int hidden,
                 float* x, Exec st) {
  if (hidden % 8 || T <= 0) return -1;
  if (wdtype_bf16)
    DS4G_LAUNCH((embed_kernel<uint16_t>), dim3(T), dim3(256), 0, st,
                       (const uint16_t*)table, ids, vocab, hidden, x);
  else
    DS4G_LAUNCH((embed_kernel<float>), dim3(T), dim3(256), 0, st, (const float*)table, ids,
                       vocab, hidden, x);
  return 0;
}

}  // namespace ds4g
