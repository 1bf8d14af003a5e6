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
// order.  The roulette is a two-level prefix sum (4096-entry segments, then
// the entries of one segment).  Every step is deterministic.
//
// Launches.  The lm_head GEMV before the sampler leaves, per block, its
// largest logit and that logit's lowest row, and clears the level-1 histogram.  Then
// one launch per grid-wide dependency: (1) weights and the level-1 histogram
// (every block reduces the GEMV's maxima to the global maximum itself);
// (2) the level-2 histogram of the crossing level-1 bucket (every block finds
// that bucket itself from the level-1 histogram); (3) per segment, the mass
// and counts above and at the exact cut (every block finds the cut itself
// from the level-2 histogram); (4) one block: the draw, the segment and the
// entry.  A decision that every block needs is recomputed by every block from
// a few KB in L2 rather than handed over through memory: on this chip a
// grid-wide hand-off inside a launch (device-scope release, arrival count,
// acquire) costs several times the 1.7 us of a launch boundary in a graph.
#include "dev.h"
#include "kernels.h"

namespace ds4g {

namespace {
constexpr int SB = 1024;           // threads per sampler block
constexpr int SEG = 4096;          // entries per block and per roulette segment (4 per thread)
constexpr int NBM = 2048;          // lm_head GEMV blocks at most (block maxima)
constexpr int NB2 = 65536;         // level-2 buckets (low 16 bits)
constexpr int NG2 = NB2 / 1024;    // level-2 groups of 1024 buckets
constexpr double FX = 35184372088832.0;   // 2^45
// level-1 keys (top 16 bits of q) below KLO (q < 2^-45, exponent field < 82)
// have no fixed-point mass: fx(q) = 0 there, so they need no bucket
constexpr int KLO = 82 << 7;
constexpr int NKEY = 0x3F80 + 1 - KLO;   // keys KLO..0x3F80 (q <= 1)
constexpr int MAX_SEGS = (1 << 18) / SEG;   // V <= 2^18: one pick thread per segment

__device__ __forceinline__ uint64_t fx(float q) { return (uint64_t)((double)q * FX); }

// Decisions the last kernels share (written by block 0 of the kernel that
// makes them, read by later launches).
struct SampState {
  uint32_t b1;               // level-1 crossing key (q bits >> 16)
  int found;                 // the level-1 crossing exists (some mass)
  unsigned long long above1; // mass of keys above b1
  double target;             // top_p * total mass (at least 0.5)
  uint32_t vstar;            // bits of the cut weight q*
  int m;                     // entries equal to q* that are kept (index order)
};

struct SampWs {
  unsigned long long* h1;   // [NKEY] level-1 mass per key (cleared by the lm_head launch)
  unsigned long long* h2;   // [NB2] level-2 mass per bucket    } cleared by
  unsigned int* c2;         // [NB2] level-2 entries per bucket } the weight
  unsigned long long* g2;   // [NG2] level-2 mass per group     } launch
  float* bmax;              // [NBM] per lm_head block: largest logit
  int* barg;                // [NBM] and its lowest row
  float* q;                 // [V] weights
  unsigned long long* seg_gt; int* seg_gtn; int* seg_tie;   // per segment
  SampState* st;
};

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// h1, h2, c2 and g2, contiguous from the start of the workspace
constexpr size_t kH2Off = align256((size_t)NKEY * 8);
constexpr size_t kC2Off = kH2Off + (size_t)NB2 * 8;
constexpr size_t kG2Off = kC2Off + (size_t)NB2 * 4;
constexpr size_t kZeroBytes = kG2Off + (size_t)NG2 * 8;

__host__ __device__ inline SampWs carve(void* base, int V, size_t* total = nullptr) {
  const int ns = (V + SEG - 1) / SEG;
  char* p = static_cast<char*>(base);
  SampWs w;
  w.h1 = (unsigned long long*)p;
  w.h2 = (unsigned long long*)(p + kH2Off);
  w.c2 = (unsigned int*)(p + kC2Off);
  w.g2 = (unsigned long long*)(p + kG2Off);
  size_t o = align256(kZeroBytes);
  w.bmax = (float*)(p + o); o = align256(o + NBM * sizeof(float));
  w.barg = (int*)(p + o); o = align256(o + NBM * sizeof(int));
  w.q = (float*)(p + o); o = align256(o + (size_t)V * sizeof(float));
  w.seg_gt = (unsigned long long*)(p + o); o = align256(o + ns * 8);
  w.seg_gtn = (int*)(p + o); o = align256(o + ns * 4);
  w.seg_tie = (int*)(p + o); o = align256(o + ns * 4);
  w.st = (SampState*)(p + o); o = align256(o + sizeof(SampState));
  if (total) *total = o;
  return w;
}

// inclusive scans of one value per lane / per thread (blockDim SB; red holds
// one value per wave)
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}
__device__ __forceinline__ int wave_incl_scan_int(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  return v;
}
__device__ unsigned long long block_incl_scan_u64(unsigned long long v, unsigned long long* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_incl_scan_u64(v);
  __syncthreads();
  if (lane == 63) red[wid] = v;
  __syncthreads();
  unsigned long long base = 0;
  for (int w = 0; w < wid; ++w) base += red[w];
  __syncthreads();
  return v + base;
}
__device__ int block_incl_scan_int(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_incl_scan_int(v);
  __syncthreads();
  if (lane == 63) red[wid] = v;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += red[w];
  __syncthreads();
  return v + base;
}

// wave sum of an int on the DPP lane network (as wave_sum); every lane gets it
__device__ __forceinline__ int wave_sum_int_dpp(int v) {
#define DS4G_DPP_I(ctrl, rm, bc) v += __builtin_amdgcn_update_dpp(0, v, ctrl, rm, 0xF, bc)
  DS4G_DPP_I(0x111, 0xF, true); DS4G_DPP_I(0x112, 0xF, true); DS4G_DPP_I(0x114, 0xF, true);
  DS4G_DPP_I(0x118, 0xF, true); DS4G_DPP_I(0x142, 0xA, false); DS4G_DPP_I(0x143, 0xC, false);
#undef DS4G_DPP_I
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint64_t splitmix64_next(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The temperature of a call: a host value, or one read from device memory
// each time (tdev), so that a captured graph can switch between sampling and
// argmax without being captured again.
__device__ __forceinline__ float call_temperature(float temperature, const float* tdev) {
  return tdev ? *tdev : temperature;
}

// The largest logit and its first index, from the lm_head blocks' maxima
// (block-wide, every thread gets both).  INT_MAX when every logit is NaN or
// -inf.
__device__ __forceinline__ void global_argmax(const SampWs& w, int nbm, float& m, int& mi,
                                              float* redf, int* redi) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  m = -INFINITY;
  mi = 0x7fffffff;
  for (int b = threadIdx.x; b < nbm; b += blockDim.x) {
    const float v = w.bmax[b];
    const int i = w.barg[b];
    if (v > m || (v == m && i < mi)) { m = v; mi = i; }
  }
  wave_argmax(m, mi);
  if (lane == 0) { redf[wid] = m; redi[wid] = mi; }
  __syncthreads();
  m = redf[0];
  mi = redi[0];
  for (int k = 1; k < (int)(blockDim.x >> 6); ++k)
    if (redf[k] > m || (redf[k] == m && redi[k] < mi)) { m = redf[k]; mi = redi[k]; }
}

// The level-1 crossing (block-wide, every thread): the total mass, the
// target, and the key where the descending cumulative mass reaches it.
// Returns whether a crossing exists (false when no weight has mass).
__device__ bool level1_cut(const SampWs& w, float top_p, uint32_t* b1,
                           unsigned long long* above1, double* target,
                           unsigned long long* red, unsigned long long* sh) {
  constexpr int PER = (NKEY + SB - 1) / SB;
  const int tid = threadIdx.x;
  unsigned long long loc[PER], s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int k = NKEY - 1 - (tid * PER + j);
    loc[j] = (k >= 0) ? w.h1[k] : 0ull;
    s += loc[j];
  }
  const unsigned long long inc = block_incl_scan_u64(s, red);
  if (tid == SB - 1) sh[0] = inc;
  if (tid == 0) sh[1] = ~0ull;
  __syncthreads();
  double tg = (double)top_p * (double)sh[0];
  if (tg < 0.5) tg = 0.5;   // keep at least one token
  *target = tg;
  unsigned long long run = inc - s;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const unsigned long long nxt = run + loc[j];
    if ((double)run < tg && (double)nxt >= tg) {
      sh[1] = (unsigned long long)(KLO + (NKEY - 1 - (tid * PER + j)));
      sh[2] = run;
    }
    run = nxt;
  }
  __syncthreads();
  const bool found = sh[1] != ~0ull;
  *b1 = (uint32_t)sh[1];
  *above1 = sh[2];
  __syncthreads();
  return found;
}

// The exact cut (block-wide, every thread): bits of q* and how many entries
// equal to it are kept, from the level-1 decision and the level-2 histogram
// (top-p), then min-p.
// st: the level-1 decision; gs (wave 0): lane l holds the mass of level-2
// group NG2 - 1 - l.
__device__ void exact_cut(const SampWs& w, const SampState& st, unsigned long long gs,
                          float top_p, float min_p, uint32_t* vstar, int* m,
                          unsigned long long* red, unsigned long long* sh) {
  const int tid = threadIdx.x, wid = tid >> 6;
  uint32_t vs = 0u;          // top_p >= 1: every entry, those equal to 0 too
  int mk = 0x7fffffff;
  if (top_p < 1.0f) {
    // the group of 1024 level-2 buckets that holds the crossing (descending)
    if (tid == 0) sh[0] = ~0ull;
    __syncthreads();
    if (wid == 0) {
      const int lane = tid & 63;
      const unsigned long long run0 = st.above1 + wave_incl_scan_u64(gs) - gs;
      if ((double)run0 < st.target && (double)(run0 + gs) >= st.target) {
        sh[0] = (unsigned long long)(NG2 - 1 - lane);
        sh[1] = run0;
      }
    }
    __syncthreads();
    const int grp = (int)sh[0];
    const unsigned long long grun = sh[1];
    // that group's buckets, one per thread (descending), prefix-summed
    const uint32_t b2 = (grp >= 0 && grp < NG2) ? (uint32_t)(grp * 1024 + 1023 - tid) : 0u;
    const unsigned long long hv = (grp >= 0 && grp < NG2) ? w.h2[b2] : 0ull;
    const unsigned long long run = grun + block_incl_scan_u64(hv, red) - hv;   // mass before b2
    if (tid == 0) { sh[2] = 0ull; sh[3] = 0x7fffffffull; }
    __syncthreads();
    if (grp >= 0 && grp < NG2 && (double)run < st.target && (double)(run + hv) >= st.target) {
      const uint32_t vbits = (st.b1 << 16) | b2;
      const unsigned long long qf = fx(__uint_as_float(vbits));
      const unsigned int cnt = w.c2[b2];
      // the fewest equal-to-q* entries (in index order) that reach the target
      long long mm = (long long)ceil((st.target - (double)run) / (double)qf);
      if (mm < 1) mm = 1;
      if (mm > (long long)cnt) mm = cnt;
      while (mm > 1 && (double)(run + (unsigned long long)(mm - 1) * qf) >= st.target) --mm;
      while (mm < (long long)cnt && (double)(run + (unsigned long long)mm * qf) < st.target) ++mm;
      sh[2] = vbits;
      sh[3] = (unsigned long long)mm;
    }
    __syncthreads();
    vs = (uint32_t)sh[2];
    mk = (int)sh[3];
    __syncthreads();
  }
  // min-p: weights below min(min_p, 1) are dropped (the largest weight is
  // exactly 1); when that threshold lies above the top-p cut it becomes the
  // cut, and every entry equal to it is kept
  if (min_p > 0.f) {
    const float thr = fminf(min_p, 1.f);
    if (thr > __uint_as_float(vs)) { vs = __float_as_uint(thr); mk = 0x7fffffff; }
  }
  *vstar = vs;
  *m = mk;
}
}  // namespace

size_t sample_ws_bytes(int V) {
  size_t total = 0;
  carve(nullptr, V, &total);
  return total;
}

SampleScratch sample_scratch(void* ws, int V) {
  const SampWs w = carve(ws, V);
  SampleScratch s;
  s.zero = reinterpret_cast<uint32_t*>(w.h1);
  s.zero_words = NKEY * 2;   // h1 (the weight launch clears the level-2 histogram)
  s.bmax = w.bmax;
  s.barg = w.barg;
  return s;
}

// argmax over the lm_head blocks' maxima (host temperature <= 0)
__global__ void __launch_bounds__(SB)
samp_argmax_kernel(int nbm, SampWs w, int* token) {
  __shared__ float redf[16];
  __shared__ int redi[16];
  float m;
  int mi;
  global_argmax(w, nbm, m, mi, redf, redi);
  if (threadIdx.x == 0) *token = (mi == 0x7fffffff) ? 0 : mi;   // every logit NaN / -inf: 0
}

// (1) q = exp((l - M) / T) for this block's SEG entries, and their level-1
// masses: summed per key in LDS first, so that equal keys (a narrow logit
// spread puts thousands of weights in one key) cost one global atomic per
// block instead of one per entry.  A device temperature <= 0: block 0 writes
// the argmax and every later kernel returns at once.
__global__ void __launch_bounds__(SB)
samp_q_kernel(const float* __restrict__ logits, int V, int nbm, float temperature,
              const float* tdev, SampWs w, int* token) {
  __shared__ unsigned long long hist[NKEY];
  __shared__ float redf[16];
  __shared__ int redi[16];
  const int tid = threadIdx.x;
  // this block's logits are requested before anything waits on memory
  const int lo = blockIdx.x * SEG, hi = min(V, lo + SEG);
  float lg[SEG / SB];
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + tid + j * SB;
    lg[j] = (i < hi) ? logits[i] : 0.f;
  }
  for (int k = tid; k < NKEY; k += SB) hist[k] = 0;
  float M;
  int mi;
  global_argmax(w, nbm, M, mi, redf, redi);   // its barrier also covers the clearing
  const float t = call_temperature(temperature, tdev);
  if (!(t > 0.f)) {
    if (blockIdx.x == 0 && tid == 0) *token = (mi == 0x7fffffff) ? 0 : mi;
    return;
  }
  {   // clear the level-2 histogram for the next launch
    uint32_t* z = reinterpret_cast<uint32_t*>(w.h2);
    const int nz = (int)((kZeroBytes - kH2Off) / 4);
    for (int i = blockIdx.x * SB + tid; i < nz; i += gridDim.x * SB) z[i] = 0u;
  }
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + tid + j * SB;
    if (i >= hi) break;
    float q = expf((lg[j] - M) / t);
    q = (q == q) ? fminf(q, 1.f) : 0.f;   // a NaN logit weighs nothing; keys stay <= 0x3F80
    w.q[i] = q;
    const int key = (int)(__float_as_uint(q) >> 16) - KLO;
    if (key >= 0) atomicAdd(&hist[key], (unsigned long long)fx(q));
  }
  __syncthreads();
  for (int k = tid; k < NKEY; k += SB) {
    const unsigned long long v = hist[k];
    if (v) atomicAdd(&w.h1[k], v);
  }
}

// (2) every block: the level-1 crossing key b1 (block 0 records it for the
// later launches); then the level-2 histogram (mass, count, group mass) of
// this block's entries in bucket b1.
__global__ void __launch_bounds__(SB)
samp_hist2_kernel(int V, float top_p, float temperature, const float* tdev, SampWs w) {
  if (!(call_temperature(temperature, tdev) > 0.f) || top_p >= 1.0f) return;
  __shared__ unsigned long long red[16], sh[4];
  const int lo = blockIdx.x * SEG, hi = min(V, lo + SEG);
  float qv[SEG / SB];   // requested before the level-1 histogram is read
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + threadIdx.x + j * SB;
    qv[j] = (i < hi) ? w.q[i] : 0.f;
  }
  uint32_t b1;
  unsigned long long above1;
  double target;
  const bool found = level1_cut(w, top_p, &b1, &above1, &target, red, sh);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    SampState* st = w.st;
    st->b1 = b1; st->found = found ? 1 : 0; st->above1 = above1; st->target = target;
  }
  if (!found) return;
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + threadIdx.x + j * SB;
    if (i >= hi) break;
    const float q = qv[j];
    const uint32_t bits = __float_as_uint(q);
    if ((bits >> 16) == b1) {
      const unsigned long long f = fx(q);
      atomicAdd(&w.h2[bits & 0xFFFF], f);
      atomicAdd(&w.c2[bits & 0xFFFF], 1u);
      atomicAdd(&w.g2[(bits & 0xFFFF) >> 10], f);
    }
  }
}

// (3) every block: the exact cut (block 0 records it); then, for this
// block's segment, the mass strictly above q*, how many such entries, and how
// many entries equal q*.
__global__ void __launch_bounds__(SB)
samp_segsum_kernel(int V, float top_p, float min_p, float temperature, const float* tdev,
                   SampWs w) {
  if (!(call_temperature(temperature, tdev) > 0.f)) return;
  __shared__ unsigned long long red[16], sh[4];
  __shared__ int sn[16], st_[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // everything this block reads that no decision depends on, requested first
  const SampState sst = *w.st;
  const unsigned long long gs = (wid == 0) ? w.g2[NG2 - 1 - lane] : 0ull;
  const int lo = blockIdx.x * SEG, hi = min(V, lo + SEG);
  float qv[SEG / SB];
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + tid + j * SB;
    qv[j] = (i < hi) ? w.q[i] : 0.f;
  }
  if (top_p < 1.0f && !sst.found) return;
  uint32_t vstar;
  int mk;
  exact_cut(w, sst, gs, top_p, min_p, &vstar, &mk, red, sh);
  if (blockIdx.x == 0 && tid == 0) { w.st->vstar = vstar; w.st->m = mk; }
  const float qs = __uint_as_float(vstar);
  unsigned long long s = 0;
  int n = 0, t = 0;
#pragma unroll
  for (int j = 0; j < SEG / SB; ++j) {
    const int i = lo + tid + j * SB;
    if (i >= hi) break;
    const float q = qv[j];
    if (q > qs) { s += fx(q); ++n; }
    else if (q == qs) ++t;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  n = wave_sum_int_dpp(n);
  t = wave_sum_int_dpp(t);
  if (lane == 0) { red[wid] = s; sn[wid] = n; st_[wid] = t; }
  __syncthreads();
  if (tid == 0) {
    unsigned long long ss = 0;
    int nn = 0, tt = 0;
    for (int k = 0; k < SB / 64; ++k) { ss += red[k]; nn += sn[k]; tt += st_[k]; }
    w.seg_gt[blockIdx.x] = ss;
    w.seg_gtn[blockIdx.x] = nn;
    w.seg_tie[blockIdx.x] = tt;
  }
}

// (4) one block: the draw u, the kept mass K (exact, per segment in fixed
// point), r = u * K, then the segment and the entry where the running kept
// mass (vocabulary order) first reaches r.
__global__ void __launch_bounds__(SB)
samp_pick_kernel(int V, int ns, int nbm, float top_p, uint64_t* rng, SampWs w, int* token,
                 float temperature, const float* tdev) {
  if (!(call_temperature(temperature, tdev) > 0.f)) return;
  __shared__ unsigned long long red[16];
  __shared__ int redi[16];
  __shared__ int seg_s, tok_s, tie_base_s;
  __shared__ unsigned long long cum_before_s;
  __shared__ double r_s;
  __shared__ float redf[16];
  const int tid = threadIdx.x, lane = tid & 63;
  // what level A reads, requested at once: the cut, the segment sums, the
  // generator state
  const SampState sst = *w.st;
  const int b = lane;   // wave 0: one segment per lane (ns <= 64)
  const int tie = (tid < 64 && b < ns) ? w.seg_tie[b] : 0;
  const unsigned long long sgt = (tid < 64 && b < ns) ? w.seg_gt[b] : 0ull;
  const int sgn = (tid < 64 && b < ns) ? w.seg_gtn[b] : 0;
  const uint64_t rs = (tid == 0) ? *rng : 0ull;
  if (top_p < 1.0f && !sst.found) {   // no weight has mass: the argmax, no draw
    float m;
    int mi;
    global_argmax(w, nbm, m, mi, redf, redi);
    if (tid == 0) *token = (mi == 0x7fffffff) ? 0 : mi;
    return;
  }
  const float qs = __uint_as_float(sst.vstar);
  const unsigned long long qf = fx(qs);
  const int mk = sst.m;
  if (tid < 64) {
    double u = 0.0;
    if (tid == 0) {
      uint64_t st = rs;
      const uint64_t z = splitmix64_next(&st);
      *rng = st;
      u = (double)(z >> 40) * (1.0 / 16777216.0);
    }
    u = __shfl(u, 0, 64);
    // level A: the kept mass per segment (ties kept in index order) and its
    // running sum
    const int tie_before = wave_incl_scan_int(tie) - tie;
    long long kt = (long long)mk - tie_before;
    if (kt < 0) kt = 0;
    if (kt > tie) kt = tie;
    const unsigned long long segk = sgt + (unsigned long long)kt * qf;
    const int segn = sgn + (int)kt;
    const unsigned long long cinc = wave_incl_scan_u64(segk);
    const unsigned long long kept = __shfl(cinc, 63, 64);
    const double r = u * (double)kept;
    // the first segment with kept entries whose cumulative kept mass reaches r
    const uint64_t hit = __ballot(b < ns && segn > 0 && (double)cinc >= r);
    const int f = hit ? __builtin_ctzll(hit) : 0x7fffffff;
    if (tid == 0) { seg_s = f; tok_s = 0x7fffffff; r_s = r; }
    if (hit && lane == f) { cum_before_s = cinc - segk; tie_base_s = tie_before; }
  }
  __syncthreads();
  const double r = r_s;
  const int sg = seg_s;
  if (sg != 0x7fffffff) {
    // level B: that segment's entries in index order, 4 consecutive per
    // thread: the first kept one whose running kept mass reaches r
    const int i0 = sg * SEG + 4 * tid;
    float q[4];
    int ties = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[j] = (i0 + j < V) ? w.q[i0 + j] : 0.f;
      ties += (i0 + j < V && q[j] == qs) ? 1 : 0;
    }
    int rank = tie_base_s + block_incl_scan_int(ties, redi) - ties;
    bool kept[4];
    unsigned long long ms[4], lsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = i0 + j < V;
      const bool is_tie = ok && q[j] == qs;
      kept[j] = ok && (q[j] > qs || (is_tie && rank < mk));
      rank += is_tie ? 1 : 0;
      ms[j] = kept[j] ? ((q[j] > qs) ? fx(q[j]) : qf) : 0ull;
      lsum += ms[j];
    }
    unsigned long long cum = cum_before_s + block_incl_scan_u64(lsum, red) - lsum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kept[j]) {
        cum += ms[j];
        if ((double)cum >= r) { atomicMin(&tok_s, i0 + j); break; }
      }
    }
  }
  __syncthreads();
  int tk = tok_s;
  if (tk == 0x7fffffff) {   // defensive (r < K always meets a kept entry): never an invalid id
    float m;
    int mi;
    global_argmax(w, nbm, m, mi, redf, redi);
    tk = (mi == 0x7fffffff) ? 0 : mi;
  }
  if (tid == 0) *token = tk;
}

int launch_sample(const SampleArgs& s, Exec st) {
  if (s.V <= 0 || s.V > MAX_SEGS * SEG || s.nbm <= 0 || s.nbm > NBM) return -1;
  const SampWs w = carve(s.ws, s.V);
  const int ns = (s.V + SEG - 1) / SEG;
  const float T = s.temperature;
  const float* td = s.temperature_dev;
  if (!td && !(T > 0.f)) {
    DS4G_LAUNCH(samp_argmax_kernel, dim3(1), dim3(SB), 0, st, s.nbm, w, s.token);
    return 0;
  }
  DS4G_LAUNCH(samp_q_kernel, dim3(ns), dim3(SB), 0, st, s.logits, s.V, s.nbm, T, td, w, s.token);
  DS4G_LAUNCH(samp_hist2_kernel, dim3(ns), dim3(SB), 0, st, s.V, s.top_p, T, td, w);
  DS4G_LAUNCH(samp_segsum_kernel, dim3(ns), dim3(SB), 0, st, s.V, s.top_p, s.min_p, T, td, w);
  DS4G_LAUNCH(samp_pick_kernel, dim3(1), dim3(SB), 0, st, s.V, ns, s.nbm, s.top_p, s.rng, w,
              s.token,
              T, td);
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
