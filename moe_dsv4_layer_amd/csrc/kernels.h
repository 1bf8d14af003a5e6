// Internal interfaces between the ds4g host code and its HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4g {

// Where a launcher enqueues its kernels.  With dry set it only checks its
// preconditions and returns their verdict (0 or -1) without enqueuing
// anything: the C ABI runs every call's whole launch sequence dry first, so
// a shape some launcher cannot handle is rejected before any kernel runs.
struct Exec {
  hipStream_t stream;
  bool dry;
};
#define DS4G_LAUNCH(kern, grid, block, shm, ex, ...)                              \
  do {                                                                           \
    if (!(ex).dry) hipLaunchKernelGGL(kern, grid, block, shm, (ex).stream, __VA_ARGS__); \
  } while (0)

// ---------------------------------------------------------------- GEMM
enum Epi {
  EPI_F32 = 0,          // C[r, n] = acc                      (fp32)
  EPI_BF16 = 1,         // C[r, n] = bf16(acc)
  EPI_RESID = 2,        // C[r, n] += acc                     (fp32)
  EPI_SWIGLU_BF16 = 3,  // C[r, n] = bf16(silu(A.G^T) * (A.U^T))
  EPI_SWIGLU_F32 = 4,   // same, fp32 out
  // [q | k | v] = A.B^T with RoPE applied to q and k, all rounded to fp16:
  // q -> C [rows, ldc], k -> rope_kc [rows, dh], v -> rope_vc [rows, dh]
  EPI_ROPE_QKV = 5,
  EPI_F16 = 6           // C[r, n] = fp16(acc)
};

struct GemmArgs {
  const void* A;        // activations [rows, K]: bf16 / fp16 (MFMA) or fp32 (SIMT)
  int lda;
  int f16;              // MFMA: A and B are fp16 (else bf16)
  // optional per-output-column factor applied to the accumulator before the
  // epilogue (the inverse of a weight row's power-of-two scale)
  const float* colscale;
  const int* gather;    // optional: A row of output row r is gather[r]
  const void* B;        // weights [N, K] (group g at B + g*b_stride)
  const void* B2;       // SwiGLU: up weights (B holds gate)
  long b_stride;
  int brep;             // MFMA: B [N, brep] is repeated along K (K = a multiple of brep);
                        // B rows at stride brep, column k % brep (0: B is [N, K])
  int M, N, K;          // M: rows when not grouped
  const int* tiles;     // grouped: packed (group << 16 | m_tile), device
  const int* ntiles;    // grouped: number of valid tiles, device
  const int* row_off;   // grouped: [G+1] first row of each group, device
  int max_tiles;        // grouped: grid bound (>= *ntiles)
  int rows_hint;        // grouped: expected rows per group (picks the tile height)
  int epi;
  void* C;
  int ldc;
  // SIMT split-K: blockIdx.z of ksplit writes its partial sum to C + z * part_stride
  int ksplit;
  long part_stride;
  int xcd_remap;        // MFMA: renumber tiles so each XCD runs a contiguous run
  int stage16;          // MFMA, 16-bit outputs: store 16-byte row chunks through LDS (for
                        // tiles that are mostly full; 16-byte aligned C, N and ldc % 8 == 0)
  // EPI_ROPE_QKV: cos / sin of pair i at row r in rope_c / rope_s [i * rope_ld + r]
  // (rope_ld a multiple of 4, >= rows); q columns [0, qd) are heads of dh,
  // then k, then v; pairs (e, e+1) with e >= dh - rd rotate
  const float* rope_c;
  const float* rope_s;
  int rope_ld, rope_dh, rope_rd;
  uint16_t* rope_kc;
  uint16_t* rope_vc;
};
// fp16 image of a bf16 weight matrix W [N, K]: row n is scaled by a power of
// two 2^s_n that puts its largest magnitude in [2^14, 2^15) (s_n = 0 for a
// zero row), so every bf16 value of magnitude at least 2^-32 times the row's
// largest converts exactly; inv[n] = 2^-s_n undoes it in an epilogue.
int launch_f16_image(const uint16_t* W, int N, int K, uint16_t* img, float* inv, Exec st);
// cos / sin of pair i for rows t < T at position *pos + t into c / s
// [i * ld + t] (rows T..ld-1: 1 and 0), i < rd / 2
int launch_rope_table(const int64_t* pos, int T, int ld, int rd, float base, float* c, float* s,
                      Exec st);
int launch_gemm(const GemmArgs& g, bool mfma, int wdtype_bf16, Exec st);
// sum of nsplit fp32 partials part[s * pstride + m * N + n] in split order,
// then the column factor (colscale, optional) and the epilogue epi (F32,
// BF16, F16, RESID: C += sum, SWIGLU_BF16: part2 holds the up projection's
// partials) into C [M, ldc]
int launch_splitk_reduce(const float* part, const float* part2, int nsplit, long pstride, int M,
                         int N, int epi, void* C, int ldc, const float* colscale, Exec st);

// ---------------------------------------------------------------- GEMV
// out[n] (= or +=) sum_k W[n, k] xs[k], xs = x or RMSNorm(x) * gamma.
struct GemvArgs {
  const void* W;
  int N, K;
  const float* x;
  const void* gamma;    // optional fused RMSNorm gain
  float eps;
  float* out;
  int accumulate;
  float* router_in;     // optional copy of xs (block 0)
  // optional (the lm_head launch feeds the sampler with them): per block,
  // the largest output it wrote and its lowest row (INT_MAX when every
  // output was NaN or -inf), one entry per block of gemv_grid(N, K); and
  // zero_words 32-bit words at zero to clear
  float* blockmax;
  int* blockarg;
  uint32_t* zero;
  int zero_words;
};
template <typename WT>
int launch_gemv(const GemvArgs& a, Exec st);
// blocks of the launch_gemv grid for N rows of K (0 when K is too long)
int gemv_grid(int N, int K);

// out[m, n] = sum_k W[n, k] X[m, k] for the M <= 8 rows of a batched decode
// call: W [N, K] bf16 (row stride K), X [M, K] bf16 or fp16 (x_f16; row
// stride lda).  epi: EPI_F32, EPI_BF16, EPI_F16, EPI_RESID (C[m, n] += out) or
// EPI_SWIGLU_BF16 (W: gate, W2: up, C = bf16(silu(gate) * up)); C [M, ldc].
// -1 when the shape is not covered (M > 8, K > 4096, K % 8), launching
// nothing.
struct GemvRowsArgs {
  const uint16_t* W;
  const uint16_t* W2;
  int N, K;
  const uint16_t* X;
  int x_f16;
  int lda, M;
  int epi;
  void* C;
  int ldc;
};
int launch_gemv_rows(const GemvRowsArgs& a, Exec st);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const float* qkv;     // [T, H*dh + 2*dh] fp32
  int T, H, dh, rd, W;
  float base;
  int64_t* pos;         // device
  void* q;              // [T, H, dh] rotated (fp32, or fp16 with q_f16)
  int q_f16;
  uint16_t* kc;         // [T, dh] fp16 rotated keys
  uint16_t* vc;         // [T, dh] fp16 values
  uint16_t* ring_k;     // fp16 [W, dh] (batched decode: [B, W, dh])
  uint16_t* ring_v;
  void* o;              // [T, H*dh] attention output (fp32, or fp16 with o_f16)
  int o_f16;
  int heads_per_block;
  int rope_done;        // MFMA prefill: q, kc, vc already rotated (QKV GEMM epilogue)
};
int launch_attention(const AttnArgs& a, Exec st);
// single-token attention: RoPE of q/k at *pos, write (k, v) to the ring
// slot, attend over the window; o fp32 [H*dh].  Does not advance *pos.
int launch_attention_decode(const AttnArgs& a, Exec st);
// B independent sequences, one token each: row b of qkv at position pos[b],
// ring b at ring_k / ring_v + b * W * dh; o [B, H*dh] fp32 or fp16 (o_f16).
// Does not advance pos (the layer's last kernel, the combine, does).
int launch_attention_decode_batch(const AttnArgs& a, int B, Exec st);
// prefill on the matrix cores: fp16 q (q_f16 = 1) and o (o_f16 = 1)
int launch_attention_prefill_mfma(const AttnArgs& a, Exec st);

// ---------------------------------------------------------------- decode MoE
struct MoeDecodeArgs {
  const float* h2;        // [d]
  const void* ffn_norm;   // [d]
  float eps;
  const void* router;     // [E, d]
  float* logits_out;      // [E] written by the router kernel
  const float* logits;    // [E] read by the gate/up kernel (same buffer)
  int E, k, d, I, Is;
  const void *gate, *up, *down, *sh_gate, *sh_up, *sh_down;
  float* z;               // [k*I + Is]: routed slots, then the shared expert
  int nsd;                // shared gate/up blocks of the gate/up launch (set by the launcher)
  int* sel;               // [k] workspace
  float* wsel;            // [k] workspace
  // optional routing outputs
  int* topk_idx; float* topk_w; int* count; int* offset; int* perm; float* router_in;
};
// router logits, shared + routed gate/up, routed + shared down with the
// combine and residual: three launches
template <typename WT>
int launch_moe_decode(const MoeDecodeArgs& a, float* x, int64_t* pos_inc, Exec st);

// ---------------------------------------------------------------- prefill misc
// RMSNorm(x) * gamma of T rows into any of: fp32, bf16, fp16, and the
// three-term bf16 split y1 | y2 | y3 (y1 = bf16(y), y2 = bf16(y - y1), ...)
template <typename WT>
int launch_rmsnorm_rows(const float* x, int T, int d, const WT* gamma, float eps,
                        float* out_f32, uint16_t* out_bf16, uint16_t* out_f16,
                        uint16_t* out_split3, Exec st);

struct RouteArgs {
  const float* logits;  // nsplit partial sums [nsplit][T][E], added in order
  int nsplit;
  float* logits_sum;    // [T, E] the summed logits (router output)
  int T, E, k;
  int* topk_idx;        // [T, k]
  float* topk_w;        // [T, k]
  int* count;           // [E]
  int* offset;          // [E+1]
  int* rank;            // [T, k] rank of entry inside its expert within its chunk
  int* chunk;           // [ceil(T*k / kRankChunk), E] per chunk: entries of each expert,
                        // then the entries of that expert in earlier chunks
  int* perm;            // [T*k]
  int* gather;          // [T*k] token of each permuted row
  int* pos_of;          // [T*k] permuted row of entry t*k+j
  int* tiles;           // [max_tiles]
  int* ntiles;          // [1]
  int tile_m;           // rows per GEMM tile
  // optional user copies
  int* out_count; int* out_offset;
};
// entries ranked per chunk (one block of kRankChunk threads each: little LDS,
// so it fits beside the shared expert's GEMM blocks on the second stream)
constexpr int kRankChunk = 256;
int launch_route(const RouteArgs& r, Exec st);
// x[t] += sum_j w[t,j] part[pos_of[t*k+j]] (fixed j order); part is fp32, or bf16
// when part_bf16 (the bf16 path rounds each routed expert output to bf16).
// pos_inc (optional, batched decode): pos_inc[t] += 1 for every row t.
int launch_moe_combine(float* x, const void* part, int part_bf16, const int* pos_of,
                       const float* w, int T, int d, int k, int64_t* pos_inc, Exec st);

// ---------------------------------------------------------------- sampler
struct SampleArgs {
  const float* logits;
  int V;
  float temperature, top_p, min_p;
  const float* temperature_dev;   // optional device temperature (overrides temperature)
  uint64_t* rng;
  int* token;
  void* ws;             // sampler workspace
  int nbm;              // blocks of the lm_head GEMV that wrote the maxima
};
size_t sample_ws_bytes(int V);
// What the lm_head GEMV writes for the sampler inside its workspace: the
// words to clear and the per-block maxima (GemvArgs::zero / blockmax).
struct SampleScratch {
  uint32_t* zero;
  int zero_words;
  float* bmax;
  int* barg;
};
SampleScratch sample_scratch(void* ws, int V);
int launch_embed(const void* table, int wdtype_bf16, const int* ids, int T, int vocab, int hidden,
                 float* x, Exec st);
int launch_sample(const SampleArgs& s, Exec st);

}  // namespace ds4g
