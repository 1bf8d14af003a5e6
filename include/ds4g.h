/*
 * ds4g -- one DeepSeek-V4-style transformer layer (ds4 / DwarfStar), its
 * layer-major prefill, its single-token decode, and the lm_head sampler, on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed follows the layer pseudo-code on the ds4-learning page
 * 端到端推理流程 (ds4.c 学习笔记), section 阶段四 4.2 单层前向:
 *
 *   x  = RMSNorm(h) * g1
 *   c  = A x ;  [q | k | v] = B c          low-rank QKV (one shared bottleneck)
 *   q, k <- RoPE(q, k, pos)                interleaved pairs, theta_i = base^(-2i/rope_dim)
 *   ring[pos mod W] <- (k, v)              KV cache kept as a W-slot ring
 *   o  = MQA(q, ring)                      H heads share one K/V; window of W keys incl. self
 *   h2 = h + W_o o
 *   y  = RMSNorm(h2) * g2
 *   s  = W_r y ; p = softmax(s) ; S = top-k(s)          (ties -> lower index)
 *   out = h2 + sum_{e in S} p_e D_e(silu(G_e y) * U_e y) + D_sh(silu(G_sh y) * U_sh y)
 *
 * Prefill runs this for T tokens layer-major (section 阶段三 逐层批处理);
 * decode is T = 1 (阶段四).  The lm_head and sampler follow 阶段四 4.3 采样:
 * logits = W_lm RMSNorm(x) * g_f, then temperature, top-p, roulette in
 * vocabulary order, or argmax at temperature 0.
 *
 * Conventions shared by every call:
 *   - Every pointer argument named "device" is HIP device memory owned by the
 *     caller; the library allocates nothing and keeps no global state (one
 *     exception: the static scratch array of ds4g_layer_decode_noalloc).
 *   - Weight matrices are row-major [out, in], all in cfg->wdtype
 *     (DS4G_BF16: raw bf16 bits; DS4G_F32: float).  Expert stacks are
 *     [n_experts, out, in].  Gains (norm weights) are in wdtype too.
 *   - The residual stream x is fp32, updated in place; on the matrix-core
 *     path some residual adds (the shared down, short prefills) are
 *     device-memory float atomics (one per element), so x must be ordinary
 *     device memory (hipMalloc), not host or managed memory.
 *   - The KV ring holds K (after RoPE) and V as fp16 (IEEE binary16)
 *     [window, head_dim]; position p lives in slot p % window; *pos (device
 *     int64) is the position of the next token and is advanced by every call.
 *   - With bf16 weights, a prefill (and a batched decode) carries the
 *     attention path -- normalised input, low-rank code, q, k, v, attention
 *     probabilities and output -- in fp16 on the matrix cores, against fp16
 *     images of QKV-A, QKV-B and W_o that the call makes in its workspace
 *     (each row scaled by a power of two; exact for every value at least 2^-32
 *     times the row's largest).  These activations must stay inside fp16's range
 *     (|v| < 65504).  The expert path stays bf16; the router sees fp32-quality
 *     inputs.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream).  They never synchronise and never call the allocator, so a
 *     decode step can be captured in a HIP graph and replayed.  A prefill or
 *     batched decode of 32 or more rows runs the shared expert on a second
 *     stream that the library creates once per device (default priority,
 *     never while `stream` is being captured; without it the work stays on
 *     `stream`), forked from and joined back into `stream` with events, so
 *     the call's work is still ordered on `stream`.
 *   - Every argument check runs on the host before anything is enqueued; on
 *     an error nothing is written and a negative ds4g_status is returned.
 *     A call first walks its whole launch sequence without enqueuing (each
 *     kernel launcher checks the shape it is given), so a size that some
 *     kernel does not implement is DS4G_ERR_UNSUPPORTED before the first
 *     launch, never a partial update.  DS4G_ERR_HIP reports a launch the HIP
 *     runtime refused (the stream state is then undefined).
 *   - A ring and a workspace must not be used by two calls at once.
 */
#ifndef DS4G_H
#define DS4G_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DS4G_OK = 0,
  DS4G_ERR_INVALID_ARG = -1,  /* null pointer, non-positive or inconsistent size */
  DS4G_ERR_UNSUPPORTED = -2,  /* a size outside what the kernels implement      */
  DS4G_ERR_WORKSPACE = -3,    /* ws_bytes smaller than ds4g_workspace_bytes()   */
  DS4G_ERR_HIP = -4           /* a HIP launch failed                            */
} ds4g_status;

typedef enum { DS4G_F32 = 0, DS4G_BF16 = 1 } ds4g_dtype;

/* The three layer calls, for ds4g_layer_supported. */
typedef enum {
  DS4G_MODE_PREFILL = 0,       /* ds4g_layer_prefill, T tokens            */
  DS4G_MODE_DECODE = 1,        /* ds4g_layer_decode, T = 1                */
  DS4G_MODE_DECODE_BATCH = 2   /* ds4g_layer_decode_batch, T sequences    */
} ds4g_mode;

/* Layer dimensions.  Supported: head_dim in {64, 128}; rope_dim even and
 * <= head_dim (0 = head_dim); window in [1, 128]; n_experts in [top_k+1, 512];
 * top_k in [1, 8]; n_heads a multiple of 4; hidden, qkv_rank, ffn_inter,
 * shared_inter and n_heads*head_dim multiples of 64; hidden, qkv_rank and
 * n_heads*head_dim <= 16384 (hidden <= 8192 for ds4g_layer_decode);
 * ffn_inter, shared_inter <= 2048 and top_k*ffn_inter + shared_inter <=
 * 12288.  ds4g_layer_supported answers for a given shape. */
typedef struct {
  int32_t hidden;        /* d: residual width (4096)                         */
  int32_t n_heads;       /* H: query heads (64); one K/V head (MQA)          */
  int32_t head_dim;      /* dh (128)                                         */
  int32_t qkv_rank;      /* r: low-rank bottleneck of the QKV projection     */
  int32_t window;        /* W: sliding-window length (128)                   */
  int32_t n_experts;     /* E: routed experts (256)                          */
  int32_t top_k;         /* k: experts per token (6)                         */
  int32_t ffn_inter;     /* I: SwiGLU inner width of a routed expert         */
  int32_t shared_inter;  /* inner width of the shared expert                 */
  int32_t rope_dim;      /* rotated tail of each head; 0 = whole head        */
  float rope_base;       /* 10000                                            */
  float rms_eps;         /* 1e-6                                             */
  int32_t wdtype;        /* ds4g_dtype of every weight                       */
} ds4g_layer_cfg;

/* Device pointers to one layer's weights ([out, in], wdtype). */
typedef struct {
  const void *attn_norm;  /* [d]                     g1                      */
  const void *qkv_a;      /* [r, d]                  A                       */
  const void *qkv_b;      /* [H*dh + 2*dh, r]        B: q heads, then k, v   */
  const void *wo;         /* [d, H*dh]               W_o                     */
  const void *ffn_norm;   /* [d]                     g2                      */
  const void *router;     /* [E, d]                  W_r                     */
  const void *gate;       /* [E, I, d]               G_e                     */
  const void *up;         /* [E, I, d]               U_e                     */
  const void *down;       /* [E, d, I]               D_e                     */
  const void *sh_gate;    /* [Is, d]                                         */
  const void *sh_up;      /* [Is, d]                                         */
  const void *sh_down;    /* [d, Is]                                         */
  /* Optional (bf16 weights): the layer's fp16 attention-path images made once
   * by ds4g_make_f16_images, device memory, 256-byte aligned.  NULL: every
   * prefill and batched decode makes them in its workspace (a read and a
   * write of QKV-A, QKV-B and W_o per call). */
  const void *f16_images;
} ds4g_layer_weights;

/* One layer's KV ring (device memory). */
typedef struct {
  void *k;        /* fp16 [window, head_dim], K after RoPE                   */
  void *v;        /* fp16 [window, head_dim]                                 */
  int64_t *pos;   /* position of the next token (>= 0)                       */
} ds4g_kv_ring;

/* Optional routing outputs (device memory; any member may be NULL). */
typedef struct {
  int32_t *topk_idx;       /* [T, k]  chosen experts, descending logit       */
  float *topk_w;           /* [T, k]  their softmax probabilities            */
  int32_t *expert_count;   /* [E]                                            */
  int32_t *expert_offset;  /* [E+1]  exclusive scan of expert_count          */
  int32_t *perm;           /* [T*k]  entries t*k+j grouped by expert, token
                                     order inside an expert                  */
  float *router_in;        /* [T, d]  y = RMSNorm(h2)*g2 as the router saw it */
  float *router_logits;    /* [T, E]  s                                       */
} ds4g_routing;

/* Bytes of the fp16 image buffer of ds4g_make_f16_images for this layer
 * shape: fp16 copies of QKV-A, QKV-B and W_o, each row scaled by a power of
 * two, and the rows' inverse factors.  0 for fp32 weights (they have none)
 * or invalid dimensions. */
size_t ds4g_f16_images_bytes(const ds4g_layer_cfg *cfg);

/* Make the fp16 images of a layer's attention-path weights once, so that its
 * prefills and batched decodes read them (set w->f16_images) instead of
 * making them per call.  images: device, >= ds4g_f16_images_bytes(cfg)
 * bytes, 256-byte aligned; owned by the caller and valid while the weights
 * are unchanged.  Asynchronous on `stream`.  Returns DS4G_OK or a negative
 * ds4g_status (DS4G_ERR_UNSUPPORTED for fp32 weights). */
int ds4g_make_f16_images(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w, void *images,
                         size_t images_bytes, void *stream);

/* Optional copies of a prefill's intermediate activations, in the order the
 * layer computes them (阶段四 4.2), for step-by-step parity checks: each
 * step's output can be compared with that step applied to the previous
 * step's copy.  Device memory; any member may be NULL.  "act" is the
 * attention path's activation type: fp16 with bf16 weights, fp32 with fp32
 * weights; k and v are always fp16 (the ring's type).
 *   x_norm [T, hidden]    act   RMSNorm(h) * g1, as QKV-A read it
 *   c      [T, qkv_rank]  act   A x_norm
 *   q      [T, H*dh]      act   B c, query heads, after RoPE
 *   k, v   [T, dh]        fp16  B c, key after RoPE, value (as cached)
 *   o      [T, H*dh]      act   attention output, as W_o read it
 *   h2     [T, hidden]    fp32  h + W_o o */
typedef struct {
  void *x_norm, *c, *q, *k, *v, *o;
  float *h2;
} ds4g_trace;

/* Bytes of workspace that covers every layer call for up to max_tokens
 * tokens (the largest need is a prefill's: its activations plus the fp16
 * images of QKV-A, QKV-B and W_o), and ds4g_lmhead_sample for `vocab` (pass
 * cfg = NULL for the lm_head alone).  ds4g_layer_decode needs less; each call
 * checks ws_bytes against its own need.  Returns 0 on invalid arguments. */
size_t ds4g_workspace_bytes(const ds4g_layer_cfg *cfg, int32_t max_tokens,
                            int32_t vocab);

/* Whether a layer call of this mode with these dimensions would be accepted
 * (DS4G_OK), or the status it would return for a shape reason
 * (DS4G_ERR_INVALID_ARG, DS4G_ERR_UNSUPPORTED).  Runs the host checks and
 * the call's launch sequence without enqueuing anything; needs no device and
 * touches no memory.  T: tokens (prefill), 1 (decode), or sequences (batched
 * decode).  Pointer, alignment and workspace-size checks are not covered. */
int ds4g_layer_supported(const ds4g_layer_cfg *cfg, int32_t T, int32_t mode);

/* Layer-major prefill of T >= 1 tokens at positions *ring->pos ..
 * *ring->pos + T - 1 (阶段三 逐层批处理; 阶段四 4.2 for the layer).
 *   x:  device fp32 [T, hidden], the layer input h; overwritten with the
 *       layer output.
 *   ring: updated with the last min(T, window) keys/values; *pos += T.
 *   routing: optional outputs (NULL = none).
 *   ws: device workspace of at least ds4g_workspace_bytes(cfg, T, 0) bytes,
 *       256-byte aligned.
 * Returns DS4G_OK or a negative ds4g_status. */
int ds4g_layer_prefill(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w,
                       ds4g_kv_ring *ring, float *x, int32_t T,
                       ds4g_routing *routing, void *ws, size_t ws_bytes,
                       void *stream);

/* ds4g_layer_prefill that also writes the intermediate activations named in
 * `trace` (NULL: none).  Same arguments, results and errors otherwise. */
int ds4g_layer_prefill_trace(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w,
                             ds4g_kv_ring *ring, float *x, int32_t T, ds4g_routing *routing,
                             const ds4g_trace *trace, void *ws, size_t ws_bytes, void *stream);

/* One decode step (T = 1) of the layer at position *ring->pos (阶段四 4.2).
 * Same contract as ds4g_layer_prefill with T = 1; uses the bandwidth-bound
 * decode kernels.  x: device fp32 [hidden]. */
int ds4g_layer_decode(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w,
                      ds4g_kv_ring *ring, float *x, ds4g_routing *routing,
                      void *ws, size_t ws_bytes, void *stream);

/* ds4g_layer_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as ds4g_layer_decode, minus
 * the workspace: the step's scratch is a static device array of 2 MiB that
 * the library holds on every GPU it runs on until the process ends (the
 * first call on a device looks up its address; nothing is allocated, ever).
 * Every decode shape ds4g_layer_supported accepts fits in it; a layer whose
 * decode would need more returns DS4G_ERR_WORKSPACE.  The array keeps what
 * the last call left, and no byte of it needs to start at zero (every byte a
 * step reads was written earlier in the same step).  All calls on one GPU
 * share the array: calls that overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller. */
int ds4g_layer_decode_noalloc(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w,
                              ds4g_kv_ring *ring, float *x, ds4g_routing *routing,
                              void *stream);

/* Batched decode: one token of each of B >= 1 independent sequences through
 * the layer (the throughput form of 阶段四 4.2's single-token step; the
 * pages' server decodes one sequence at a time).  Sequence b is at position
 * rings->pos[b] and owns ring b.
 *   rings: k, v device [B, window, head_dim] in the ring's dtype (ring b at
 *          offset b * window * head_dim), pos device int64 [B]; ring b gets the
 *          token's key/value at slot pos[b] % window and pos[b] += 1.
 *   x:     device fp32 [B, hidden], row b the layer input of sequence b;
 *          overwritten with the layer output.
 *   routing: optional outputs as for ds4g_layer_prefill with T = B (row b =
 *          sequence b).
 *   ws:    at least ds4g_workspace_bytes(cfg, B, 0) bytes, 256-byte aligned.
 * The projections, router and experts run as in ds4g_layer_prefill over the
 * B rows (weights read once for all of them); each row's attention sees only
 * its own ring.  Returns DS4G_OK or a negative ds4g_status (B > 65535:
 * DS4G_ERR_UNSUPPORTED). */
int ds4g_layer_decode_batch(const ds4g_layer_cfg *cfg, const ds4g_layer_weights *w,
                            ds4g_kv_ring *rings, float *x, int32_t B,
                            ds4g_routing *routing, void *ws, size_t ws_bytes,
                            void *stream);

/* lm_head + sampler for one token (阶段四 4.3 采样).
 *   final_norm: device [hidden] gain in wdtype, or NULL to skip the norm.
 *   w_lm:   device [vocab, hidden] in wdtype.
 *   x:      device fp32 [hidden].
 *   temperature <= 0 picks the argmax (first index among equal maxima) and
 *   leaves *rng_state alone; otherwise q_i = exp((l_i - max l)/temperature),
 *   top-p keeps the most probable tokens (ties -> lower index) until their
 *   share reaches top_p (the crossing token is kept; top_p >= 1 keeps all),
 *   and the roulette walks the vocabulary in index order with
 *   r = u * (sum of kept q), u from one splitmix64 draw of *rng_state
 *   (top 24 bits / 2^24).
 *   rng_state: device uint64 (may be NULL when temperature <= 0).
 *   logits: device fp32 [vocab] out.  token: device int32 out.
 *   embed_table, x_next: optional, both or neither: after sampling, x_next
 *   (device fp32 [hidden]) receives the embedding of the sampled token
 *   (table [vocab, hidden] in wdtype), so a decode loop stays on the device.
 *   ws: at least ds4g_workspace_bytes(NULL, 0, vocab) bytes. */
int ds4g_lmhead_sample(int32_t hidden, int32_t vocab, int32_t wdtype,
                       const void *final_norm, float rms_eps, const void *w_lm,
                       const float *x, float temperature, float top_p,
                       uint64_t *rng_state, float *logits, int32_t *token,
                       const void *embed_table, float *x_next,
                       void *ws, size_t ws_bytes, void *stream);

/* Sampling parameters of ds4g_lmhead_sample_ex.
 *   temperature, top_p: as for ds4g_lmhead_sample.
 *   min_p: the min-p filter that the page's function index names together
 *     with top-p (sample_top_p_min_p; 阶段四 4.3 and the index table): a
 *     token stays only if q_i >= min(min_p, 1) * max q; with top-p a token is
 *     kept when both keep it.  min_p <= 0 disables it.
 *   temperature_dev: NULL, or a device float read by every call in place of
 *     `temperature` (<= 0 or NaN: argmax, rng untouched).  It is the per-token
 *     temperature override of the page's tool-call mode (阶段六 温度覆盖:
 *     structural tokens at temperature 0): a captured decode graph switches
 *     between sampling and argmax by writing that float, with no re-capture.
 *     rng_state must then be non-NULL. */
typedef struct {
  float temperature, top_p, min_p;
  const float *temperature_dev;
} ds4g_sample_params;

/* ds4g_lmhead_sample with min-p and the device temperature override;
 * ds4g_lmhead_sample is this call with min_p = 0 and temperature_dev = NULL.
 * params: host pointer, read during the call.  Other arguments, results and
 * errors as for ds4g_lmhead_sample; DS4G_ERR_INVALID_ARG also for a NaN
 * min_p or a NULL params. */
int ds4g_lmhead_sample_ex(int32_t hidden, int32_t vocab, int32_t wdtype,
                          const void *final_norm, float rms_eps, const void *w_lm,
                          const float *x, const ds4g_sample_params *params,
                          uint64_t *rng_state, float *logits, int32_t *token,
                          const void *embed_table, float *x_next,
                          void *ws, size_t ws_bytes, void *stream);

/* Token embedding (阶段四 4.1): x[t] = widen(table[ids[t]]) for t < T.
 *   table: device [vocab, hidden] in wdtype; ids: device int32 [T];
 *   x: device fp32 [T, hidden] out.  An id outside [0, vocab) yields a row
 *   of zeros (the kernel never reads outside the table).  hidden % 8 == 0. */
int ds4g_embed(int32_t vocab, int32_t hidden, int32_t wdtype, const void *table,
               const int32_t *ids, int32_t T, float *x, void *stream);

/* Calibration of the matrix-core roofline: `blocks` blocks of 4 waves each
 * issue iters x 8 independent bf16 v_mfma_f32_32x32x16 steps on register
 * operands (2*32*32*16 flops each), with no memory traffic but one float per
 * wave written to out (device, blocks*4 floats).  Time it with events on
 * `stream`: flops / time is the rate the chip sustains at its current clocks.
 * DS4G_ERR_INVALID_ARG for a non-positive size or NULL out. */
int ds4g_probe_mfma(int32_t blocks, int32_t iters, float *out, void *stream);

/* ds4g_probe_mfma on random operands: each wave draws 8 A and 8 B operand
 * sets of bf16 values with random signs and mantissas (|v| in [0.5, 1)) from
 * `seed` and its position, and every one of the iters x 64 MFMAs per wave
 * pairs a different A and B set, so the matrix cores switch as in a GEMM on
 * random data.  blocks x 4 waves; out: device, blocks*4 floats.  Errors as
 * for ds4g_probe_mfma. */
int ds4g_probe_mfma_random(int32_t blocks, int32_t iters, uint32_t seed, float *out,
                           void *stream);

/* Calibration of the HBM read rate of an access shape.  src: device buffer
 * of src_bytes (16-byte aligned), read as rows of row_stride bytes (>= 8192,
 * a multiple of 16) of which the first 8192 are read.  read_bytes (a
 * multiple of step_rows * 8192) are read as units of step_rows rows
 * (a power of two in [4, 2048]); each unit in steps of 32 KB that take
 * 32768 / step_rows bytes of every row of the unit, left to right (the walk
 * of an MFMA GEMM over a weight panel; step_rows = 4 with row_stride = 8192
 * is a contiguous stream).  `blocks` blocks of 256 threads split the units
 * into contiguous ranges; out (device, blocks * 256 words) receives an xor of
 * what each thread read.  Time it with events on `stream`.
 * DS4G_ERR_INVALID_ARG for sizes outside these rules or a read that would
 * pass src_bytes. */
int ds4g_probe_read(const void *src, int64_t src_bytes, int32_t step_rows, int64_t row_stride,
                    int64_t read_bytes, int32_t blocks, uint32_t *out, void *stream);

/* Calibration of the cost of a launch: enqueues n_kernels launches of
 * `blocks` blocks on `stream` (capture it in a graph to price graph
 * dispatch).  buf: device, 2 words, ping-ponged.  chained != 0: every thread
 * of launch i reads the word launch i - 1 wrote and one thread writes it plus
 * one (so launch i's loads depend on launch i - 1); otherwise one thread of
 * each launch writes 1.  DS4G_ERR_INVALID_ARG for a non-positive size or
 * NULL buf. */
int ds4g_probe_chain(int32_t blocks, int32_t n_kernels, int32_t chained, uint32_t *buf,
                     void *stream);

/* Static text for a ds4g_status value. */
const char *ds4g_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DS4G_H */
