// The ds4g C ABI (include/ds4g.h): argument checks, workspace layout and the
// launch sequences of prefill, decode and lm_head + sampling.  Host code only;
// every step of the math runs in the kernels of this directory.
#include "../../include/ds4g.h"
#include "kernels.h"
#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>
#include <stdio.h>

namespace ds4g {
namespace {

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// The prefill router GEMM splits K into up to this many parts (partial sums
// added in split order by the top-k kernel).  fp32 weights: K = hidden on the
// vector ALUs; bf16 weights: K = 3 * hidden (the three-term bf16 split of y)
// on the matrix cores.
constexpr int kRouterSplit = 24;
constexpr int kBatchRouterSplit = 12;   // batched decode (<= kRouterSplit)

// GEMMs with 16-bit outputs store them through LDS in 16-byte row chunks
// (GemmArgs::stage16) when their tiles are mostly full: dense GEMMs of at
// least this many rows, grouped expert GEMMs of at least half as many rows
// per expert on average.  A tile with a few rows stores less the direct way.
constexpr int kStageRows = 64;

// Batched decode (a few rows per GEMM): split K so that a dense GEMM runs
// ~256 blocks instead of one per N tile.  A power of two dividing K / 64, at
// most 64; 1 beyond 256 rows or on the fp32-weight path.  The tile shapes
// follow launch_gemm (64 x 256 up to 64 rows, else 128 x 128).
inline int batch_split(int M, int N, int K, bool mfma) {
  if (!mfma || M > 256) return 1;
  const long bm = M <= 64 ? 64 : 128, bn = M <= 64 ? 256 : 128;
  const long tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  int s = 1;
  while (s < 64 && tiles * s * 2 <= 256 && K % (64 * s * 2) == 0) s *= 2;
  return s;
}
inline int router_split(int hidden, bool mfma) {
  if (mfma) {
    // hidden / 1024 slices of K = 3 * hidden (each a multiple of 64); fixed by
    // the shape alone, so a token's logits never depend on the batch size
    const int s = (hidden % 1024 == 0 && hidden / 1024 <= 8) ? hidden / 1024 : 1;
    return s;
  }
  int s = hidden / 512;
  if (s < 1) s = 1;
  if (s > 8) s = 8;
  while (hidden % (16 * s)) --s;
  return s;
}

// The fp16 image buffer: QKV-A, QKV-B and W_o in fp16, then each one's row
// factors; the same carve inside a workspace and in a caller's image buffer.
struct ImageLayout {
  size_t img[3], inv[3], total;
};
ImageLayout image_layout(const ds4g_layer_cfg& c, size_t base) {
  const size_t d = c.hidden, r = c.qkv_rank, qd = (size_t)c.n_heads * c.head_dim,
               qkvd = qd + 2 * (size_t)c.head_dim;
  const size_t n[3] = {r, qkvd, d}, k[3] = {d, r, qd};
  ImageLayout L;
  size_t o = base;
  for (int m = 0; m < 3; ++m) {
    L.img[m] = o; o = a256(o + n[m] * k[m] * 2);
    L.inv[m] = o; o = a256(o + n[m] * 4);
  }
  L.total = o - base;
  return L;
}

struct Layout {
  size_t xn, c, qkv, q, kc, vc, o, yf, ys, logits, lpart, tidx, tw, rank, perm, gather, pos_of,
      count, chunk, offset, tiles, ntiles, z, zs, part, skp, rope, img[3], inv[3], total;
};

// Byte offsets of every workspace buffer for T tokens.  fp32-sized slots are
// used for buffers that hold 16-bit values on the MFMA path and fp32 on the
// SIMT path.  images: the fp16 images of QKV-A, QKV-B and W_o (and their row
// factors) that the attention path's MFMA GEMMs read; prefill and batched
// decode with bf16 weights only (the single-token decode streams the bf16
// weights themselves).
Layout layout(const ds4g_layer_cfg& c, int T, bool images) {
  const size_t d = c.hidden, r = c.qkv_rank, qd = (size_t)c.n_heads * c.head_dim,
               qkvd = qd + 2 * (size_t)c.head_dim, E = c.n_experts, k = c.top_k,
               I = c.ffn_inter, Is = c.shared_inter, dh = c.head_dim;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = a256(o + bytes); return at; };
  L.xn = take((size_t)T * d * 4);
  L.c = take((size_t)T * r * 4);
  L.qkv = take((size_t)T * qkvd * 4);
  L.q = take((size_t)T * qd * 4);
  L.kc = take((size_t)T * dh * 2);
  L.vc = take((size_t)T * dh * 2);
  L.o = take((size_t)T * qd * 4);
  L.yf = take((size_t)T * d * 4);
  L.ys = take((size_t)T * 3 * d * 2);
  L.logits = take((size_t)T * E * 4);
  L.lpart = take((size_t)T * E * 4 * kRouterSplit);
  L.tidx = take((size_t)T * k * 4);
  L.tw = take((size_t)T * k * 4);
  L.rank = take((size_t)T * k * 4);
  L.perm = take((size_t)T * k * 4);
  L.gather = take((size_t)T * k * 4);
  L.pos_of = take((size_t)T * k * 4);
  L.count = take(E * 4);
  L.chunk = take((size_t)((T * k + kRankChunk - 1) / kRankChunk) * E * 4);
  L.offset = take((E + 1) * 4);
  L.tiles = take((E + (size_t)T * k + 1) * 4);
  L.ntiles = take(4);
  L.z = take(((size_t)T * k * I + I + Is) * 4);
  L.zs = take((size_t)T * Is * 4);
  L.part = take((size_t)T * k * d * 4);
  {   // split-K partial sums of the batched decode's dense GEMMs
    const bool mfma = c.wdtype == DS4G_BF16;
    size_t m = 0;
    auto need = [&](int N, int K, int parts) {
      m = std::max(m, (size_t)batch_split(T, N, K, mfma) * T * N * 4 * parts);
    };
    need(r, d, 1); need((int)qkvd, r, 1); need(d, (int)qd, 1); need(Is, d, 2); need(d, Is, 1);
    L.skp = take(T <= 256 ? m : 0);
  }
  L.rope = take((size_t)dh * (((size_t)T + 3) & ~(size_t)3) * 4);   // cos, sin [rd/2][T pad 4]
  if (images && c.wdtype == DS4G_BF16) {
    const ImageLayout IL = image_layout(c, o);
    for (int m = 0; m < 3; ++m) { L.img[m] = IL.img[m]; L.inv[m] = IL.inv[m]; }
    o += IL.total;
  } else {
    for (int m = 0; m < 3; ++m) L.img[m] = L.inv[m] = o;
  }
  L.total = o;
  return L;
}

int check_cfg(const ds4g_layer_cfg* c) {
  if (!c) return DS4G_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->qkv_rank <= 0 ||
      c->window <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->ffn_inter <= 0 ||
      c->shared_inter <= 0 || c->rope_dim < 0 || !(c->rms_eps >= 0.f) || !(c->rope_base > 0.f))
    return DS4G_ERR_INVALID_ARG;
  if (c->wdtype != DS4G_F32 && c->wdtype != DS4G_BF16) return DS4G_ERR_INVALID_ARG;
  if (c->top_k >= c->n_experts) return DS4G_ERR_INVALID_ARG;
  const int rd = c->rope_dim ? c->rope_dim : c->head_dim;
  if (rd > c->head_dim || (rd & 1)) return DS4G_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return DS4G_ERR_UNSUPPORTED;
  if (c->window > 128 || c->n_experts > 512 || c->top_k > 8 || c->n_heads % 4)
    return DS4G_ERR_UNSUPPORTED;
  if (c->hidden % 64 || c->qkv_rank % 64 || c->ffn_inter % 64 || c->shared_inter % 64 ||
      (c->n_heads * c->head_dim) % 64)
    return DS4G_ERR_UNSUPPORTED;
  if (c->hidden > 16384 || c->qkv_rank > 16384 || c->n_heads * c->head_dim > 16384 ||
      c->ffn_inter > 2048 || c->shared_inter > 2048)
    return DS4G_ERR_UNSUPPORTED;
  if ((long)c->top_k * c->ffn_inter + c->shared_inter > 12288) return DS4G_ERR_UNSUPPORTED;
  return DS4G_OK;
}

int check_weights(const ds4g_layer_weights* w) {
  if (!w || !w->attn_norm || !w->qkv_a || !w->qkv_b || !w->wo || !w->ffn_norm || !w->router ||
      !w->gate || !w->up || !w->down || !w->sh_gate || !w->sh_up || !w->sh_down)
    return DS4G_ERR_INVALID_ARG;
  return DS4G_OK;
}

int check_ring(const ds4g_kv_ring* r) {
  if (!r || !r->k || !r->v || !r->pos) return DS4G_ERR_INVALID_ARG;
  return DS4G_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Status of a real (non-dry) launch sequence.  Its dry run accepted the same
// arguments, so a launcher cannot refuse here; a refusal would be a bug and
// is reported as a launch failure.
int hip_status(int launch_rc) {
  if (launch_rc != 0) return DS4G_ERR_HIP;
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return DS4G_OK;
  fprintf(stderr, "ds4g: HIP launch error: %s\n", hipGetErrorString(e));
  return DS4G_ERR_HIP;
}

// Clear an error left by an earlier, unrelated HIP call so that the check at
// the end of a call reports only this call's launches.
void clear_stale_error() { (void)hipGetLastError(); }

// copy an optional routing output
void copy_out(void* dst, const void* src, size_t bytes, Exec st) {
  if (dst && bytes && !st.dry)
    (void)hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st.stream);
}

// Run a call's launch sequence dry (every launcher checks its preconditions,
// nothing is enqueued), then for real.  A shape that any launcher refuses is
// reported as DS4G_ERR_UNSUPPORTED before the first kernel is enqueued.
template <typename F>
int dry_then_run(hipStream_t stream, F&& seq) {
  if (seq(Exec{stream, true}) != 0) return DS4G_ERR_UNSUPPORTED;
  clear_stale_error();
  return hip_status(seq(Exec{stream, false}));
}

// ------------------------------------------------------------------ prefill
// A second stream per device, for the shared expert: it needs only y, so it
// runs beside the router, the routing and the routed experts, and the
// combine waits for it.  Created on the first prefill on each device (never
// while the caller's stream is being captured into a graph); nullptr if HIP
// refuses, and then the shared expert runs on the caller's stream.  Default
// priority, non-blocking; the fork and join events are reused by every call,
// so enqueueing from the fork to the join holds side_mutex().
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
};
std::mutex& side_mutex() {
  static std::mutex mu;
  return mu;
}
SideStream* side_stream(hipStream_t main) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static SideStream ss[kMaxDevices] = {};
  static bool tried[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!tried[dev]) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return nullptr;
    tried[dev] = true;
    SideStream t{};
    if (hipStreamCreateWithFlags(&t.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&t.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&t.join, hipEventDisableTiming) != hipSuccess) {
      fprintf(stderr, "ds4g: no events for the shared-expert stream; it runs inline\n");
      return nullptr;
    }
    ss[dev] = t;
  }
  return ss[dev].s ? &ss[dev] : nullptr;
}

// Layer-major prefill of T tokens of one sequence, or (batch) one decode
// token of each of T independent sequences: the same GEMMs, router and
// experts over T rows; only the attention stage differs.
int prefill_impl(const ds4g_layer_cfg& c, const ds4g_layer_weights& w, ds4g_kv_ring& ring,
                 float* x, int T, ds4g_routing* routing, void* ws, Exec st,
                 bool batch = false, const ds4g_trace* trace = nullptr) {
  const Layout L = layout(c, T, true);
  const bool bf = c.wdtype == DS4G_BF16;
  const int d = c.hidden, r = c.qkv_rank, H = c.n_heads, dh = c.head_dim, qd = H * dh,
            qkvd = qd + 2 * dh, E = c.n_experts, k = c.top_k, I = c.ffn_inter,
            Is = c.shared_inter;
  const int rd = c.rope_dim ? c.rope_dim : dh;
  int rc = 0;
  Exec cur = st;   // the stream the dense GEMMs below go to

  // x_norm = RMSNorm(h) * g1.  bf16 weights: the attention path (x_norm, c,
  // q, k, v, probabilities, o) runs in fp16 on the matrix cores; fp32
  // weights: fp32 on the vector ALUs.
  if (bf)
    rc |= launch_rmsnorm_rows<uint16_t>(x, T, d, (const uint16_t*)w.attn_norm, c.rms_eps, nullptr,
                                        nullptr, at<uint16_t>(ws, L.xn), nullptr, st);
  else
    rc |= launch_rmsnorm_rows<float>(x, T, d, (const float*)w.attn_norm, c.rms_eps,
                                     at<float>(ws, L.xn), nullptr, nullptr, nullptr, st);

  // fp16 images of the attention path's weights (QKV-A, QKV-B, W_o), each
  // made right before the first GEMM that reads it
  const void* const wsrc[3] = {w.qkv_a, w.qkv_b, w.wo};
  const int wN[3] = {r, qkvd, d}, wK[3] = {d, r, qd};
  // (or read from the caller's prepared images, w.f16_images)
  bool made[3] = {false, false, false};
  void* ibase = w.f16_images ? const_cast<void*>(w.f16_images) : ws;
  size_t img_off[3], inv_off[3];
  if (w.f16_images) {
    const ImageLayout IL = image_layout(c, 0);
    for (int m = 0; m < 3; ++m) { img_off[m] = IL.img[m]; inv_off[m] = IL.inv[m]; }
  } else {
    for (int m = 0; m < 3; ++m) { img_off[m] = L.img[m]; inv_off[m] = L.inv[m]; }
  }
  auto image = [&](int m) {
    if (!made[m] && !w.f16_images)
      rc |= launch_f16_image(static_cast<const uint16_t*>(wsrc[m]), wN[m], wK[m],
                             at<uint16_t>(ws, L.img[m]), at<float>(ws, L.inv[m]), st);
    made[m] = true;
  };

  // dense GEMM; batched decode splits K (fp32 partials, then a reduce that
  // applies the epilogue).  B2: the up projection of a SwiGLU pair.  img >= 0:
  // A is fp16 and B is attention-path weight img, read from its fp16 image
  // (the multi-row GEMV reads the bf16 weights directly).
  auto gemm = [&](const void* A, int lda, const void* B, int M, int N, int K, int epi, void* C,
                  int ldc, const void* B2 = nullptr, int img = -1) {
    if (batch && bf && M <= 8) {   // a few rows: stream each weight row once (multi-row GEMV)
      GemvRowsArgs v{};
      v.W = static_cast<const uint16_t*>(B); v.W2 = static_cast<const uint16_t*>(B2);
      v.N = N; v.K = K; v.X = static_cast<const uint16_t*>(A); v.x_f16 = img >= 0 ? 1 : 0;
      v.lda = lda; v.M = M; v.epi = epi; v.C = C; v.ldc = ldc;
      if (launch_gemv_rows(v, cur) == 0) return;
    }
    const float* cs = nullptr;
    if (bf && img >= 0) {
      image(img);
      B = at<void>(ibase, img_off[img]);
      cs = at<float>(ibase, inv_off[img]);
    }
    const int s = batch ? batch_split(M, N, K, bf) : 1;
    if (s > 1) {
      float* part = at<float>(ws, L.skp);
      const long ps = (long)M * N;
      GemmArgs g{};
      g.A = A; g.lda = lda; g.M = M; g.N = N; g.K = K; g.epi = EPI_F32; g.ldc = N;
      g.ksplit = s; g.part_stride = ps; g.f16 = img >= 0 ? 1 : 0;
      g.B = B; g.C = part;
      rc |= launch_gemm(g, bf, 1, cur);
      if (B2) {
        g.B = B2; g.C = part + (size_t)s * ps;
        rc |= launch_gemm(g, bf, 1, cur);
      }
      rc |= launch_splitk_reduce(part, B2 ? part + (size_t)s * ps : nullptr, s, ps, M, N, epi, C,
                                 ldc, cs, cur);
      return;
    }
    GemmArgs g{};
    g.A = A; g.lda = lda; g.B = B; g.B2 = B2; g.M = M; g.N = N; g.K = K; g.epi = epi; g.C = C;
    g.ldc = ldc; g.f16 = (bf && img >= 0) ? 1 : 0; g.colscale = cs;
    g.stage16 = M >= kStageRows;
    rc |= launch_gemm(g, bf, bf ? 1 : 0, cur);
  };
  // c = A x ; qkv = B c (prefill on the matrix cores: RoPE in the epilogue,
  // q / k / v written rotated in fp16, as attention reads them)
  gemm(at<void>(ws, L.xn), d, w.qkv_a, T, r, d, bf ? EPI_F16 : EPI_F32, at<void>(ws, L.c), r,
       nullptr, 0);
  const bool rope_epi = bf && !batch;
  const int tpad = (T + 3) & ~3;
  if (rope_epi) {
    float* rc_tab = at<float>(ws, L.rope);
    rc |= launch_rope_table(ring.pos, T, tpad, rd, c.rope_base, rc_tab, rc_tab + (size_t)(rd / 2) * tpad,
                            st);
    image(1);
    GemmArgs g{};
    g.A = at<void>(ws, L.c); g.lda = r; g.B = at<void>(ibase, img_off[1]); g.M = T; g.N = qkvd;
    g.K = r; g.f16 = 1; g.colscale = at<float>(ibase, inv_off[1]);
    g.epi = EPI_ROPE_QKV; g.C = at<void>(ws, L.q); g.ldc = qd;
    g.rope_c = rc_tab; g.rope_s = rc_tab + (size_t)(rd / 2) * tpad; g.rope_ld = tpad;
    g.rope_dh = dh; g.rope_rd = rd;
    g.rope_kc = at<uint16_t>(ws, L.kc); g.rope_vc = at<uint16_t>(ws, L.vc);
    g.stage16 = T >= kStageRows;
    rc |= launch_gemm(g, true, 1, st);
  } else {
    gemm(at<void>(ws, L.c), r, w.qkv_b, T, qkvd, r, EPI_F32, at<void>(ws, L.qkv), qkvd, nullptr,
         1);
  }

  // RoPE, attention over the window, ring update (*pos += T)
  AttnArgs aa{};
  aa.qkv = at<float>(ws, L.qkv); aa.T = T; aa.H = H; aa.dh = dh; aa.rd = rd; aa.W = c.window;
  aa.base = c.rope_base; aa.pos = ring.pos; aa.q = at<void>(ws, L.q); aa.q_f16 = bf ? 1 : 0;
  aa.kc = at<uint16_t>(ws, L.kc); aa.vc = at<uint16_t>(ws, L.vc);
  aa.ring_k = (uint16_t*)ring.k; aa.ring_v = (uint16_t*)ring.v;
  aa.o = at<void>(ws, L.o); aa.o_f16 = bf ? 1 : 0; aa.heads_per_block = H < 64 ? H : 64;
  aa.rope_done = rope_epi ? 1 : 0;
  if (batch)   // RoPE at each sequence's position, its own ring, *pos[b] += 1
    rc |= launch_attention_decode_batch(aa, T, st);
  else
    rc |= bf ? launch_attention_prefill_mfma(aa, st) : launch_attention(aa, st);

  // h2 = h + W_o o   (in place in x)
  gemm(at<void>(ws, L.o), qd, w.wo, T, d, qd, EPI_RESID, x, d, nullptr, 2);
  if (trace) {   // the attention path's buffers are intact until the next call
    const size_t ae = bf ? 2 : 4;   // activation element size
    copy_out(trace->x_norm, at<void>(ws, L.xn), (size_t)T * d * ae, st);
    copy_out(trace->c, at<void>(ws, L.c), (size_t)T * r * ae, st);
    copy_out(trace->q, at<void>(ws, L.q), (size_t)T * qd * ae, st);
    copy_out(trace->k, at<void>(ws, L.kc), (size_t)T * dh * 2, st);
    copy_out(trace->v, at<void>(ws, L.vc), (size_t)T * dh * 2, st);
    copy_out(trace->o, at<void>(ws, L.o), (size_t)T * qd * ae, st);
    copy_out(trace->h2, x, (size_t)T * d * 4, st);
  }

  // y = RMSNorm(h2) * g2: fp32, and (bf16 weights) its three-term bf16 split,
  // whose first term is bf16(y), the expert GEMMs' input
  if (bf)   // fp32 y only when the caller asks for the router input
    rc |= launch_rmsnorm_rows<uint16_t>(x, T, d, (const uint16_t*)w.ffn_norm, c.rms_eps,
                                        (routing && routing->router_in) ? at<float>(ws, L.yf)
                                                                        : nullptr,
                                        nullptr, nullptr, at<uint16_t>(ws, L.ys), st);
  else
    rc |= launch_rmsnorm_rows<float>(x, T, d, (const float*)w.ffn_norm, c.rms_eps,
                                     at<float>(ws, L.yf), nullptr, nullptr, nullptr, st);

  // the shared expert, x = h2 + D_sh(silu(G_sh y) * (U_sh y)), on the side
  // stream when there is one (nothing on this stream touches x until the
  // combine, which waits for it)
  const void* yA = bf ? at<void>(ws, L.ys) : at<void>(ws, L.yf);
  const int ylda = bf ? 3 * d : d;
  // (a few rows: the fork and join cost more than the overlap gives)
  SideStream* side = (st.dry || T < 32) ? nullptr : side_stream(st.stream);
  std::unique_lock<std::mutex> side_lock(side_mutex(), std::defer_lock);
  if (side) {
    side_lock.lock();
    if (hipEventRecord(side->fork, st.stream) == hipSuccess &&
        hipStreamWaitEvent(side->s, side->fork, 0) == hipSuccess) {
      cur = Exec{side->s, false};
    } else {   // no fork: the shared expert runs on the caller's stream
      side = nullptr;
      side_lock.unlock();
    }
  }
  gemm(yA, ylda, w.sh_gate, T, Is, d, bf ? EPI_SWIGLU_BF16 : EPI_SWIGLU_F32, at<void>(ws, L.zs),
       Is, w.sh_up);
  gemm(at<void>(ws, L.zs), Is, w.sh_down, T, d, Is, EPI_RESID, x, d);
  if (side && hipEventRecord(side->join, side->s) != hipSuccess) {
    // no join event: wait for the side stream here instead
    if (hipStreamSynchronize(side->s) != hipSuccess) rc |= -1;
    side_lock.unlock();
    side = nullptr;
  }
  cur = st;

  // router logits at fp32 quality (they decide integer expert choices):
  // bf16 weights: y1|y2|y3 against [W_r|W_r|W_r] on the matrix cores; fp32
  // weights: fp32 y on the vector ALUs.  Split-K partial sums, added in split
  // order by the top-k kernel.
  // batched decode: more slices for more blocks (a function of the shape)
  const int rsplit = (batch && bf && (3 * d) % (64 * kBatchRouterSplit) == 0)
                         ? kBatchRouterSplit
                         : router_split(d, bf);
  {
    GemmArgs g{};
    g.M = T; g.N = E; g.epi = EPI_F32; g.C = at<void>(ws, L.lpart); g.ldc = E;
    g.ksplit = rsplit; g.part_stride = (long)T * E;
    if (bf) {
      // y1|y2|y3 against W_r repeated three times along K (read in place)
      g.A = at<void>(ws, L.ys); g.lda = 3 * d; g.B = w.router; g.brep = d; g.K = 3 * d;
    } else {
      g.A = at<void>(ws, L.yf); g.lda = d; g.B = w.router; g.K = d;
    }
    rc |= launch_gemm(g, bf, bf ? 1 : 0, st);
  }
  // tile height of the grouped expert GEMMs: follow the mean rows per expert
  const int mean_rows = (T * k + E - 1) / E;
#ifndef DS4G_TILE_M_MAX   // cap on the expert tile height (128: measured 3% slower at 16994)
#define DS4G_TILE_M_MAX 256
#endif
#ifndef DS4G_DOWN_XCD_REMAP_MIN   // routed down tiles in the per-XCD order from this tile height
#define DS4G_DOWN_XCD_REMAP_MIN 256
#endif
  const int tile_m = std::min((!bf || mean_rows <= 64) ? 64 : mean_rows < 160 ? 128 : 256,
                              DS4G_TILE_M_MAX);
  RouteArgs ra{};
  ra.logits = at<float>(ws, L.lpart); ra.nsplit = rsplit;
  // the summed logits only when the caller asked for them
  ra.logits_sum = (routing && routing->router_logits) ? at<float>(ws, L.logits) : nullptr;
  ra.T = T; ra.E = E; ra.k = k;
  ra.topk_idx = at<int>(ws, L.tidx); ra.topk_w = at<float>(ws, L.tw);
  ra.count = at<int>(ws, L.count); ra.offset = at<int>(ws, L.offset);
  ra.rank = at<int>(ws, L.rank); ra.perm = at<int>(ws, L.perm);
  ra.chunk = at<int>(ws, L.chunk);
  ra.gather = at<int>(ws, L.gather); ra.pos_of = at<int>(ws, L.pos_of);
  ra.tiles = at<int>(ws, L.tiles); ra.ntiles = at<int>(ws, L.ntiles); ra.tile_m = tile_m;
  ra.out_count = routing ? routing->expert_count : nullptr;
  ra.out_offset = routing ? routing->expert_offset : nullptr;
  rc |= launch_route(ra, st);
  const int max_tiles = E + (T * k + tile_m - 1) / tile_m;

  // routed gate/up + SwiGLU over the permuted rows
  {
    GemmArgs g{};
    g.A = yA; g.lda = ylda; g.gather = ra.gather; g.B = w.gate; g.B2 = w.up;
    g.b_stride = (long)I * d; g.N = I; g.K = d; g.tiles = ra.tiles; g.ntiles = ra.ntiles;
    g.row_off = ra.offset; g.max_tiles = max_tiles; g.rows_hint = tile_m;
    g.epi = bf ? EPI_SWIGLU_BF16 : EPI_SWIGLU_F32; g.C = at<void>(ws, L.z); g.ldc = I;
    g.xcd_remap = 1;
    g.stage16 = mean_rows >= kStageRows / 2;
    rc |= launch_gemm(g, bf, bf ? 1 : 0, st);
  }
  // routed down projections -> part (permuted rows; bf16 on the MFMA path,
  // fp32 on the fp32-weight path), combined in fp32 below
  {
    GemmArgs g{};
    g.A = at<void>(ws, L.z); g.lda = I; g.B = w.down; g.b_stride = (long)d * I; g.N = d;
    g.K = I; g.tiles = ra.tiles; g.ntiles = ra.ntiles; g.row_off = ra.offset;
    g.max_tiles = max_tiles; g.rows_hint = tile_m; g.epi = bf ? EPI_BF16 : EPI_F32;
    g.C = at<void>(ws, L.part);
    g.ldc = d;
    g.xcd_remap = tile_m >= DS4G_DOWN_XCD_REMAP_MIN;   // 1.1% at 16994 tokens, 0.5% slower at 2048
    g.stage16 = mean_rows >= kStageRows / 2;
    rc |= launch_gemm(g, bf, bf ? 1 : 0, st);
  }
  // combine, x += sum_j w_j part_j, once the shared expert is in x
  if (side) {
    if (hipStreamWaitEvent(st.stream, side->join, 0) != hipSuccess &&
        hipStreamSynchronize(side->s) != hipSuccess)
      rc |= -1;
    side_lock.unlock();
  }
  // batched decode: the combine also advances each sequence's position (the
  // attention kernel read it; nothing after the combine does)
  rc |= launch_moe_combine(x, at<void>(ws, L.part), bf ? 1 : 0, ra.pos_of, ra.topk_w, T, d, k,
                           batch ? ring.pos : nullptr, st);
  if (routing) {
    copy_out(routing->topk_idx, ra.topk_idx, (size_t)T * k * 4, st);
    copy_out(routing->topk_w, ra.topk_w, (size_t)T * k * 4, st);
    copy_out(routing->perm, ra.perm, (size_t)T * k * 4, st);
    copy_out(routing->router_in, at<void>(ws, L.yf), (size_t)T * d * 4, st);
    if (ra.logits_sum) copy_out(routing->router_logits, ra.logits_sum, (size_t)T * E * 4, st);
  }
  return rc;
}

// ------------------------------------------------------------------ decode
template <typename WT>
int decode_impl(const ds4g_layer_cfg& c, const ds4g_layer_weights& w, ds4g_kv_ring& ring,
                float* x, ds4g_routing* routing, void* ws, Exec st) {
  const Layout L = layout(c, 1, false);
  const int d = c.hidden, r = c.qkv_rank, H = c.n_heads, dh = c.head_dim, qd = H * dh,
            qkvd = qd + 2 * dh, E = c.n_experts;
  const int rd = c.rope_dim ? c.rope_dim : dh;
  int rc = 0;
  float* cbuf = at<float>(ws, L.c);
  float* qkv = at<float>(ws, L.qkv);
  float* logits = at<float>(ws, L.logits);
  // c = A RMSNorm(h) g1
  {
    GemvArgs g{};
    g.W = w.qkv_a; g.N = r; g.K = d; g.x = x; g.gamma = w.attn_norm; g.eps = c.rms_eps;
    g.out = cbuf;
    rc |= launch_gemv<WT>(g, st);
  }
  // [q | k | v] = B c
  {
    GemvArgs g{};
    g.W = w.qkv_b; g.N = qkvd; g.K = r; g.x = cbuf; g.out = qkv;
    rc |= launch_gemv<WT>(g, st);
  }
  // RoPE, ring slot write, windowed MQA
  AttnArgs aa{};
  aa.qkv = qkv; aa.T = 1; aa.H = H; aa.dh = dh; aa.rd = rd; aa.W = c.window;
  aa.base = c.rope_base; aa.pos = ring.pos; aa.ring_k = (uint16_t*)ring.k;
  aa.ring_v = (uint16_t*)ring.v; aa.o = at<void>(ws, L.o);
  rc |= launch_attention_decode(aa, st);
  // h2 = h + W_o o
  {
    GemvArgs g{};
    g.W = w.wo; g.N = d; g.K = qd; g.x = at<float>(ws, L.o); g.out = x; g.accumulate = 1;
    rc |= launch_gemv<WT>(g, st);
  }
  // router logits and the shared expert on y = RMSNorm(h2) g2, routed
  // experts, combine + residual
  MoeDecodeArgs m{};
  m.h2 = x; m.ffn_norm = w.ffn_norm; m.eps = c.rms_eps; m.router = w.router;
  m.logits_out = logits; m.logits = logits; m.E = E;
  m.k = c.top_k; m.d = d; m.I = c.ffn_inter; m.Is = c.shared_inter; m.gate = w.gate;
  m.up = w.up; m.down = w.down; m.sh_gate = w.sh_gate; m.sh_up = w.sh_up;
  m.sh_down = w.sh_down; m.z = at<float>(ws, L.z);
  m.sel = at<int>(ws, L.tidx); m.wsel = at<float>(ws, L.tw);
  if (routing) {
    m.topk_idx = routing->topk_idx; m.topk_w = routing->topk_w;
    m.count = routing->expert_count; m.offset = routing->expert_offset;
    m.perm = routing->perm; m.router_in = routing->router_in;
  }
  rc |= launch_moe_decode<WT>(m, x, ring.pos, st);
  if (routing) copy_out(routing->router_logits, logits, (size_t)E * 4, st);
  return rc;
}

// Row-count limits of a layer call (T tokens, or T sequences of a batched
// decode).  The MFMA GEMMs address their 16-bit operands with 32-bit byte
// offsets: no operand may reach 4 GiB.
int check_rows(const ds4g_layer_cfg& c, int T, int mode) {
  if (mode == DS4G_MODE_DECODE) return T == 1 ? DS4G_OK : DS4G_ERR_INVALID_ARG;
  if (mode == DS4G_MODE_DECODE_BATCH && T > 65535) return DS4G_ERR_UNSUPPORTED;
  if ((long)T * c.top_k >= (1 << 24) || T > (1 << 20)) return DS4G_ERR_UNSUPPORTED;
  if (c.wdtype == DS4G_BF16) {
    const double widest = std::max({3.0 * c.hidden, (double)c.n_heads * c.head_dim,
                                    (double)c.qkv_rank, (double)c.shared_inter,
                                    (double)c.top_k * c.ffn_inter});
    if ((double)T * widest * 2.0 >= 4294967296.0) return DS4G_ERR_UNSUPPORTED;
  }
  return DS4G_OK;
}

// Every host-side check of a layer call, in order: dimensions, pointers,
// workspace alignment, row limits, workspace size.
int check_call(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w, const ds4g_kv_ring* ring,
               const float* x, int T, const void* ws, size_t ws_bytes, int mode) {
  int s = check_cfg(cfg);
  if (s != DS4G_OK) return s;
  if ((s = check_weights(w)) != DS4G_OK) return s;
  if ((s = check_ring(ring)) != DS4G_OK) return s;
  if (!x || !ws || T <= 0) return DS4G_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return DS4G_ERR_INVALID_ARG;
  if (w->f16_images && (reinterpret_cast<uintptr_t>(w->f16_images) & 255) != 0)
    return DS4G_ERR_INVALID_ARG;
  if ((s = check_rows(*cfg, T, mode)) != DS4G_OK) return s;
  const bool images = mode != DS4G_MODE_DECODE && !w->f16_images;
  if (ws_bytes < layout(*cfg, T, images).total) return DS4G_ERR_WORKSPACE;
  return DS4G_OK;
}

// The launch sequence of a layer call of the given mode.
int layer_seq(const ds4g_layer_cfg& c, const ds4g_layer_weights& w, ds4g_kv_ring& ring, float* x,
              int T, ds4g_routing* routing, void* ws, Exec ex, int mode) {
  if (mode == DS4G_MODE_DECODE)
    return c.wdtype == DS4G_BF16 ? decode_impl<uint16_t>(c, w, ring, x, routing, ws, ex)
                                 : decode_impl<float>(c, w, ring, x, routing, ws, ex);
  return prefill_impl(c, w, ring, x, T, routing, ws, ex, mode == DS4G_MODE_DECODE_BATCH);
}

// Scratch of ds4g_layer_decode_noalloc: a file-scope device array, one copy
// per GPU at that GPU's own address, kept until the process ends.  Its name
// on the host is only a stand-in: kernels get the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoallocScratchBytes = size_t(2) << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of `scratch` on the current device, looked up on the first
// call on each device (with that device current) and kept; nullptr if HIP
// refuses.
void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fprintf(stderr, "ds4g: hipGetSymbolAddress(scratch) failed: %s\n", hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace
}  // namespace ds4g

using namespace ds4g;

extern "C" {

size_t ds4g_workspace_bytes(const ds4g_layer_cfg* cfg, int32_t max_tokens, int32_t vocab) {
  size_t n = 0;
  if (cfg) {
    if (check_cfg(cfg) != DS4G_OK || max_tokens <= 0) return 0;
    n = layout(*cfg, max_tokens, true).total;
  }
  if (vocab > 0) {
    const size_t s = sample_ws_bytes(vocab);
    if (s > n) n = s;
  } else if (vocab < 0) {
    return 0;
  }
  return n;
}

int ds4g_layer_prefill(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w,
                       ds4g_kv_ring* ring, float* x, int32_t T, ds4g_routing* routing, void* ws,
                       size_t ws_bytes, void* stream) {
  int s = check_call(cfg, w, ring, x, T, ws, ws_bytes, DS4G_MODE_PREFILL);
  if (s != DS4G_OK) return s;
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    return prefill_impl(*cfg, *w, *ring, x, T, routing, ws, ex);
  });
}

int ds4g_layer_prefill_trace(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w,
                             ds4g_kv_ring* ring, float* x, int32_t T, ds4g_routing* routing,
                             const ds4g_trace* trace, void* ws, size_t ws_bytes, void* stream) {
  int s = check_call(cfg, w, ring, x, T, ws, ws_bytes, DS4G_MODE_PREFILL);
  if (s != DS4G_OK) return s;
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    return prefill_impl(*cfg, *w, *ring, x, T, routing, ws, ex, false, trace);
  });
}

int ds4g_layer_decode_batch(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w,
                            ds4g_kv_ring* rings, float* x, int32_t B, ds4g_routing* routing,
                            void* ws, size_t ws_bytes, void* stream) {
  int s = check_call(cfg, w, rings, x, B, ws, ws_bytes, DS4G_MODE_DECODE_BATCH);
  if (s != DS4G_OK) return s;
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    return prefill_impl(*cfg, *w, *rings, x, B, routing, ws, ex, true);
  });
}

int ds4g_layer_decode(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w, ds4g_kv_ring* ring,
                      float* x, ds4g_routing* routing, void* ws, size_t ws_bytes, void* stream) {
  int s = check_call(cfg, w, ring, x, 1, ws, ws_bytes, DS4G_MODE_DECODE);
  if (s != DS4G_OK) return s;
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    return layer_seq(*cfg, *w, *ring, x, 1, routing, ws, ex, DS4G_MODE_DECODE);
  });
}

int ds4g_layer_decode_noalloc(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w,
                              ds4g_kv_ring* ring, float* x, ds4g_routing* routing, void* stream) {
  // every check, and the dry launch sequence, before the device is touched
  // (a placeholder stands for the scratch address until then)
  void* const placeholder = reinterpret_cast<void*>(uintptr_t(1) << 40);
  const int s = check_call(cfg, w, ring, x, 1, placeholder, kNoallocScratchBytes,
                           DS4G_MODE_DECODE);
  if (s == DS4G_ERR_WORKSPACE)
    fprintf(stderr, "ds4g_layer_decode_noalloc: the layer needs %zu bytes of scratch, the "
            "library holds %zu\n", layout(*cfg, 1, false).total, kNoallocScratchBytes);
  if (s != DS4G_OK) return s;
  if (layer_seq(*cfg, *w, *ring, x, 1, routing, placeholder, Exec{(hipStream_t)stream, true},
                DS4G_MODE_DECODE) != 0)
    return DS4G_ERR_UNSUPPORTED;
  void* ws = scratch_ptr();
  if (!ws) return DS4G_ERR_HIP;
  clear_stale_error();
  return hip_status(layer_seq(*cfg, *w, *ring, x, 1, routing, ws,
                              Exec{(hipStream_t)stream, false}, DS4G_MODE_DECODE));
}

size_t ds4g_f16_images_bytes(const ds4g_layer_cfg* cfg) {
  if (check_cfg(cfg) != DS4G_OK || cfg->wdtype != DS4G_BF16) return 0;
  return image_layout(*cfg, 0).total;
}

int ds4g_make_f16_images(const ds4g_layer_cfg* cfg, const ds4g_layer_weights* w, void* images,
                         size_t images_bytes, void* stream) {
  int s = check_cfg(cfg);
  if (s != DS4G_OK) return s;
  if ((s = check_weights(w)) != DS4G_OK) return s;
  if (cfg->wdtype != DS4G_BF16) return DS4G_ERR_UNSUPPORTED;
  if (!images || (reinterpret_cast<uintptr_t>(images) & 255) != 0) return DS4G_ERR_INVALID_ARG;
  const ImageLayout IL = image_layout(*cfg, 0);
  if (images_bytes < IL.total) return DS4G_ERR_WORKSPACE;
  const int d = cfg->hidden, r = cfg->qkv_rank, qd = cfg->n_heads * cfg->head_dim,
            qkvd = qd + 2 * cfg->head_dim;
  const void* const src[3] = {w->qkv_a, w->qkv_b, w->wo};
  const int N[3] = {r, qkvd, d}, K[3] = {d, r, qd};
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    int rc = 0;
    for (int m = 0; m < 3; ++m)
      rc |= launch_f16_image(static_cast<const uint16_t*>(src[m]), N[m], K[m],
                             at<uint16_t>(images, IL.img[m]), at<float>(images, IL.inv[m]), ex);
    return rc;
  });
}

int ds4g_layer_supported(const ds4g_layer_cfg* cfg, int32_t T, int32_t mode) {
  int s = check_cfg(cfg);
  if (s != DS4G_OK) return s;
  if (mode != DS4G_MODE_PREFILL && mode != DS4G_MODE_DECODE && mode != DS4G_MODE_DECODE_BATCH)
    return DS4G_ERR_INVALID_ARG;
  if (T <= 0 || (mode == DS4G_MODE_DECODE && T != 1)) return DS4G_ERR_INVALID_ARG;
  if ((s = check_rows(*cfg, T, mode)) != DS4G_OK) return s;
  // the launch sequence, dry, over placeholder addresses (never dereferenced)
  void* const p = reinterpret_cast<void*>(uintptr_t(1) << 40);
  ds4g_layer_weights w{p, p, p, p, p, p, p, p, p, p, p, p, nullptr};
  ds4g_kv_ring ring{p, p, static_cast<int64_t*>(p)};
  return layer_seq(*cfg, w, ring, static_cast<float*>(p), T, nullptr, p, Exec{nullptr, true}, mode)
             ? DS4G_ERR_UNSUPPORTED
             : DS4G_OK;
}

int ds4g_lmhead_sample_ex(int32_t hidden, int32_t vocab, int32_t wdtype, const void* final_norm,
                          float rms_eps, const void* w_lm, const float* x,
                          const ds4g_sample_params* params, uint64_t* rng_state, float* logits,
                          int32_t* token, const void* embed_table, float* x_next, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!params) return DS4G_ERR_INVALID_ARG;
  const float temperature = params->temperature, top_p = params->top_p, min_p = params->min_p;
  if (hidden <= 0 || vocab <= 0 || !w_lm || !x || !logits || !token || !ws)
    return DS4G_ERR_INVALID_ARG;
  if ((embed_table == nullptr) != (x_next == nullptr)) return DS4G_ERR_INVALID_ARG;
  if (wdtype != DS4G_F32 && wdtype != DS4G_BF16) return DS4G_ERR_INVALID_ARG;
  if (!(rms_eps >= 0.f) || temperature != temperature || top_p != top_p || min_p != min_p)
    return DS4G_ERR_INVALID_ARG;
  if ((temperature > 0.f || params->temperature_dev) && !rng_state) return DS4G_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return DS4G_ERR_INVALID_ARG;
  if (hidden % 8 || hidden > 16384 || vocab > (1 << 18)) return DS4G_ERR_UNSUPPORTED;
  if (ws_bytes < sample_ws_bytes(vocab)) return DS4G_ERR_WORKSPACE;
  return dry_then_run((hipStream_t)stream, [&](Exec st) {
  int rc = 0;
  // the GEMV also leaves its blocks' largest logits for the sampler and
  // clears the sampler's histogram and arrival count
  const SampleScratch sc = sample_scratch(ws, vocab);
  {
    GemvArgs g{};
    g.W = w_lm; g.N = vocab; g.K = hidden; g.x = x; g.gamma = final_norm; g.eps = rms_eps;
    g.out = logits;
    g.blockmax = sc.bmax; g.blockarg = sc.barg; g.zero = sc.zero; g.zero_words = sc.zero_words;
    rc |= (wdtype == DS4G_BF16) ? launch_gemv<uint16_t>(g, st) : launch_gemv<float>(g, st);
  }
  SampleArgs sa{};
  sa.logits = logits; sa.V = vocab; sa.temperature = temperature; sa.top_p = top_p;
  sa.min_p = min_p; sa.temperature_dev = params->temperature_dev;
  sa.rng = rng_state; sa.token = token; sa.ws = ws;
  sa.nbm = gemv_grid(vocab, hidden);
  rc |= launch_sample(sa, st);
  if (embed_table)
    rc |= launch_embed(embed_table, wdtype == DS4G_BF16, token, 1, vocab, hidden, x_next, st);
  return rc;
  });
}

int ds4g_lmhead_sample(int32_t hidden, int32_t vocab, int32_t wdtype, const void* final_norm,
                       float rms_eps, const void* w_lm, const float* x, float temperature,
                       float top_p, uint64_t* rng_state, float* logits, int32_t* token,
                       const void* embed_table, float* x_next, void* ws, size_t ws_bytes,
                       void* stream) {
  ds4g_sample_params p{temperature, top_p, 0.f, nullptr};
  return ds4g_lmhead_sample_ex(hidden, vocab, wdtype, final_norm, rms_eps, w_lm, x, &p, rng_state,
                               logits, token, embed_table, x_next, ws, ws_bytes, stream);
}

int ds4g_embed(int32_t vocab, int32_t hidden, int32_t wdtype, const void* table,
               const int32_t* ids, int32_t T, float* x, void* stream) {
  if (vocab <= 0 || hidden <= 0 || T <= 0 || !table || !ids || !x) return DS4G_ERR_INVALID_ARG;
  if (wdtype != DS4G_F32 && wdtype != DS4G_BF16) return DS4G_ERR_INVALID_ARG;
  if (hidden % 8) return DS4G_ERR_UNSUPPORTED;
  return dry_then_run((hipStream_t)stream, [&](Exec ex) {
    return launch_embed(table, wdtype == DS4G_BF16, ids, T, vocab, hidden, x, ex);
  });
}

const char* ds4g_status_string(int status) {
  switch (status) {
    case DS4G_OK: return "ok";
    case DS4G_ERR_INVALID_ARG: return "invalid argument";
    case DS4G_ERR_UNSUPPORTED: return "unsupported size";
    case DS4G_ERR_WORKSPACE: return "workspace too small";
    case DS4G_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
