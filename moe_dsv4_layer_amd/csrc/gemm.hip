// GEMMs of the layer-major prefill: C = A . B^T with A the activations
// [rows, K] and B the weights [N, K] (both K-contiguous).
//
//   gemm_dma   bf16 x bf16 or fp16 x fp16 -> fp32 on the gfx950 matrix cores
//              (v_mfma_f32_32x32x16_bf16 / _f16), BM x BN x 64 tiles, 4 or 8
//              waves, an S-stage LDS ring filled by direct global -> LDS
//              loads.  fp16 runs the attention path of a prefill (its
//              activations in fp16 against fp16 images of the bf16 weights,
//              see f16_image_kernel).
//   gemm_simt  fp32 activations x (fp32 | bf16) weights on the vector ALUs,
//              64x64x16 tiles, 4x4 outputs per thread.  Used where the
//              activations must stay fp32 (the router logits decide integer
//              expert choices) and for fp32 weights.
//
// Both take the same arguments: an optional row gather of A, optional
// grouping (one weight matrix per expert, rows of an expert contiguous in
// "permuted" order, a device tile list), and fused epilogues (fp32 store,
// bf16 store, residual add, SwiGLU of a (gate, up) pair).
//
// The layer-major prefill (ds4-learning 端到端推理流程, 阶段三 逐层批处理) runs
// every token through one weight matrix before the next, which is what turns
// the per-token GEMVs of 阶段四 4.2 into these GEMMs.
#include "dev.h"
#include "kernels.h"

#include <type_traits>

// Wave grid of the 256x256 tiles (rows x columns of waves); measured choice.
#ifndef DS4G_BIG_WM
#define DS4G_BIG_WM 2
#endif
#ifndef DS4G_BIG_WN
#define DS4G_BIG_WN 4
#endif
// LDS stages and k-step width of the 256x256 tiles (2 x 64 or 4 x 32: the
// same 128 KB of LDS)
// 128 x 256 tiles for an output of 129..256 columns over many rows (1: on)
#ifndef DS4G_WIDE_ROUTER
#define DS4G_WIDE_ROUTER 1
#endif
#ifndef DS4G_BIG_S
#define DS4G_BIG_S 2
#endif
#ifndef DS4G_BIG_BK
#define DS4G_BIG_BK 64
#endif
// dense GEMMs may run 256 x 256 tiles from this many of them (one per CU)
#ifndef DS4G_BIG_MIN_BLOCKS
#define DS4G_BIG_MIN_BLOCKS 256
#endif
// 320 x 256 tiles for the residual-epilogue GEMMs over many rows (1: on)
#ifndef DS4G_TALL_RESID
#define DS4G_TALL_RESID 1
#endif
// Dense GEMMs with at least this many 128x128 tiles run in the XCD-contiguous
// tile order of the grouped GEMMs (0: never; measured no faster at 2048 or
// 16994 rows).
#ifndef DS4G_DENSE_REMAP_TILES
#define DS4G_DENSE_REMAP_TILES 0
#endif

namespace ds4g {

// ------------------------------------------------------------------ epilogue
__device__ __forceinline__ void epi_store(const GemmArgs& g, int row, int col, float v) {
  switch (g.epi) {
    case EPI_F32: static_cast<float*>(g.C)[(long)row * g.ldc + col] = v; break;
    case EPI_BF16: static_cast<uint16_t*>(g.C)[(long)row * g.ldc + col] = f32_to_bf16(v); break;
    case EPI_RESID: {
      float* c = static_cast<float*>(g.C) + (long)row * g.ldc + col;
      *c = *c + v;
      break;
    }
    default: break;
  }
}
__device__ __forceinline__ void epi_swiglu(const GemmArgs& g, int row, int col, float gt,
                                           float up) {
  const float z = silu(gt) * up;
  if (g.epi == EPI_SWIGLU_BF16)
    static_cast<uint16_t*>(g.C)[(long)row * g.ldc + col] = f32_to_bf16(z);
  else
    static_cast<float*>(g.C)[(long)row * g.ldc + col] = z;
}

// Resolve the (group, row range, weight pointers) of an M tile.
// Returns false when the tile index is beyond the device tile count.
struct TileInfo {
  int row0, row1;   // output rows [row0, row1)
  long boff;        // weight offset of the group (elements)
};
__device__ __forceinline__ bool tile_info(const GemmArgs& g, int mtile, int BM, TileInfo& ti) {
  if (g.tiles) {
    if (mtile >= *g.ntiles) return false;
    const int packed = g.tiles[mtile];
    const int grp = packed >> 16, mt = packed & 0xFFFF;
    const int base = g.row_off[grp];
    ti.row0 = base + mt * BM;
    const int end = g.row_off[grp + 1];
    ti.row1 = ti.row0 + BM < end ? ti.row0 + BM : end;
    ti.boff = (long)grp * g.b_stride;
  } else {
    ti.row0 = mtile * BM;
    ti.row1 = ti.row0 + BM < g.M ? ti.row0 + BM : g.M;
    ti.boff = 0;
  }
  return ti.row0 < ti.row1;
}

// =========================================================================
// SIMT GEMM (fp32 activations)
template <typename WT, bool DUAL>
__global__ void __launch_bounds__(256)
gemm_simt_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float Bs2[DUAL ? BK : 1][BN + 4];
  TileInfo ti;
  if (!tile_info(g, blockIdx.y, BM, ti)) return;
  const int n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = static_cast<const float*>(g.A);
  const WT* B = static_cast<const WT*>(g.B) + ti.boff;
  const WT* B2 = DUAL ? static_cast<const WT*>(g.B2) + ti.boff : nullptr;
  // loader mapping: 64 rows x 16 k = 256 float4
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int arow = ti.row0 + lr;
  long asrc = -1;
  if (arow < ti.row1) asrc = (long)(g.gather ? g.gather[arow] : arow) * g.lda;
  const int brow = n0 + lr;

  float acc[4][4] = {}, acc2[DUAL ? 4 : 1][4] = {};
  // split-K: block z covers k in [z*Kc, (z+1)*Kc)
  const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
  const int Kc = g.K / nsplit;
  const int kbeg = blockIdx.z * Kc, kend = kbeg + Kc;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f);
    if (asrc >= 0) av = *reinterpret_cast<const float4*>(A + asrc + k0 + lk);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Bs[lk + e][lr] = (brow < g.N) ? ldw(B, (long)brow * g.K + k0 + lk + e) : 0.f;
      if (DUAL) Bs2[lk + e][lr] = (brow < g.N) ? ldw(B2, (long)brow * g.K + k0 + lk + e) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
      if (DUAL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b2[i] = Bs2[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += a[i] * b[j];
          if (DUAL) acc2[i][j] += a[i] * b2[j];
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = ti.row0 + ty * 4 + i;
    if (row >= ti.row1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= g.N) continue;
      if (DUAL) epi_swiglu(g, row, col, acc[i][j], acc2[i][j]);
      else if (nsplit > 1)
        static_cast<float*>(g.C)[blockIdx.z * g.part_stride + (long)row * g.ldc + col] = acc[i][j];
      else epi_store(g, row, col, acc[i][j]);
    }
  }
}

// =========================================================================
// MFMA GEMM (bf16 activations and weights), v_mfma_f32_32x32x16_bf16.
//
// Block tile BM x BN x 64 with WM x WN waves, wave tile TM x TN of 32x32
// fragments.  Operand layout of the instruction (lane l):
//   A: row l%32, k = 8*(l/32) .. +7 of the 16-wide k step (16 bytes)
//   B: col l%32, same k
//   C: acc[4j+i] = C[8j + 4*(l/32) + i][l%32]
// Both operands are K-contiguous in memory and in LDS.  Rows past the end of
// the tile (ragged M, N) load a clamped valid row, so no load is
// conditional; their results are never stored.  Every output element sums
// its K products in the same order whatever the tiling of M, which keeps a
// prefill split into chunks bit-identical to the whole.
// SwiGLU (EPI_SWIGLU_*): B tile rows come in 32-row blocks alternating gate /
// up rows of the same output columns, so a wave's fragment pair (fn, fn+1)
// holds gate and up of the same (row, col) in the same lane.
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// one 32x32x16 step on 16-byte operand fragments of either 16-bit type
template <bool F16>
__device__ __forceinline__ f32x16 mfma16(u32x4_t a, u32x4_t b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int EPI>
__device__ __forceinline__ void epi_store_t(const GemmArgs& g, int row, int col, float v) {
  if (EPI == EPI_F32) static_cast<float*>(g.C)[(long)row * g.ldc + col] = v;
  if (EPI == EPI_BF16) static_cast<uint16_t*>(g.C)[(long)row * g.ldc + col] = f32_to_bf16(v);
  if (EPI == EPI_F16) static_cast<uint16_t*>(g.C)[(long)row * g.ldc + col] = f32_to_f16(v);
  if (EPI == EPI_RESID) {
    float* c = static_cast<float*>(g.C) + (long)row * g.ldc + col;
    *c = *c + v;
  }
}

// Epilogue of a wave tile: rows row0 + 32 i + 8 jj + 4 (lane/32) + ii, columns
// col0 + 32 j + lane%32 (SwiGLU: fragment pairs (j, j+1) give one column
// block).  For the residual add the 16 old values of a fragment are loaded
// before any of them is stored, so the loads overlap instead of alternating
// with the stores.  A column factor (colscale) multiplies the accumulator
// first: a power of two, so it changes no bit of the significand.
template <int EPI, int FM, int FN, bool ATOMIC = true>
__device__ __forceinline__ void mfma_epilogue(const GemmArgs& g, f32x16 (&acc)[FM][FN],
                                              int row0, int row1, int col0, int lane) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_F32);
  const int lr = lane & 31, lg = lane >> 5;
  if (!DUAL && g.colscale) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float f = g.colscale[min(col0 + j * 32 + lr, g.N - 1)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= f;
    }
  }
  if (EPI == EPI_ROPE_QKV) {
    // the partner of column n in its rotation pair (n ^ 1) is in lane ^ 1:
    // x0' = x0 c - x1 s (even column), x1' = x0 s + x1 c (odd column).
    // Two rounded products and a rounded sum, no contraction: every tile
    // shape rounds a row alike, so prefills split anywhere agree bit for bit.
#pragma clang fp contract(off)
    const int dh = g.rope_dh, qd = g.N - 2 * dh, off = dh - g.rope_rd;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + j * 32 + lr;
      int e;
      uint16_t* dst;
      long ld;
      if (col < qd) { e = col % dh; dst = static_cast<uint16_t*>(g.C) + col; ld = g.ldc; }
      else if (col < qd + dh) { e = col - qd; dst = g.rope_kc + e; ld = dh; }
      else { e = col - qd - dh; dst = g.rope_vc + e; ld = dh; }
      const bool rot = col < qd + dh && e >= off;
      const long tab = (long)(rot ? (e - off) >> 1 : 0) * g.rope_ld;
      const float sgn = (col & 1) ? 1.f : -1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int rb = row0 + i * 32 + 8 * q4 + 4 * lg;
          const int rt = min(rb, g.rope_ld - 4);   // rows past the table are not stored
          // lanes lr, lr ^ 1 share the pair: the even one loads cos, the odd
          // one sin, and they swap halves
          const float4 mine = *reinterpret_cast<const float4*>(
              ((col & 1) ? g.rope_s : g.rope_c) + tab + rt);
          const float m4[4] = {mine.x, mine.y, mine.z, mine.w};
          float cv[4], sv[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float other = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(m4[k]), 0xB1, 0xF, 0xF, false));
            cv[k] = (col & 1) ? other : m4[k];
            sv[k] = (col & 1) ? m4[k] : other;
          }
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float own = acc[i][j][4 * q4 + ii];
            const float oth = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(own), 0xB1, 0xF, 0xF, false));
            const float v = rot ? own * cv[ii] + sgn * oth * sv[ii] : own;
            const int row = rb + ii;
            if (col < g.N && row < row1) dst[(long)row * ld] = f32_to_f16(v);
          }
        }
    }
    return;
  }
  if (EPI == EPI_RESID) {
    // C += acc.  ATOMIC: one fp32 add per element done in L2 (no-return
    // atomic): one tile owns each element, so it is a single read-modify-write
    // with the rounding of the load / add / store, and the wave does not wait
    // for C to arrive.  It helps the shared down (beside the routed experts)
    // and the short prefills' 64-row tiles; W_o's big fp16-operand tiles keep
    // the load / add / store, which measured faster there.
    float* C = static_cast<float*>(g.C);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + j * 32 + lr;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (ATOMIC) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = row0 + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
            if (row < row1)
              __builtin_amdgcn_global_atomic_fadd_f32(
                  (__attribute__((address_space(1))) float*)(C + (long)row * g.ldc + col),
                  acc[i][j][e]);
          }
        } else {
          float old[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = min(row0 + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3), row1 - 1);
            old[e] = C[(long)row * g.ldc + col];
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = row0 + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
            if (row < row1) C[(long)row * g.ldc + col] = old[e] + acc[i][j][e];
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = row0 + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
      if (row >= row1) continue;
      if (DUAL) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int col = col0 + (j >> 1) * 32 + lr;
          if (col < g.N) epi_swiglu(g, row, col, acc[i][j][e], acc[i][j + 1][e]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = col0 + j * 32 + lr;
          if (col < g.N) epi_store_t<EPI>(g, row, col, acc[i][j][e]);
        }
      }
    }
}

// 16-bit outputs (EPI_BF16, EPI_F16, EPI_SWIGLU_BF16, EPI_ROPE_QKV) through
// LDS: each wave writes its fragments' final values into a row-major tile
// [BM][OUTC] (row stride OUTC * 2 + 16 bytes, so the two row groups of a
// fragment write land on different banks), then the block stores 16-byte
// chunks: 8 lanes cover 128 bytes of a row, where the fragment layout stores
// two 64-byte runs of 2-byte values per instruction.  Same values, same
// rounding as mfma_epilogue.  stg: LDS bytes, free (every wave is past its
// last read of the ring).  Returns with the block synchronised.
template <int EPI, int BM, int OUTC, int NT, int FM, int FN>
__device__ __forceinline__ void staged_epilogue(const GemmArgs& g, f32x16 (&acc)[FM][FN],
                                                unsigned char* stg, int trow0, int row1,
                                                int tcol0, int wrow0, int wcol0, int lane) {
  constexpr bool DUAL = EPI == EPI_SWIGLU_BF16;
  constexpr int RS = OUTC * 2 + 16;
  const int lr = lane & 31, lg = lane >> 5;
  if (!DUAL && g.colscale) {   // as mfma_epilogue: the column factor first
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const float f = g.colscale[min(tcol0 + wcol0 + j * 32 + lr, g.N - 1)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= f;
    }
  }
  auto put = [&](int lrow, int lcol, uint16_t v) {
    *reinterpret_cast<uint16_t*>(stg + lrow * RS + lcol * 2) = v;
  };
  if constexpr (EPI == EPI_ROPE_QKV) {
#pragma clang fp contract(off)
    const int dh = g.rope_dh, qd = g.N - 2 * dh, off = dh - g.rope_rd;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int lcol = wcol0 + j * 32 + lr, col = tcol0 + lcol;
      const int e = col < qd ? col % dh : (col < qd + dh ? col - qd : col - qd - dh);
      const bool rot = col < qd + dh && e >= off;
      const long tab = (long)(rot ? (e - off) >> 1 : 0) * g.rope_ld;
      const float sgn = (col & 1) ? 1.f : -1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int lrow = wrow0 + i * 32 + 8 * q4 + 4 * lg;
          const int rt = min(trow0 + lrow, g.rope_ld - 4);   // rows past the table are not stored
          const float4 mine = *reinterpret_cast<const float4*>(
              ((col & 1) ? g.rope_s : g.rope_c) + tab + rt);
          const float m4[4] = {mine.x, mine.y, mine.z, mine.w};
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const float other = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(m4[ii]), 0xB1, 0xF, 0xF, false));
            const float cv = (col & 1) ? other : m4[ii];
            const float sv = (col & 1) ? m4[ii] : other;
            const float own = acc[i][j][4 * q4 + ii];
            const float oth = __int_as_float(
                __builtin_amdgcn_mov_dpp(__float_as_int(own), 0xB1, 0xF, 0xF, false));
            const float v = rot ? own * cv + sgn * oth * sv : own;
            put(lrow + ii, lcol, f32_to_f16(v));
          }
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int lrow = wrow0 + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
        if constexpr (DUAL) {
#pragma unroll
          for (int j = 0; j < FN; j += 2)
            put(lrow, wcol0 + (j >> 1) * 32 + lr,
                f32_to_bf16(silu(acc[i][j][e]) * acc[i][j + 1][e]));
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const float v = acc[i][j][e];
            put(lrow, wcol0 + j * 32 + lr, EPI == EPI_F16 ? f32_to_f16(v) : f32_to_bf16(v));
          }
        }
      }
  }
  __syncthreads();
  constexpr int CPRW = OUTC / 8;   // 16-byte chunks per row
  const int nrows = min(BM, row1 - trow0);
  const int qd = EPI == EPI_ROPE_QKV ? g.N - 2 * g.rope_dh : 0;
  for (int c = threadIdx.x; c < nrows * CPRW; c += NT) {
    const int lrow = c / CPRW, cc = c - lrow * CPRW;
    const int col = tcol0 + cc * 8, row = trow0 + lrow;
    if (col >= g.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(stg + lrow * RS + cc * 16);
    uint16_t* dst;
    if constexpr (EPI == EPI_ROPE_QKV) {
      const int dh = g.rope_dh;
      if (col < qd) dst = static_cast<uint16_t*>(g.C) + (long)row * g.ldc + col;
      else if (col < qd + dh) dst = g.rope_kc + (long)row * dh + (col - qd);
      else dst = g.rope_vc + (long)row * dh + (col - qd - dh);
    } else {
      dst = static_cast<uint16_t*>(g.C) + (long)row * g.ldc + col;
    }
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

// =========================================================================
// MFMA GEMM with an S-stage LDS ring filled by direct global -> LDS loads
// (buffer_load_dwordx4 ... lds): each lane's 16 bytes land in a fixed LDS
// slot (wave base in M0 + 16 * lane), so the swizzle is applied on the
// global side: LDS slot s of row r receives logical chunk s ^ f(r).  No
// registers stage the tiles and tile t+S-1 is in flight while tile t is
// multiplied.  The loads are issued from inline assembly and counted with
// explicit vmcnt waits: the compiler's own LDS-DMA tracking would wait for
// every outstanding load before any LDS read, which defeats the pipeline.
__device__ __forceinline__ void dma16(i32x4_t rs, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_byte), "v"(voff), "s"(rs) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }

// LDS slot of chunk c of row r, rows of CPR 16-byte chunks: the chunk index
// is XORed with bits of the row so that the 16 rows one fragment read takes
// at a time land on distinct banks (128-byte rows: bits 1..3; 64-byte rows:
// bits 2..3)
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return r * CPR + (c ^ (CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3)));
}

// Workgroups go to the 8 XCDs round-robin (linear id % 8), each XCD with its
// own L2.  Renumbering the nb tiles that have work so that XCD k runs a
// contiguous run of them (N tile fastest) keeps each expert's weight panels
// and gathered rows on one XCD, fetched from HBM once rather than by several
// XCDs.  A bijection of [0, nb) for any nb; the grid's blocks past nb (a
// grouped launch sizes its grid for the worst case) have no tile.
__device__ __forceinline__ bool xcd_tile(int nb, int& bx, int& by) {
  const int gx = gridDim.x;
  const int L = blockIdx.y * gx + blockIdx.x;
  if (L >= nb) return false;
  const int c = nb >> 3, r = nb & 7, k = L & 7, i = L >> 3;
  const int lt = k * c + min(k, r) + i;
  bx = lt % gx;
  by = lt / gx;
  return true;
}

template <int BM, int BN, int WM, int WN, int S, int EPI, bool F16, int BK, bool STG>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_dma_kernel(GemmArgs g) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_F32);
  constexpr int NW = WM * WN;
  constexpr int CPR = BK / 8;                // 16-byte chunks per LDS row
  constexpr int RPL = 64 / CPR;              // LDS rows per 1 KB wave load
  constexpr int KS = BK / 16;                // MFMA k steps per stage
  static_assert(BK == 64 || BK == 32, "64- or 32-wide k steps");
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int ROWS = BM + BN;              // LDS rows per stage (A rows, then B rows)
  constexpr int NDMA = ROWS / (RPL * NW);    // 1 KB loads per wave per stage
  static_assert(FM >= 1 && FN >= 1 && TM * WM == BM && TN * WN == BN, "32x32 fragments");
  static_assert(NDMA * RPL * NW == ROWS && BM % RPL == 0, "whole loads per wave");
  static_assert(!DUAL || FN % 2 == 0, "SwiGLU pairs gate/up fragments");
  static_assert(S >= 2 && (S - 2) * NDMA <= 63, "vmcnt range");
  constexpr int OUTC = DUAL ? BN / 2 : BN;
  constexpr bool STAGE = STG && (EPI == EPI_BF16 || EPI == EPI_F16 ||
                                EPI == EPI_SWIGLU_BF16 || EPI == EPI_ROPE_QKV);
  constexpr int RING = S * ROWS * CPR;                              // 16-byte entries
  constexpr int STGN = STAGE ? (BM * (OUTC * 2 + 16) + 15) / 16 : 0;   // staging entries
  __shared__ u32x4_t smem_all[RING > STGN ? RING : STGN];
  auto smem = reinterpret_cast<u32x4_t(*)[ROWS * CPR]>(smem_all);
  TileInfo ti;
  int bx = blockIdx.x, by = blockIdx.y;
  if (g.xcd_remap && gridDim.z == 1 &&
      !xcd_tile(gridDim.x * (g.tiles ? min(*g.ntiles, (int)gridDim.y) : (int)gridDim.y), bx, by))
    return;
  if (!tile_info(g, by, BM, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const int ncol0 = bx * (DUAL ? BN / 2 : BN);
  const uint16_t* Bp = static_cast<const uint16_t*>(g.B) + ti.boff;
  const uint16_t* B2p = DUAL ? static_cast<const uint16_t*>(g.B2) + ti.boff : nullptr;
  const i32x4_t rsA = buffer_rsrc(g.A), rsB = buffer_rsrc(Bp);
  const i32x4_t rsB2 = DUAL ? buffer_rsrc(B2p) : rsB;

  // per load j of this wave: source descriptor choice and byte offset at k = 0
  uint32_t voff[NDMA];
  int which[NDMA];   // 0: A, 1: B, 2: B2 (wave-uniform)
  int arow[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    arow[j] = min(ti.row0 + (wid * NDMA + j) * RPL + lane / CPR, ti.row1 - 1);
  if (g.gather) {   // all gather loads issued together
    int src[NDMA];
#pragma unroll
    for (int j = 0; j < NDMA; ++j) src[j] = g.gather[arow[j]];
#pragma unroll
    for (int j = 0; j < NDMA; ++j) arow[j] = src[j];
  }
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int I = wid * NDMA + j;            // stage rows RPL*I .. RPL*I + RPL-1
    const int row = I * RPL + lane / CPR, slot = lane % CPR;
    const int c = swz<CPR>(row, slot) - row * CPR;   // logical chunk stored in this slot
    if (I * RPL < BM) {
      voff[j] = (uint32_t)(((long)arow[j] * g.lda + c * 8) * 2);
      which[j] = 0;
    } else {
      const int r = row - BM;
      int brow;
      if (DUAL) {
        const int blk = r >> 5;
        which[j] = (blk & 1) ? 2 : 1;
        brow = ncol0 + (blk >> 1) * 32 + (r & 31);
      } else {
        which[j] = 1;
        brow = ncol0 + r;
      }
      voff[j] = (uint32_t)(((long)min(brow, g.N - 1) * (g.brep ? g.brep : g.K) + c * 8) * 2);
    }
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(&smem[0][0]);
  // split-K: slice z of ksplit covers k in [z*K/ksplit, (z+1)*K/ksplit) and
  // writes its partial sums (EPI_F32 only) to C + z * part_stride
  const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
  const int kbase = (int)blockIdx.z * (g.K / nsplit);
  const int nk = g.K / nsplit / BK;
  // k of step kt; a repeated B (brep) reads its column k % brep
  auto issue = [&](int kt, int st) {
    const int k = kbase + kt * BK;
    const int kb = g.brep ? k % g.brep : k;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const uint32_t dst = lds0 + (uint32_t)(st * ROWS * CPR * 16 + (wid * NDMA + j) * 1024);
      const i32x4_t rs = which[j] == 0 ? rsA : (which[j] == 1 ? rsB : rsB2);
      dma16(rs, __builtin_amdgcn_readfirstlane(dst),
            voff[j] + (uint32_t)((which[j] == 0 ? k : kb) * 2));
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int lr = lane & 31, lg = lane >> 5;
  // Row fragments of this wave that hold a row of the tile.  A partly filled
  // tile (the last tile of an expert, or of M) neither reads nor multiplies
  // the fragments past its last row; the rows it holds sum the same products
  // in the same order.  The main loop is instantiated per count of live
  // fragments, so every accumulator index stays a constant.
  const int vrows = __builtin_amdgcn_readfirstlane(ti.row1 - ti.row0);
  const int live = __builtin_amdgcn_readfirstlane(min(FM, max(0, (vrows - wm * TM + 31) >> 5)));
  auto run = [&](auto live_c) {
    constexpr int LIVE = decltype(live_c)::value;
    // The fragments of k step ks + 1 are read from LDS while the MFMAs of
    // step ks run (two fragment buffers), one read issued after each MFMA:
    // left to itself the scheduler put each read right before its first
    // use and the MFMAs waited on LDS latency.  Each accumulator still sums
    // its k steps in order, so the result does not change.
    auto compute = [&](int st) {
      const u32x4_t* As = &smem[st][0];
      const u32x4_t* Bs = &smem[st][BM * CPR];
      u32x4_t af[2][LIVE > 0 ? LIVE : 1], bfr[2][FN];
      auto load = [&](int ks, int b) {
#pragma unroll
        for (int i = 0; i < LIVE; ++i) af[b][i] = As[swz<CPR>(wm * TM + i * 32 + lr, ks * 2 + lg)];
        if (LIVE > 0) {
#pragma unroll
          for (int j = 0; j < FN; ++j) bfr[b][j] = Bs[swz<CPR>(wn * TN + j * 32 + lr, ks * 2 + lg)];
        }
      };
      load(0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int i = 0; i < LIVE; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = mfma16<F16>(af[ks & 1][i], bfr[ks & 1][j], acc[i][j]);
      }
      if constexpr (LIVE > 0) {   // the order the scheduler keeps (masks: 0x100 LDS read, 0x008 MFMA)
        constexpr int NL = LIVE + FN, NM = LIVE * FN, NI = NL < NM ? NL : NM;
        __builtin_amdgcn_sched_group_barrier(0x100, NL, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) {
#pragma unroll
            for (int t = 0; t < NI; ++t) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (NL > NM) __builtin_amdgcn_sched_group_barrier(0x100, NL - NM, 0);
            if (NM > NL) __builtin_amdgcn_sched_group_barrier(0x008, NM - NL, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
          }
        }
      }
    };
#pragma unroll
    for (int t = 0; t < S - 1; ++t)
      if (t < nk) issue(t, t);
    for (int kt = 0; kt < nk; ++kt) {
      // tile kt has landed once at most min(S-2, nk-1-kt) later tiles are pending
      if (kt + S - 2 < nk) wait_vm<(S - 2) * NDMA>();
      else wait_vm<0>();
      barrier_lds();   // every wave: tile kt visible, and done reading the stage refilled next
      if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
      compute(kt % S);
    }
  };
  if (live == FM) run(std::integral_constant<int, FM>{});
  else if (FM >= 5 && live == 4) run(std::integral_constant<int, (FM >= 5 ? 4 : 0)>{});
  else if (FM >= 4 && live == 3) run(std::integral_constant<int, (FM >= 4 ? 3 : 0)>{});
  else if (FM >= 3 && live == 2) run(std::integral_constant<int, (FM >= 3 ? 2 : 0)>{});
  else if (FM >= 2 && live == 1) run(std::integral_constant<int, (FM >= 2 ? 1 : 0)>{});
  else run(std::integral_constant<int, 0>{});

  GemmArgs ge = g;
  if (nsplit > 1) ge.C = static_cast<float*>(g.C) + (long)blockIdx.z * g.part_stride;
  if constexpr (STAGE) {   // g.stage16: launch_gemm checked the 16-byte alignment
    barrier_lds();        // every wave is done reading the ring
    staged_epilogue<EPI, BM, OUTC, 64 * NW, FM, FN>(
        ge, acc, reinterpret_cast<unsigned char*>(smem_all), ti.row0, ti.row1, ncol0, wm * TM,
        wn * (DUAL ? TN / 2 : TN), lane);
  } else {
    mfma_epilogue<EPI, FM, FN, (!F16 || BM < 128)>(ge, acc, ti.row0 + wm * TM, ti.row1,
                               ncol0 + wn * (DUAL ? TN / 2 : TN), lane);
  }
}

template <int BM, int BN, int WM, int WN, int S, int BK = 64>
int launch_dma_cfg(const GemmArgs& g, Exec st) {
  const bool dual = (g.epi == EPI_SWIGLU_BF16 || g.epi == EPI_SWIGLU_F32);
  const int bn_out = dual ? BN / 2 : BN;
  const int mt = g.tiles ? g.max_tiles : (g.M + BM - 1) / BM;
  const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
  const dim3 grid((g.N + bn_out - 1) / bn_out, mt, nsplit), block(64 * WM * WN);
#define DS4G_DMA(E, F)                                                                     \
  {                                                                                        \
    if (g.stage16)                                                                         \
      DS4G_LAUNCH((gemm_dma_kernel<BM, BN, WM, WN, S, E, F, BK, true>), grid, block, 0, st, g); \
    else                                                                                   \
      DS4G_LAUNCH((gemm_dma_kernel<BM, BN, WM, WN, S, E, F, BK, false>), grid, block, 0, st, g); \
  }
  if (g.f16) {   // the attention path: fp16 operands
    if (g.tiles) return -1;
    switch (g.epi) {
      case EPI_F32: DS4G_DMA(EPI_F32, true); break;
      case EPI_F16: DS4G_DMA(EPI_F16, true); break;
      case EPI_RESID: DS4G_DMA(EPI_RESID, true); break;
      case EPI_ROPE_QKV:
        if (nsplit > 1) return -1;
        DS4G_DMA(EPI_ROPE_QKV, true);
        break;
      default: return -1;
    }
    return 0;
  }
  switch (g.epi) {
    case EPI_F32: DS4G_DMA(EPI_F32, false); break;
    case EPI_BF16: DS4G_DMA(EPI_BF16, false); break;
    case EPI_RESID: DS4G_DMA(EPI_RESID, false); break;
    case EPI_SWIGLU_BF16: DS4G_DMA(EPI_SWIGLU_BF16, false); break;
    default: return -1;
  }
#undef DS4G_DMA
  return 0;
}

// fp16 image of bf16 weights, one wave per row (see launch_f16_image): the
// largest magnitude of the row (bf16 magnitudes order like their bit
// patterns), then every element times 2^s rounded to fp16, s = 14 - e with
// 2^e <= max < 2^(e+1).  The row is read twice; the second read hits L2.
__global__ void __launch_bounds__(256)
f16_image_kernel(const uint16_t* __restrict__ W, int N, int K, uint16_t* __restrict__ img,
                 float* __restrict__ inv) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint16_t* row = W + (long)n * K;
  uint16_t* out = img + (long)n * K;
  const int nchunk = K >> 3;
  uint32_t mb = 0;
  for (int c = lane; c < nchunk; c += 64) {
    const uint4 q = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) mb = max(mb, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  mb = (uint32_t)wave_max((float)mb);              // exact: below 2^15
  const int eb = (int)(mb >> 7);                   // biased bf16 exponent of the largest
  const int sc = (mb == 0 || eb == 255) ? 0 : 141 - eb;   // 14 - (eb - 127)
  for (int c = lane; c < nchunk; c += 64) {
    const uint4 q = *reinterpret_cast<const uint4*>(row + c * 8);
    float f[8];
    unpack8(q, f);
    uint4 o;
    o.x = pack_f16x2(ldexpf(f[0], sc), ldexpf(f[1], sc));
    o.y = pack_f16x2(ldexpf(f[2], sc), ldexpf(f[3], sc));
    o.z = pack_f16x2(ldexpf(f[4], sc), ldexpf(f[5], sc));
    o.w = pack_f16x2(ldexpf(f[6], sc), ldexpf(f[7], sc));
    *reinterpret_cast<uint4*>(out + c * 8) = o;
  }
  if (lane == 0) inv[n] = ldexpf(1.f, -sc);
}

int launch_f16_image(const uint16_t* W, int N, int K, uint16_t* img, float* inv, Exec st) {
  if (N <= 0 || K <= 0 || K % 8) return -1;
  DS4G_LAUNCH(f16_image_kernel, dim3((N + 3) / 4), dim3(256), 0, st, W, N, K, img, inv);
  return 0;
}

// Split-K partial sums part[s][m][n] (s < nsplit, stride pstride), times the
// column factor (colscale, optional), then the epilogue: F32, BF16, F16,
// RESID (C += sum) or SWIGLU_BF16 (C = bf16(silu(sum part) * sum part2)).  A block takes 32 consecutive elements; its 8 groups of
// 32 threads add the splits g, g + 8, ... of their element, and the 8 group
// sums are added in group order (a fixed order: results do not depend on
// timing).  Spreading the splits over threads keeps many loads in flight.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, const float* __restrict__ part2, int nsplit,
                     long pstride, int M, int N, int epi, void* C, int ldc,
                     const float* __restrict__ colscale) {
  __shared__ float acc[2][8][32];
  const int e = threadIdx.x & 31, g = threadIdx.x >> 5;
  const long i = (long)blockIdx.x * 32 + e;
  const bool live = i < (long)M * N;
  float v = 0.f, u = 0.f;
  if (live) {
#pragma unroll 4
    for (int s = g; s < nsplit; s += 8) v += part[s * pstride + i];
    if (epi == EPI_SWIGLU_BF16) {
#pragma unroll 4
      for (int s = g; s < nsplit; s += 8) u += part2[s * pstride + i];
    }
  }
  acc[0][g][e] = v;
  acc[1][g][e] = u;
  __syncthreads();
  if (g != 0 || !live) return;
  v = 0.f;
  u = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) { v += acc[0][q][e]; u += acc[1][q][e]; }
  const int m = (int)(i / N), n = (int)(i - (long)m * N);
  if (colscale) v *= colscale[n];
  if (epi == EPI_SWIGLU_BF16) {
    static_cast<uint16_t*>(C)[(long)m * ldc + n] = f32_to_bf16(silu(v) * u);
  } else if (epi == EPI_BF16) {
    static_cast<uint16_t*>(C)[(long)m * ldc + n] = f32_to_bf16(v);
  } else if (epi == EPI_F16) {
    static_cast<uint16_t*>(C)[(long)m * ldc + n] = f32_to_f16(v);
  } else if (epi == EPI_RESID) {
    float* c = static_cast<float*>(C) + (long)m * ldc + n;
    *c = *c + v;
  } else {
    static_cast<float*>(C)[(long)m * ldc + n] = v;
  }
}

int launch_splitk_reduce(const float* part, const float* part2, int nsplit, long pstride, int M,
                         int N, int epi, void* C, int ldc, const float* colscale, Exec st) {
  if (epi != EPI_F32 && epi != EPI_BF16 && epi != EPI_F16 && epi != EPI_RESID &&
      epi != EPI_SWIGLU_BF16)
    return -1;
  if (epi == EPI_SWIGLU_BF16 && (!part2 || colscale)) return -1;
  const long n = (long)M * N;
  DS4G_LAUNCH(splitk_reduce_kernel, dim3((unsigned)((n + 31) / 32)), dim3(256), 0, st,
                     part, part2, nsplit, pstride, M, N, epi, C, ldc, colscale);
  return 0;
}

#ifndef DS4G_TALL_SINGLE_PASS   // 320 x 256 for fp16 / fp32 outputs that then fit one round (1: on)
#define DS4G_TALL_SINGLE_PASS 1
#endif
#if DS4G_TALL_RESID
// 320 x 256 tiles, residual epilogue only (the staged 16-bit epilogue would
// need more LDS than a CU has)
static int launch_tall_resid(const GemmArgs& g, Exec st) {
  const dim3 grid((g.N + 255) / 256, (g.M + 319) / 320, 1), block(512);
  if (g.f16) DS4G_LAUNCH((gemm_dma_kernel<320, 256, 2, 4, 2, EPI_RESID, true, 64, false>), grid, block, 0, st, g);
  else DS4G_LAUNCH((gemm_dma_kernel<320, 256, 2, 4, 2, EPI_RESID, false, 64, false>), grid, block, 0, st, g);
  return 0;
}
#endif

int launch_gemm(const GemmArgs& g0, bool mfma, int wdtype_bf16, Exec st) {
  const bool dual = (g0.epi == EPI_SWIGLU_BF16 || g0.epi == EPI_SWIGLU_F32);
  GemmArgs g = g0;
  if (mfma && !g.tiles && DS4G_DENSE_REMAP_TILES > 0) {
    const long nt = ((g.M + 127) / 128) * (((dual ? 2L * g.N : g.N) + 127) / 128);
    if (nt >= DS4G_DENSE_REMAP_TILES) g.xcd_remap = 1;
  }
  if (mfma) {
    const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
    if (g.K % (64 * nsplit)) return -1;
    if (nsplit > 1 && (g.epi != EPI_F32 || g.tiles)) return -1;
    // byte offsets of the direct loads are 32-bit
    if ((double)g.N * (g.brep ? g.brep : g.K) * 2 >= 4294967296.0) return -1;
    if (g.brep && (g.brep % 64 || g.K % g.brep)) return -1;
    // 16-bit outputs are stored 16 bytes at a time (staged_epilogue)
    const bool out16 = g.epi == EPI_BF16 || g.epi == EPI_F16 || g.epi == EPI_SWIGLU_BF16 ||
                       g.epi == EPI_ROPE_QKV;
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!out16) g.stage16 = 0;
    if (g.stage16 && (g.N % 8 || g.ldc % 8 || !a16(g.C))) return -1;
    if (g.stage16 && g.epi == EPI_ROPE_QKV &&
        (g.rope_dh % 8 || !a16(g.rope_kc) || !a16(g.rope_vc)))
      return -1;
    if (g.tiles) {   // the tile list was built for exactly rows_hint rows per tile
      // 64-row tiles (few rows per expert: a 2048-token prefill, batched
      // decode): 128 columns per tile, so small calls have more blocks to
      // spread over the CUs and two blocks fit a CU's LDS
      if (g.rows_hint == 64) return launch_dma_cfg<64, 128, 2, 2, 3>(g, st);
      if (g.rows_hint == 128) return launch_dma_cfg<128, 256, 2, 4, 3>(g, st);
      if (g.rows_hint == 256) return launch_dma_cfg<256, 256, DS4G_BIG_WM, DS4G_BIG_WN, DS4G_BIG_S, DS4G_BIG_BK>(g, st);
      return -1;
    }
    const long nout = dual ? g.N * 2L : g.N;           // B rows per output row
    const long big_blocks = ((g.M + 255) / 256) * ((nout + 255) / 256) * nsplit;
#if DS4G_TALL_RESID
    // residual epilogue (W_o, the shared down) over many rows: 320 x 256 tiles,
    // a tenth fewer operand bytes per flop than 256 x 256
    if (g.epi == EPI_RESID && !g.tiles && nsplit == 1 && !dual && g.M >= 4096) {
      const long nt = (nout + 255) / 256, mt = (g.M + 319) / 320;
      const int mb = (int)((mt * nt / 256) * 256 / nt) * 320;   // rows in whole rounds
      if (mb > 0 && mb < g.M && (mt * nt) % 256 != 0) {
        GemmArgs hi = g, lo = g;
        hi.M = mb;
        lo.M = g.M - mb;
        lo.A = static_cast<const uint16_t*>(g.A) + (long)mb * g.lda;
        lo.C = static_cast<char*>(g.C) + (size_t)mb * g.ldc * 4;
        const int r = launch_tall_resid(hi, st);
        if (r) return r;
        return launch_gemm(lo, mfma, wdtype_bf16, st);
      }
      return launch_tall_resid(g, st);
    }
#endif
#if DS4G_TALL_SINGLE_PASS
    // fp16 and fp32 outputs (QKV-A, the split-K router) whose rows need one
    // round and a few tiles more at 256 x 256 but fit one round at 320 x 256:
    // every row in one launch, stored directly (the staged epilogue does not
    // fit LDS beside a 320-row ring).  Not the shared gate/up: beside the
    // router on the second stream its 225-VGPR blocks left no room on their
    // CUs for the small routing kernels, and the layer was slower.
    if (((g.epi == EPI_F16 && nsplit == 1) || (g.epi == EPI_F32 && !g.f16)) && !dual &&
        !g.tiles && g.M >= 4096) {
      const long nt = (nout + 255) / 256;
      if (((g.M + 319) / 320) * nt * nsplit <= 256 && ((g.M + 255) / 256) * nt * nsplit > 256) {
        const dim3 grid((unsigned)((g.N + 255) / 256), (unsigned)((g.M + 319) / 320),
                        (unsigned)nsplit), block(512);
        if (g.epi == EPI_F32)
          DS4G_LAUNCH((gemm_dma_kernel<320, 256, 2, 4, 2, EPI_F32, false, 64, false>), grid, block, 0, st, g);
        else if (g.f16)
          DS4G_LAUNCH((gemm_dma_kernel<320, 256, 2, 4, 2, EPI_F16, true, 64, false>), grid, block, 0, st, g);
        else
          DS4G_LAUNCH((gemm_dma_kernel<320, 256, 2, 4, 2, EPI_F16, false, 64, false>), grid, block, 0, st, g);
        return 0;
      }
    }
#endif
    // Rows past the last whole round of 256x256 tiles (one per CU) run as
    // 128x128 tiles, a quarter of the work each, when they would fill less
    // than half of one more round of big tiles.  Every element keeps its K
    // order, so the split changes no bit of the result.
    const long bnt = (nout + 255) / 256, bmt = (g.M + 255) / 256;
    const long brem = (bmt * bnt) % 256;
    const int bmb = (int)((bmt * bnt / 256) * 256 / bnt) * 256;   // rows in whole rounds
    const bool bsplit = nsplit == 1 && g.epi != EPI_ROPE_QKV && brem > 0 && brem <= 128 &&
                        bmb > 0 && bmb < g.M;
    // 256x256 tiles from 512 of them; from 256 when the rows past the whole
    // round split off as above, or when split-K slices fill the round (the
    // prefill router: 268 blocks of 256x256 beat 532 of 128x256)
    if (big_blocks >= 512 || (big_blocks >= DS4G_BIG_MIN_BLOCKS && (bsplit || nsplit > 1))) {
      const long nt = bnt;
      const int mb = bmb;
      if (bsplit) {
        GemmArgs hi = g, lo = g;
        hi.M = mb;
        lo.M = g.M - mb;
        if (g.gather) lo.gather = g.gather + mb;
        else lo.A = static_cast<const uint16_t*>(g.A) + (long)mb * g.lda;
        const size_t es =
            (g.epi == EPI_BF16 || g.epi == EPI_F16 || g.epi == EPI_SWIGLU_BF16) ? 2 : 4;
        lo.C = static_cast<char*>(g.C) + (size_t)mb * g.ldc * es;
        const int r = launch_dma_cfg<256, 256, DS4G_BIG_WM, DS4G_BIG_WN, DS4G_BIG_S, DS4G_BIG_BK>(hi, st);
        if (r) return r;
        const long lblocks = ((lo.M + 127) / 128) * ((nout + 127) / 128);
        if (lblocks <= 256) return launch_dma_cfg<128, 128, 2, 2, 3>(lo, st);
        return launch_dma_cfg<128, 128, 2, 2, 2>(lo, st);
      }
      return launch_dma_cfg<256, 256, DS4G_BIG_WM, DS4G_BIG_WN, DS4G_BIG_S, DS4G_BIG_BK>(g, st);
    }
    if (g.M <= 64) return launch_dma_cfg<64, 256, 1, 4, 3>(g, st);
    // Output 129..256 columns wide (the router's experts) over many rows: one
    // 128 x 256 tile spans every column, so each row block of A is read once
    // rather than by two blocks on different XCDs (16 994 rows: 200 -> 162 us
    // in isolation).  With few rows the 128 x 128 grid's extra blocks win.
    if (DS4G_WIDE_ROUTER && nout > 128 && nout <= 256 && (g.M + 127) / 128 * nsplit >= 512)
      return launch_dma_cfg<128, 256, 2, 4, 3>(g, st);
    const long blocks = ((g.M + 127) / 128) * ((nout + 127) / 128) * nsplit;
    // a short prefill (a few row tiles) fills few CUs: 64-row tiles give
    // twice the blocks, each streaming a quarter fewer operand bytes.  Not
    // the shared expert's GEMMs (SwiGLU, and the residual add on bf16
    // operands): they run on the second stream, where more blocks only
    // crowd the kernels of the critical path.
    const bool shared_expert = dual || (g.epi == EPI_RESID && !g.f16);
    if (!shared_expert && blocks <= 192 && g.M > 64 && g.M <= 1024)
      return launch_dma_cfg<64, 128, 2, 2, 3>(g, st);
    // one block per CU either way: spend the LDS on a deeper pipeline
    if (blocks <= 256) return launch_dma_cfg<128, 128, 2, 2, 3>(g, st);
    return launch_dma_cfg<128, 128, 2, 2, 2>(g, st);
  } else {
    const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
    if (g.K % (16 * nsplit)) return -1;
    if (g.brep) return -1;   // the repeated B operand is an MFMA-path feature
    if (nsplit > 1 && (dual || g.epi != EPI_F32)) return -1;
    const int mt = g.tiles ? g.max_tiles : (g.M + 63) / 64;
    dim3 grid((g.N + 63) / 64, mt, nsplit);
    if (wdtype_bf16) {
      if (dual) DS4G_LAUNCH((gemm_simt_kernel<uint16_t, true>), grid, dim3(256), 0, st, g);
      else DS4G_LAUNCH((gemm_simt_kernel<uint16_t, false>), grid, dim3(256), 0, st, g);
    } else {
      if (dual) DS4G_LAUNCH((gemm_simt_kernel<float, true>), grid, dim3(256), 0, st, g);
      else DS4G_LAUNCH((gemm_simt_kernel<float, false>), grid, dim3(256), 0, st, g);
    }
  }
  return 0;
}

}  // namespace ds4g
