// GEMMs of the layer-major prefill: C = A . B^T with A the activations
// [rows, K] and B the weights [N, K] (both K-contiguous).
//
//   gemm_mfma  bf16 x bf16 -> fp32 on the gfx950 matrix cores
//              (v_mfma_f32_16x16x32_bf16), 128x128x64 tiles, 4 waves of
//              64x64, LDS double buffer with an XOR swizzle so the 16-byte
//              operand reads of 8 consecutive rows hit distinct banks.
//   gemm_simt  fp32 activations x (fp32 | bf16) weights on the vector ALUs,
//              64x64x16 tiles, 4x4 outputs per thread.  Used where the
//              activations must stay fp32 (the router logits decide integer
//              expert choices) and for fp32 weights.
//
// Both take the same arguments: an optional row gather of A, optional
// grouping (one weight matrix per expert, rows of an expert contiguous in
// "permuted" order, a device tile list), and fused epilogues (fp32 store,
// bf16 store, residual add, SwiGLU of a (gate, up) pair, MoE combine).
//
// The layer-major prefill (ds4-learning 端到端推理流程, 阶段三 逐层批处理) runs
// every token through one weight matrix before the next, which is what turns
// the per-token GEMVs of 阶段四 4.2 into these GEMMs.
#include "dev.h"
#include "kernels.h"

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
    case EPI_COMBINE: {
      // x[t] = h2[t] + shared[t] + sum_j w[t, j] * part[pos_of[t*k + j]]
      float* c = static_cast<float*>(g.C) + (long)row * g.ldc + col;
      float acc = *c + v;
      for (int j = 0; j < g.topk; ++j) {
        const int e = row * g.topk + j;
        acc += g.topk_w[e] * g.part[(long)g.pos_of[e] * g.ldp + col];
      }
      *c = acc;
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
// Block tile BM x BN x 64, 4 waves in a WM x WN grid, wave tile TM x TN of
// 32x32 fragments.  Operand layout of the instruction (lane l):
//   A: row l%32, k = 8*(l/32) .. +7 of the 16-wide k step (16 bytes)
//   B: col l%32, same k
//   C: acc[4j+i] = C[8j + 4*(l/32) + i][l%32]
// Both operands are K-contiguous in memory and in LDS; an LDS row is 8
// chunks of 16 bytes and chunk c of row r is stored at c ^ (r & 7), so the
// 8 rows read by 8 consecutive lanes hit 8 different chunk slots.  Global
// loads for the next k tile are issued before the current tile's MFMAs;
// LDS is double buffered (one barrier per k tile).
// SwiGLU (DUAL): B tile rows come in 32-row blocks alternating gate / up
// rows of the same output columns, so a wave's fragment pair (fn, fn+1)
// holds gate and up of the same (row, col) in the same lane.
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

#ifndef DS4G_SWZ_SHIFT
#define DS4G_SWZ_SHIFT 0
#endif
__device__ __forceinline__ int swz(int r, int c) {
  return r * 8 + (c ^ ((r >> DS4G_SWZ_SHIFT) & 7));
}

template <int BM, int BN, int WM, int WN, bool DUAL>
__global__ void __launch_bounds__(256)
gemm_mfma_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 1, "4 waves, 32x32 fragments");
  static_assert(!DUAL || FN % 2 == 0, "SwiGLU pairs gate/up fragments");
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][BN * 8];
  TileInfo ti;
  if (!tile_info(g, blockIdx.y, BM, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const uint16_t* A = static_cast<const uint16_t*>(g.A);
  const uint16_t* B = static_cast<const uint16_t*>(g.B) + ti.boff;
  const uint16_t* B2 = DUAL ? static_cast<const uint16_t*>(g.B2) + ti.boff : nullptr;
  const int ncol0 = blockIdx.x * (DUAL ? BN / 2 : BN);

  const uint16_t* asrc[ACH];
  const uint16_t* bsrc[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const int arow = ti.row0 + r;
    asrc[i] = nullptr;
    if (arow < ti.row1) asrc[i] = A + (long)(g.gather ? g.gather[arow] : arow) * g.lda + c * 8;
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    int brow;
    const uint16_t* bb = B;
    if (DUAL) {
      const int blk = r >> 5;
      bb = (blk & 1) ? B2 : B;
      brow = ncol0 + (blk >> 1) * 32 + (r & 31);
    } else {
      brow = ncol0 + r;
    }
    bsrc[i] = (brow < g.N) ? bb + (long)brow * g.K + c * 8 : nullptr;
  }
  uint4 ra[ACH], rb[BCH];
  auto gload_into = [&](int k0, uint4 (&xa)[ACH], uint4 (&xb)[BCH]) {
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      xa[i] = asrc[i] ? *reinterpret_cast<const uint4*>(asrc[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      xb[i] = bsrc[i] ? ldg_nt16(bsrc[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto lstore_from = [&](int st, const uint4 (&xa)[ACH], const uint4 (&xb)[BCH]) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int q = tid + 256 * i;
      As[st][swz(q >> 3, q & 7)] = xa[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int q = tid + 256 * i;
      Bs[st][swz(q >> 3, q & 7)] = xb[i];
    }
  };
  auto gload = [&](int k0) { gload_into(k0, ra, rb); };
  auto lstore = [&](int st) { lstore_from(st, ra, rb); };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = g.K / BK;
  const int lr = lane & 31, lg = lane >> 5;
  auto compute = [&](int st) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint4 v = As[st][swz(wm * TM + i * 32 + lr, ks * 2 + lg)];
        af[i] = *reinterpret_cast<const bf16x8*>(&v);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint4 v = Bs[st][swz(wn * TN + j * 32 + lr, ks * 2 + lg)];
        bfr[j] = *reinterpret_cast<const bf16x8*>(&v);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };
#if DS4G_GEMM_PF2
  // two register sets: tile t is loaded into set t&1 two iterations before
  // it is computed, and stored to LDS at the end of the iteration before
  uint4 ra2[ACH], rb2[BCH];
  gload_into(0, ra, rb);
  lstore_from(0, ra, rb);
  if (nk > 1) gload_into(BK, ra2, rb2);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) gload_into((kt + 2) * BK, ra, rb);
    compute(0);
    if (kt + 1 < nk) lstore_from(1, ra2, rb2);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 3 < nk) gload_into((kt + 3) * BK, ra2, rb2);
    compute(1);
    if (kt + 2 < nk) lstore_from(0, ra, rb);
    __syncthreads();
  }
#else
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    compute(st);
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }
#endif

  // epilogue
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int row = ti.row0 + wm * TM + i * 32 + 8 * jj + 4 * lg + ii;
        if (row >= ti.row1) continue;
        if (DUAL) {
#pragma unroll
          for (int j = 0; j < FN; j += 2) {
            const int col = ncol0 + (wn * (TN / 2)) + (j >> 1) * 32 + lr;
            if (col < g.N) epi_swiglu(g, row, col, acc[i][j][4 * jj + ii], acc[i][j + 1][4 * jj + ii]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = ncol0 + wn * TN + j * 32 + lr;
            if (col < g.N) epi_store(g, row, col, acc[i][j][4 * jj + ii]);
          }
        }
      }
    }
  }
}

int launch_gemm(const GemmArgs& g, bool mfma, int wdtype_bf16, hipStream_t st) {
  const bool dual = (g.epi == EPI_SWIGLU_BF16 || g.epi == EPI_SWIGLU_F32);
  if (mfma) {
    if (g.K % 64) return -1;
    // rows per tile: follow the rows a group (or the whole problem) has
    int rows = g.M;
    if (g.tiles) rows = g.rows_hint > 0 ? g.rows_hint : 128;
#define DS4G_MF(BM_, BN_, WM_, WN_)                                                      \
  {                                                                                      \
    const int bn_out = dual ? BN_ / 2 : BN_;                                             \
    const int mt = g.tiles ? g.max_tiles : (g.M + BM_ - 1) / BM_;                        \
    dim3 grid((g.N + bn_out - 1) / bn_out, mt);                                          \
    if (dual) hipLaunchKernelGGL((gemm_mfma_kernel<BM_, BN_, WM_, WN_, true>), grid, dim3(256), 0, st, g);  \
    else hipLaunchKernelGGL((gemm_mfma_kernel<BM_, BN_, WM_, WN_, false>), grid, dim3(256), 0, st, g);      \
    return 0;                                                                            \
  }
    if (g.tiles) {   // the tile list was built for exactly rows_hint rows per tile
      if (rows == 64) DS4G_MF(64, 256, 1, 4)
      if (rows == 128) DS4G_MF(128, 128, 2, 2)
      return -1;
    }
    // 256x128 tiles measured slower than 128x128 on every layer shape
    if (rows <= 64) DS4G_MF(64, 256, 1, 4)
    DS4G_MF(128, 128, 2, 2)
#undef DS4G_MF
  } else {
    const int nsplit = g.ksplit > 1 ? g.ksplit : 1;
    if (g.K % (16 * nsplit)) return -1;
    if (nsplit > 1 && (dual || g.epi != EPI_F32)) return -1;
    const int mt = g.tiles ? g.max_tiles : (g.M + 63) / 64;
    dim3 grid((g.N + 63) / 64, mt, nsplit);
    if (wdtype_bf16) {
      if (dual) hipLaunchKernelGGL((gemm_simt_kernel<uint16_t, true>), grid, dim3(256), 0, st, g);
      else hipLaunchKernelGGL((gemm_simt_kernel<uint16_t, false>), grid, dim3(256), 0, st, g);
    } else {
      if (dual) hipLaunchKernelGGL((gemm_simt_kernel<float, true>), grid, dim3(256), 0, st, g);
      else hipLaunchKernelGGL((gemm_simt_kernel<float, false>), grid, dim3(256), 0, st, g);
    }
  }
  return 0;
}

}  // namespace ds4g
