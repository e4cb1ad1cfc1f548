// launch.h - internal launch interface between the C ABI (api.cpp) and the
// device code (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace lora {

// rows per tile of the rank-r panel kernel (the split choice in api.cpp uses it)
constexpr int PANEL_BM = 128;
// The bf16 panel (G_BF16_PANEL_SPLIT_NT) runs panel_dma_kernel, which alone
// takes Bop rows from several sources (GemmArgs::n_src), for these shapes.
bool panel_dma_fits(int64_t n_store, int64_t lda, int64_t ldb);
// The whole-tile kernels' buffer offsets stay in range for operands with row
// strides up to ld (elements).
bool whole_ld_fits(int64_t ld);

// GEMM instances.  Suffixes: NT/NN = layout of the second operand, then the
// epilogue.  "BIG" = 256x256 tiles, "MED" = 128x128 (4 waves), "PANEL" =
// 64x64 rank-r panels, "SPLIT" = 64x256 split-contraction partials,
// "PANEL_SPLIT" = 256x64 split-contraction partials of a rank-r panel,
// "MED_*_PARTIAL" = 128x128 split-contraction partials of the layer's own
// GEMMs when their tiles alone cannot fill the chip (few tokens), "ADD" =
// the product plus an addend (the merge of the adapter into W).
enum GemmKind : int {
  G_BF16_BIG_NT_STORE,
  G_BF16_BIG_NT_ROPE,
  G_BF16_MED_NT_STORE,
  G_BF16_MED_NT_ROPE,
  G_BF16_BIG_NN_STORE,
  G_BF16_MED_NN_STORE,
  G_NF4_BIG_NT_STORE,
  G_NF4_MED_NT_STORE,
  G_NF4_BIG_NN_STORE,
  G_NF4_MED_NN_STORE,
  G_BF16_SPLIT_NN_PARTIAL,
  G_F32_NT_STORE,
  G_F32_NT_ROPE,
  G_F32_NN_STORE,
  G_F32_PANEL_NT_STORE,
  G_F32_PANEL_NT_STORE_T,
  G_F32_PANEL_NN_BOTH,
  G_F32_SPLIT_NN_PARTIAL,
  G_BF16_PANEL_SPLIT_NT,
  G_BF16_MED_NT_PARTIAL,
  G_BF16_MED_NN_PARTIAL,
  G_NF4_MED_NT_PARTIAL,
  G_NF4_MED_NN_PARTIAL,
  G_BF16_MED_NN_ADD,
  G_F32_NN_ADD,
  G_BF16_WHOLE_SWIGLU,
  G_BF16_MED_NN_ADD_MASKED,
  G_F32_NN_ADD_MASKED,
  G_BF16_WHOLE_GROUP,  // several projections' forward GEMMs in one whole-tile launch (GemmArgs::n_mem)
  G_NF4_WHOLE_NT_STORE,  // whole-tile forward GEMM, NF4 W expanded in the load stage (gemm_w4_nf4_kernel)
  G_KIND_COUNT
};

struct TileShape {
  int bm, bn;
};
TileShape gemm_tile(GemmKind k);

// Sets a.tiles_m from a.m_store and launches over (tiles_m * tiles_n, 1, splits).
hipError_t launch_gemm(GemmKind k, GemmArgs a, int splits, hipStream_t st);

// Bt[q, i] = q < r ? B[i, q] : 0, bf16 [rows, r] -> [r_pad, rows].
hipError_t launch_transpose_pad(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t r, int64_t r_pad,
                                hipStream_t st);

// dst[c, q] = q < R ? src[q, c] : 0 (c < C, q < Rpad; row strides lds, ldd):
// src [R, C] bf16 transposed to [C, Rpad] with zero columns R..Rpad.
hipError_t launch_transpose_tile(const uint16_t* src, int64_t lds, int64_t R, int64_t C, uint16_t* dst, int64_t ldd,
                                 int64_t Rpad, hipStream_t st);

// dst[i, j] = j < r ? src[i, j] : 0 for a [rows, r] matrix widened to [rows, r_pad].
hipError_t launch_pad_cols(int elem_bytes, const void* src, void* dst, int64_t rows, int64_t r,
                           int64_t r_pad, hipStream_t st);

// G = R(-angle) dY for rotate-half pairs of 128-wide heads.
hipError_t launch_rope_inverse(int elem_bytes, const void* dY, void* G, int64_t M, int64_t d_out,
                               const int32_t* pos, const float* cosc, const float* sinc, int64_t max_pos,
                               hipStream_t st);

hipError_t launch_rope_cache(int64_t max_pos, int head_dim, double theta, float* cosc, float* sinc,
                             hipStream_t st);

// out = sum over z < splits of part[z] (fixed order).  part[z] is [rows_pad, N]
// fp32.  transpose = false: out[q * N + n]; true: out[n * rows + q]; q < rows.
hipError_t launch_reduce_splits(const float* part, int splits, int64_t rows, int64_t N,
                                int64_t part_stride, bool transpose, float* out, hipStream_t st);

// Several independent launch_reduce_splits / launch_transpose_tile jobs in ONE
// launch (a layer's dA and dB sums, a group's A^T and B^T): the blocks are
// dealt to the jobs in order.  add() checks each job as the single launch
// would and returns hipErrorInvalidValue (job not added) otherwise.
constexpr int kBatchJobsMax = 16;
struct ReduceJob {
  const float* part;
  float* out;
  int64_t rows, N, part_stride;
  int splits, transpose, block0, tiles_n;
};
struct ReduceBatch {
  int n = 0, blocks = 0;
  ReduceJob j[kBatchJobsMax];
  hipError_t add(const float* part, int splits, int64_t rows, int64_t N, int64_t part_stride, bool transpose,
                 float* out);
};
hipError_t launch_reduce_batch(const ReduceBatch& b, hipStream_t st);

struct TransposeJob {
  const uint16_t* src;
  uint16_t* dst;
  int64_t lds, R, C, ldd, Rpad;
  int block0, tiles_c;
};
struct TransposeBatch {
  int n = 0, blocks = 0;
  TransposeJob j[kBatchJobsMax];
  hipError_t add(const uint16_t* src, int64_t lds, int64_t R, int64_t C, uint16_t* dst, int64_t ldd, int64_t Rpad);
};
hipError_t launch_transpose_batch(const TransposeBatch& b, hipStream_t st);

// Per-column scale of a panel: column c takes s[i] for the first i < n with
// c < end[i] (one entry per projection of a group; n = 1 for one projection).
constexpr int kColScaleMax = 8;
struct ColScale {
  int n;
  int64_t end[kColScaleMax];
  float s[kColScaleMax];
};
inline ColScale col_scale(float s) {
  ColScale c{};
  c.n = 1;
  c.end[0] = INT64_MAX;
  c.s[0] = s;
  return c;
}

// Rank-r panel from split partials: v = scale(c) * sum over z < splits of
// part[z][q, c] (fixed order) for q < rows, c < n; written as bf16 to
// out[q * ldo + c] and/or outt[c * ldot + q] (either may be null).
hipError_t launch_panel_reduce(const float* part, int splits, int64_t part_stride, int64_t ldp, int64_t rows,
                               int64_t n, const ColScale& scale, uint16_t* out, int64_t ldo, uint16_t* outt,
                               int64_t ldot, hipStream_t st);

// out [M, N] bf16 (row stride ldo) = fixed-order sum of split partials
// (part[z * part_stride + m * N + n]); with pos != NULL also the RoPE rotation
// of the pairs (n, n + 64) of each 128-wide head (N a multiple of 128; a
// position outside [0, max_pos) gives zeros).
hipError_t launch_split_finish(const float* part, int splits, int64_t part_stride, int64_t M, int64_t N,
                               uint16_t* out, int64_t ldo, const int32_t* pos, const float* cosc, const float* sinc,
                               int64_t max_pos, hipStream_t st);

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// SwiGLU elementwise passes over n elements of bf16 (elem_bytes 2) or fp32:
// H = silu(G) U; dG = dH U silu'(G), dU = dH silu(G); dst += src.
hipError_t launch_swiglu_apply(int elem_bytes, const void* G, const void* U, void* H, int64_t n, hipStream_t st);
hipError_t launch_swiglu_grad(int elem_bytes, const void* dH, const void* G, const void* U, void* dG, void* dU,
                              int64_t n, hipStream_t st);
hipError_t launch_add_into(int elem_bytes, void* dst, const void* src, int64_t n, hipStream_t st);

// out = X with the elements whose keep bit is clear set to 0 (n elements,
// n % 8 == 0, bit b of keep[e] is element 8 e + b).
hipError_t launch_mask_copy(int elem_bytes, const void* X, const uint8_t* keep, void* out, int64_t n,
                            hipStream_t st);
// Philox4x32-10 keep mask of n elements (8 | n): packed bits into keep and/or
// the masked copy of X into out (either may be null; out needs X).
hipError_t launch_dropout_philox(int elem_bytes, const void* X, void* out, uint8_t* keep, int64_t n, uint32_t thr,
                                 uint64_t seed, uint64_t offset, hipStream_t st);

// blocks x 256 threads of the MFMA-rate kernel (iters rounds of 8 MFMAs per
// wave); out [blocks * 256] receives one float per thread.
hipError_t launch_mfma_rate(int iters, int blocks, float* out, hipStream_t st);

// Tiny fp32 problems (tiny.h): forward (bwd false) Y = X W^T + s (X A^T) B^T
// in one launch; backward dX (nullable), dA, dB of it for G in two launches,
// the rank rows s X A^T and s G B going through Ps and Qs (M r floats each).
// Only where tiny_fits holds (else hipErrorInvalidValue).
bool tiny_fits(int64_t M, int64_t K, int64_t N, int64_t r);
hipError_t launch_tiny(bool bwd, const float* X, const float* W, const float* A, const float* B, const float* G,
                       float* Y, float* dX, float* dA, float* dB, float* Ps, float* Qs, int64_t M, int64_t K,
                       int64_t N, int64_t r, float s, hipStream_t st);

// Few-token forward in one launch (skinny.h): Y = X W^T + bf16(s X A^T) B^T,
// mode 0 plain, 1 RoPE (pos / cosc / sinc, N % 128 == 0), bf16 W.  Requires
// 1 <= M <= 64, r % 8 == 0, r <= 64 (skinny_fits).
struct SkinnyArgs;
bool skinny_fits(int64_t M, int64_t K, int64_t N, int64_t r, int mode);
hipError_t launch_skinny_fwd(const SkinnyArgs& a, int mode, hipStream_t st);

// W^T [cols, rows] bf16 from the NF4 codes of W [rows, cols] (cols % 64 == 0,
// rows % 8 == 0), the same values as launch_nf4_dequant.
hipError_t launch_nf4_dequant_t(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                                const float* table16, uint16_t* out, hipStream_t st);

hipError_t launch_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n,
                              const float* table16, uint16_t* out, hipStream_t st);

// Few-token path (few.h), MB = 16-row blocks of tokens (1, 2, 4 or 8): the
// panel partials (Sp + Sq blocks); the backward's panel sums when the stream
// does not fold them; the W stream of the forward (NF4 or bf16 W) or of the
// backward (nblk <= 256 blocks, each a contiguous range of the tiles' stages).
struct FewArgs;
hipError_t launch_few_panel(const FewArgs& a, int MB, hipStream_t st);
hipError_t launch_few_reduce(const FewArgs& a, hipStream_t st);  // backward: P_s, Q_s between the launches
hipError_t launch_few_fwd(const FewArgs& a, int MB, bool nf4, hipStream_t st);
hipError_t launch_few_bwd(const FewArgs& a, int MB, bool nf4, hipStream_t st);

}  // namespace lora
