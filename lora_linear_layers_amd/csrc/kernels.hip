// kernels.hip - gfx950 device code of the fused LoRA linear layer: the GEMM
// instances and the small element-wise kernels around them, plus their
// host-side launchers (internal interface in launch.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>

#include "gemm.h"
#include "gemm_w4.h"
#include "gemm_w4_nt.h"
#include "gemm_w4_nf4.h"
#include "gemm_panel.h"
#include "skinny.h"
#include "tiny.h"
#include "few.h"
#include "launch.h"

namespace lora {

namespace {

template <typename T, int BM, int BN, int WM, int WN, bool B_NN, int EPI, int BL>
hipError_t run(GemmArgs a, int splits, hipStream_t st) {
  a.tiles_m = (int)((a.m_store + BM - 1) / BM);
  const int64_t tiles_n = (a.n_store + BN - 1) / BN;
  const int64_t nblocks = (int64_t)a.tiles_m * tiles_n;
  if (nblocks <= 0 || splits <= 0) return hipSuccess;
  dim3 grid((unsigned)nblocks, 1, (unsigned)splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, B_NN, EPI, BL>), grid, dim3(64 * WM * WN), 0, st,
                     a);
  return hipGetLastError();
}

// Whole-tile launches (every tile inside m and n, the first contraction
// segment a whole number of 64-wide stages, no split, every lane offset of a
// tile below the 1 GiB buffer-resource range) take gemm_w4_nt_kernel (NT) or
// gemm_w4_nn_kernel (NN).
bool whole_tiles(const GemmArgs& a, int splits) {
  const int64_t ld = std::max(std::max(std::max(a.lda1, a.lda2), std::max(a.ldb1, a.ldb2)), a.ldb2u);
  return splits == 1 && a.m_load == a.m_store && a.m_store % w4::BM == 0 && a.n_load == a.n_store &&
         a.n_store % w4::BN == 0 && a.K1 % w4::BK == 0 && ld * 2 * (w4::BM + w4::BK) < (int64_t)w4::BIG;
}

template <bool B_NN, int EPI>
hipError_t run_whole(GemmArgs a, hipStream_t st) {
  static_assert(!B_NN || EPI == EPI_STORE, "the NN kernel stores");
  const int64_t tiles_m = a.m_store / w4::BM;
  const int64_t nblocks = tiles_m * (a.n_store / w4::BN);
  if (nblocks <= 0) return hipSuccess;
  if (nblocks > INT32_MAX) return hipErrorInvalidValue;  // one block per tile, a 1D grid
  a.tiles_m = (int)tiles_m;
  if constexpr (B_NN)
    hipLaunchKernelGGL((gemm_w4_nn_kernel<2>), dim3((unsigned)nblocks), dim3(w4::NT), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_w4_nt_kernel<EPI>), dim3((unsigned)nblocks), dim3(w4::NT), 0, st, a);
  return hipGetLastError();
}

// rank-r panel split partials (K1 only, at most 256 panel columns): one
// 128-row tile per block and split, every column in the tile
hipError_t run_panel(GemmArgs a, int splits, hipStream_t st) {
  constexpr int BM = PANEL_BM;
  a.tiles_m = (int)((a.m_store + BM - 1) / BM);
  const int64_t nblocks = (int64_t)a.tiles_m * splits;
  if (nblocks <= 0) return hipSuccess;
  if (a.n_store <= 64)
    hipLaunchKernelGGL((panel_dma_kernel<BM, 64>), dim3((unsigned)nblocks), dim3(pdma::NT), 0, st, a);
  else if (a.n_store <= 128)
    hipLaunchKernelGGL((panel_dma_kernel<BM, 128>), dim3((unsigned)nblocks), dim3(pdma::NT), 0, st, a);
  else
    hipLaunchKernelGGL((panel_dma_kernel<BM, 256>), dim3((unsigned)nblocks), dim3(pdma::NT), 0, st, a);
  return hipGetLastError();
}

// token-split partials of dA / dB for up to 128 rows: every row in a
// 256-column tile, one block per tile and split
hipError_t run_splitnn(GemmArgs a, int splits, hipStream_t st) {
  const int64_t tiles_n = (a.n_store + sdma::BN - 1) / sdma::BN;
  if (tiles_n <= 0 || splits <= 0) return hipSuccess;
  const dim3 grid((unsigned)tiles_n, (unsigned)splits);
  // up to 64 rows and more blocks than CUs: two blocks per CU (80 KB rings of
  // 2 stages), else one per CU with every stage the LDS holds
  if (a.m_store <= 64 && tiles_n * splits > 256)
    hipLaunchKernelGGL((splitnn_dma_kernel<64, 2>), grid, dim3(sdma::NT), 0, st, a);
  else if (a.m_store <= 64)
    hipLaunchKernelGGL((splitnn_dma_kernel<64, 4>), grid, dim3(sdma::NT), 0, st, a);
  else
    hipLaunchKernelGGL((splitnn_dma_kernel<128, 3>), grid, dim3(sdma::NT), 0, st, a);
  return hipGetLastError();
}

bool splitnn_fits(const GemmArgs& a) {
  return a.K2 == 0 && a.m_store > 0 && a.m_store <= 128 && a.m_load <= a.m_store && a.n_load == a.n_store &&
         (a.k_split + sdma::BK) * a.ldb1 * 2 + a.n_store * 2 < (int64_t)w4::BIG &&
         a.lda1 * 2 * 128 < (int64_t)w4::BIG;
}

bool panel_fits(const GemmArgs& a) {
  return a.K2 == 0 && a.n_load <= a.n_store && panel_dma_fits(a.n_store, a.lda1, a.ldb1);
}

using bf = uint16_t;

}  // namespace

bool whole_ld_fits(int64_t ld) { return ld * 2 * (w4::BM + w4::BK) < (int64_t)w4::BIG; }

bool panel_dma_fits(int64_t n_store, int64_t lda, int64_t ldb) {
  const int64_t ld = std::max(lda, ldb);
  return n_store <= 256 && ld * 2 * 256 < (int64_t)w4::BIG;
}

TileShape gemm_tile(GemmKind k) {
  switch (k) {
    case G_BF16_BIG_NT_STORE:
    case G_BF16_BIG_NT_ROPE:
    case G_BF16_BIG_NN_STORE:
    case G_NF4_BIG_NT_STORE:
    case G_NF4_BIG_NN_STORE:
      return {256, 256};
    case G_BF16_MED_NT_STORE:
    case G_BF16_MED_NT_ROPE:
    case G_BF16_MED_NN_STORE:
    case G_NF4_MED_NT_STORE:
    case G_NF4_MED_NN_STORE:
    case G_BF16_MED_NT_PARTIAL:
    case G_BF16_MED_NN_PARTIAL:
    case G_NF4_MED_NT_PARTIAL:
    case G_NF4_MED_NN_PARTIAL:
    case G_BF16_MED_NN_ADD:
    case G_BF16_MED_NN_ADD_MASKED:
      return {128, 128};
    case G_F32_PANEL_NT_STORE:
    case G_F32_PANEL_NT_STORE_T:
    case G_F32_PANEL_NN_BOTH:
      return {64, 64};
    case G_BF16_SPLIT_NN_PARTIAL:
    case G_F32_SPLIT_NN_PARTIAL:
      return {64, 256};
    case G_BF16_WHOLE_SWIGLU:
    case G_BF16_WHOLE_GROUP:
    case G_NF4_WHOLE_NT_STORE:
      return {256, 256};
    case G_BF16_PANEL_SPLIT_NT:
      return {256, 64};
    case G_F32_NT_STORE:
    case G_F32_NT_ROPE:
    case G_F32_NN_STORE:
    case G_F32_NN_ADD:
    case G_F32_NN_ADD_MASKED:
      return {64, 128};
    default:
      return {0, 0};
  }
}

hipError_t launch_gemm(GemmKind k, GemmArgs a, int splits, hipStream_t st) {
  switch (k) {
    case G_BF16_BIG_NT_STORE:
      if (whole_tiles(a, splits)) return run_whole<false, EPI_STORE>(a, st);
      return run<bf, 256, 256, 2, 4, false, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_BF16_BIG_NT_ROPE:
      if (whole_tiles(a, splits)) return run_whole<false, EPI_ROPE>(a, st);
      return run<bf, 256, 256, 2, 2, false, EPI_ROPE, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NT_STORE: return run<bf, 128, 128, 4, 1, false, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NT_ROPE: return run<bf, 128, 128, 4, 1, false, EPI_ROPE, BL_PLAIN>(a, splits, st);
    case G_BF16_BIG_NN_STORE:
      if (whole_tiles(a, splits)) return run_whole<true, EPI_STORE>(a, st);
      return run<bf, 256, 256, 2, 4, true, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NN_STORE: return run<bf, 128, 128, 4, 1, true, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_NF4_BIG_NT_STORE: return run<bf, 256, 256, 2, 4, false, EPI_STORE, BL_NF4>(a, splits, st);
    case G_NF4_MED_NT_STORE: return run<bf, 128, 128, 4, 1, false, EPI_STORE, BL_NF4>(a, splits, st);
    case G_NF4_BIG_NN_STORE: return run<bf, 256, 256, 2, 4, true, EPI_STORE, BL_NF4>(a, splits, st);
    case G_NF4_MED_NN_STORE: return run<bf, 128, 128, 4, 1, true, EPI_STORE, BL_NF4>(a, splits, st);
    case G_BF16_SPLIT_NN_PARTIAL:
      if (splitnn_fits(a)) return run_splitnn(a, splits, st);
      return run<bf, 64, 256, 1, 4, true, EPI_PARTIAL, BL_PLAIN>(a, splits, st);
    case G_F32_NT_STORE: return run<float, 64, 128, 4, 1, false, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_F32_NT_ROPE: return run<float, 64, 128, 4, 1, false, EPI_ROPE, BL_PLAIN>(a, splits, st);
    case G_F32_NN_STORE: return run<float, 64, 128, 4, 1, true, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_F32_PANEL_NT_STORE: return run<float, 64, 64, 2, 2, false, EPI_STORE, BL_PLAIN>(a, splits, st);
    case G_F32_PANEL_NT_STORE_T: return run<float, 64, 64, 2, 2, false, EPI_STORE_T, BL_PLAIN>(a, splits, st);
    case G_F32_PANEL_NN_BOTH: return run<float, 64, 64, 2, 2, true, EPI_STORE_BOTH, BL_PLAIN>(a, splits, st);
    case G_F32_SPLIT_NN_PARTIAL: return run<float, 64, 256, 1, 4, true, EPI_PARTIAL, BL_PLAIN>(a, splits, st);
    case G_BF16_PANEL_SPLIT_NT:
      if (panel_fits(a)) return run_panel(a, splits, st);
      if (a.n_src > 0) return hipErrorInvalidValue;  // row sources: the DMA kernel only
      return run<bf, 256, 64, 4, 1, false, EPI_PARTIAL, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NT_PARTIAL: return run<bf, 128, 128, 4, 1, false, EPI_PARTIAL, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NN_PARTIAL: return run<bf, 128, 128, 4, 1, true, EPI_PARTIAL, BL_PLAIN>(a, splits, st);
    case G_NF4_MED_NT_PARTIAL: return run<bf, 128, 128, 4, 1, false, EPI_PARTIAL, BL_NF4>(a, splits, st);
    case G_NF4_MED_NN_PARTIAL: return run<bf, 128, 128, 4, 1, true, EPI_PARTIAL, BL_NF4>(a, splits, st);
    case G_BF16_MED_NN_ADD: return run<bf, 128, 128, 4, 1, true, EPI_ADD, BL_PLAIN>(a, splits, st);
    case G_BF16_WHOLE_SWIGLU:
      if (!whole_tiles(a, splits)) return hipErrorInvalidValue;
      return run_whole<false, EPI_SWIGLU>(a, st);
    case G_BF16_WHOLE_GROUP:
      // the members' tile ranges must tile the launch exactly
      if (!whole_tiles(a, splits) || a.n_mem < 1 || a.n_mem > kGroupGemmMax || a.mem_tile0[0] != 0 ||
          (int64_t)a.mem_tile0[a.n_mem] != (a.m_store / w4::BM) * (a.n_store / w4::BN))
        return hipErrorInvalidValue;
      return run_whole<false, EPI_GROUP>(a, st);
    case G_NF4_WHOLE_NT_STORE: {
      // whole tiles, codes and absmax present, every lane offset of a tile's
      // codes and absmax below the buffer-resource range
      if (!whole_tiles(a, splits) || !a.codes || !a.absmax || a.K1 < w4::BK || a.codes_ld * 2 != a.K1 ||
          a.blocks_per_row * w4::BK != a.K1 || a.codes_ld * (w4::BN + 1) >= (int64_t)w4::BIG)
        return hipErrorInvalidValue;
      const int64_t tiles_m = a.m_store / w4::BM;
      const int64_t nblocks = tiles_m * (a.n_store / w4::BN);
      if (nblocks <= 0) return hipSuccess;
      if (nblocks > INT32_MAX) return hipErrorInvalidValue;
      a.tiles_m = (int)tiles_m;
      hipLaunchKernelGGL(gemm_w4_nf4_kernel, dim3((unsigned)nblocks), dim3(w4::NT), 0, st, a);
      return hipGetLastError();
    }
    case G_F32_NN_ADD: return run<float, 64, 128, 4, 1, true, EPI_ADD, BL_PLAIN>(a, splits, st);
    case G_BF16_MED_NN_ADD_MASKED: return run<bf, 128, 128, 4, 1, true, EPI_ADD_MASKED, BL_PLAIN>(a, splits, st);
    case G_F32_NN_ADD_MASKED: return run<float, 64, 128, 4, 1, true, EPI_ADD_MASKED, BL_PLAIN>(a, splits, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// small kernels
// ---------------------------------------------------------------------------

// Bt[q, i] = q < r ? B[i, q] : 0 for B [rows, r] -> Bt [r_pad, rows].
__global__ void transpose_pad_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t rows,
                                     int64_t r, int64_t r_pad) {
  const int64_t n = rows * r_pad;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = e / rows, i = e - q * rows;
    dst[e] = q < r ? src[i * r + q] : (uint16_t)0;
  }
}

// dst[c, q] = q < R ? src[q, c] : 0 for c < C, q < Rpad: a bf16 transpose
// through a 64 x 64 LDS tile, 16-byte loads and stores (C and Rpad multiples
// of 8).
// One 64 x 64 tile of dst[c, q] = q < R ? src[q, c] : 0, columns c0 .., rows
// of the transpose q0 ...
// The tile row rr holds its 16-byte chunk ch at chunk ch ^ ((rr >> 3) & 7): the
// column reads below (rows 8 qc + 2 k, qc < 8, of one column) then fall in
// 8 different chunks, so in different banks (with a plain or padded
// 16-byte-aligned row they share one bank, 8 ways)
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ src, int64_t lds, int64_t R, int64_t C,
                                               uint16_t* __restrict__ dst, int64_t ldd, int64_t Rpad, int64_t c0,
                                               int64_t q0, uint16_t (*t)[64]) {
  for (int e = threadIdx.x; e < 512; e += 256) {
    const int rr = e >> 3, ch = e & 7;
    const int64_t q = q0 + rr, c = c0 + 8 * ch;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < R && c < C) v = *reinterpret_cast<const u32x4*>(src + q * lds + c);
    *reinterpret_cast<u32x4*>(&t[rr][8 * (ch ^ ((rr >> 3) & 7))]) = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 512; e += 256) {
    const int cc = e >> 3, qc = e & 7;
    const int64_t c = c0 + cc, q = q0 + 8 * qc;
    if (c >= C || q >= Rpad) continue;
    const int col = 8 * ((cc >> 3) ^ qc) + (cc & 7);  // rows 8 qc .. 8 qc + 7 share (row >> 3) & 7 = qc
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (uint32_t)t[8 * qc + 2 * k][col] | ((uint32_t)t[8 * qc + 2 * k + 1][col] << 16);
    *reinterpret_cast<u32x4*>(dst + c * ldd + q) = o;
  }
}

__global__ void __launch_bounds__(256) transpose_tile_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                             int64_t R, int64_t C, uint16_t* __restrict__ dst,
                                                             int64_t ldd, int64_t Rpad) {
  __shared__ __attribute__((aligned(16))) uint16_t t[64][64];
  transpose_tile(src, lds, R, C, dst, ldd, Rpad, (int64_t)blockIdx.x * 64, (int64_t)blockIdx.y * 64, t);
}

// the jobs' tiles, job by job (the job of a block: a scalar search)
__global__ void __launch_bounds__(256) transpose_batch_kernel(const TransposeBatch b) {
  __shared__ __attribute__((aligned(16))) uint16_t t[64][64];
  const int blk = blockIdx.x;
  int g = 0;
  for (int i = 1; i < b.n; ++i) g = blk >= b.j[i].block0 ? i : g;
  const TransposeJob& J = b.j[g];
  const int lb = blk - J.block0;
  transpose_tile(J.src, J.lds, J.R, J.C, J.dst, J.ldd, J.Rpad, (int64_t)(lb % J.tiles_c) * 64,
                 (int64_t)(lb / J.tiles_c) * 64, t);
}

hipError_t TransposeBatch::add(const uint16_t* src, int64_t lds, int64_t R, int64_t C, uint16_t* dst, int64_t ldd,
                               int64_t Rpad) {
  if (R <= 0 || C <= 0 || Rpad <= 0) return hipSuccess;  // nothing to do
  if (n >= kBatchJobsMax || C % 8 || Rpad % 8 || Rpad < R || ldd < Rpad || ldd % 8 || lds % 8)
    return hipErrorInvalidValue;
  const int64_t tc = (C + 63) / 64, tiles = tc * ((Rpad + 63) / 64);
  if (blocks + tiles > INT32_MAX) return hipErrorInvalidValue;
  j[n] = TransposeJob{src, dst, lds, R, C, ldd, Rpad, blocks, (int)tc};
  blocks += (int)tiles;
  ++n;
  return hipSuccess;
}

hipError_t launch_transpose_batch(const TransposeBatch& b, hipStream_t st) {
  if (b.n == 0 || b.blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_batch_kernel, dim3((unsigned)b.blocks), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_transpose_tile(const uint16_t* src, int64_t lds, int64_t R, int64_t C, uint16_t* dst, int64_t ldd,
                                 int64_t Rpad, hipStream_t st) {
  if (R <= 0 || C <= 0 || Rpad <= 0) return hipSuccess;
  if (C % 8 || Rpad % 8 || Rpad < R || ldd < Rpad || ldd % 8 || lds % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((Rpad + 63) / 64));
  hipLaunchKernelGGL(transpose_tile_kernel, grid, dim3(256), 0, st, src, lds, R, C, dst, ldd, Rpad);
  return hipGetLastError();
}

template <typename T>
__global__ void pad_cols_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows, int64_t r,
                                int64_t r_pad) {
  const int64_t n = rows * r_pad;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = e / r_pad, j = e - i * r_pad;
    dst[e] = j < r ? src[i * r + j] : T(0);
  }
}

static unsigned grid_for(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  if (b > 65535 * 4) b = 65535 * 4;
  return (unsigned)(b > 0 ? b : 1);
}

hipError_t launch_transpose_pad(const uint16_t* src, uint16_t* dst, int64_t rows, int64_t r, int64_t r_pad,
                                hipStream_t st) {
  const int64_t n = rows * r_pad;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, src, dst, rows, r, r_pad);
  return hipGetLastError();
}

hipError_t launch_pad_cols(int elem_bytes, const void* src, void* dst, int64_t rows, int64_t r, int64_t r_pad,
                           hipStream_t st) {
  const int64_t n = rows * r_pad;
  if (n <= 0) return hipSuccess;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(pad_cols_kernel<uint16_t>, dim3(grid_for(n, 256)), dim3(256), 0, st,
                       (const uint16_t*)src, (uint16_t*)dst, rows, r, r_pad);
  else
    hipLaunchKernelGGL(pad_cols_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, (const float*)src,
                       (float*)dst, rows, r, r_pad);
  return hipGetLastError();
}

template <typename T>
__device__ __forceinline__ float ld_as_f32(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 2)
    return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
  else
    return p[i];
}

// One thread per (row t, head h, group of 8 frequencies): rotates the pairs
// (h*128 + f, h*128 + f + 64) for f in [8q, 8q+8) by the negated angle:
//   g1 = y1 cos + y2 sin,   g2 = y2 cos - y1 sin.
// Every access is a 16-byte vector: the 8 values of each half of the pair
// group (bf16: one vector, fp32: two), their 8 cos and 8 sin; the 8 lanes of
// a (row, head) read and write whole 128-byte pieces.  (Scalar 2-byte
// accesses, one frequency per instruction, ran this pass at 1.5 TB/s.)
template <typename T>
__global__ void rope_inverse_kernel(const T* __restrict__ dY, T* __restrict__ G, int64_t M, int64_t d_out,
                                    const int32_t* __restrict__ pos, const float* __restrict__ cosc,
                                    const float* __restrict__ sinc, int64_t max_pos) {
  const int64_t heads = d_out / 128;
  const int64_t n = M * heads * 8;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t q = e & 7;
    const int64_t th = e >> 3;
    const int64_t t = th / heads, h = th - t * heads;
    const int32_t ps = pos[t];
    const bool ok = rope_pos_ok(ps, max_pos);
    const int64_t prow = (ok ? (int64_t)ps * 64 : 0) + 8 * q;
    const int64_t i1 = t * d_out + h * 128 + 8 * q, i2 = i1 + 64;
    float c[8], sn[8], y1[8], y2[8];
    {
      const float4 c0 = *reinterpret_cast<const float4*>(cosc + prow);
      const float4 c1 = *reinterpret_cast<const float4*>(cosc + prow + 4);
      const float4 s0 = *reinterpret_cast<const float4*>(sinc + prow);
      const float4 s1 = *reinterpret_cast<const float4*>(sinc + prow + 4);
      const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        c[u] = ok ? cv[u] : 0.f;
        sn[u] = ok ? sv[u] : 0.f;
      }
    }
    if constexpr (sizeof(T) == 2) {
      const uint4 a = *reinterpret_cast<const uint4*>(dY + i1);
      const uint4 b = *reinterpret_cast<const uint4*>(dY + i2);
      const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y1[2 * k] = __builtin_bit_cast(float, av[k] << 16);
        y1[2 * k + 1] = __builtin_bit_cast(float, av[k] & 0xffff0000u);
        y2[2 * k] = __builtin_bit_cast(float, bv[k] << 16);
        y2[2 * k + 1] = __builtin_bit_cast(float, bv[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(dY + i1 + 4 * k);
        const float4 b = *reinterpret_cast<const float4*>(dY + i2 + 4 * k);
        y1[4 * k] = a.x; y1[4 * k + 1] = a.y; y1[4 * k + 2] = a.z; y1[4 * k + 3] = a.w;
        y2[4 * k] = b.x; y2[4 * k + 1] = b.y; y2[4 * k + 2] = b.z; y2[4 * k + 3] = b.w;
      }
    }
    float g1[8], g2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      g1[u] = y1[u] * c[u] + y2[u] * sn[u];
      g2[u] = y2[u] * c[u] - y1[u] * sn[u];
    }
    if constexpr (sizeof(T) == 2) {
      uint4 o1, o2;
      o1.x = pack_bf16x2(g1[0], g1[1]); o1.y = pack_bf16x2(g1[2], g1[3]);
      o1.z = pack_bf16x2(g1[4], g1[5]); o1.w = pack_bf16x2(g1[6], g1[7]);
      o2.x = pack_bf16x2(g2[0], g2[1]); o2.y = pack_bf16x2(g2[2], g2[3]);
      o2.z = pack_bf16x2(g2[4], g2[5]); o2.w = pack_bf16x2(g2[6], g2[7]);
      *reinterpret_cast<uint4*>(G + i1) = o1;
      *reinterpret_cast<uint4*>(G + i2) = o2;
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        *reinterpret_cast<float4*>(G + i1 + 4 * k) = make_float4(g1[4 * k], g1[4 * k + 1], g1[4 * k + 2], g1[4 * k + 3]);
        *reinterpret_cast<float4*>(G + i2 + 4 * k) = make_float4(g2[4 * k], g2[4 * k + 1], g2[4 * k + 2], g2[4 * k + 3]);
      }
    }
  }
}

hipError_t launch_rope_inverse(int elem_bytes, const void* dY, void* G, int64_t M, int64_t d_out,
                               const int32_t* pos, const float* cosc, const float* sinc, int64_t max_pos,
                               hipStream_t st) {
  const int64_t n = M * (d_out / 128) * 8;
  if (n <= 0) return hipSuccess;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(rope_inverse_kernel<uint16_t>, dim3(grid_for(n, 256)), dim3(256), 0, st,
                       (const uint16_t*)dY, (uint16_t*)G, M, d_out, pos, cosc, sinc, max_pos);
  else
    hipLaunchKernelGGL(rope_inverse_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, (const float*)dY,
                       (float*)G, M, d_out, pos, cosc, sinc, max_pos);
  return hipGetLastError();
}

__global__ void rope_cache_kernel(int64_t max_pos, int half, double theta, float* __restrict__ cosc,
                                  float* __restrict__ sinc) {
  const int64_t n = max_pos * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = e / half;
    const int i = (int)(e - p * half);
    const double inv_freq = pow(theta, -(2.0 * i) / (2.0 * half));
    const double a = (double)p * inv_freq;
    cosc[e] = (float)cos(a);
    sinc[e] = (float)sin(a);
  }
}

hipError_t launch_rope_cache(int64_t max_pos, int head_dim, double theta, float* cosc, float* sinc,
                             hipStream_t st) {
  const int64_t n = max_pos * (head_dim / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_cache_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, max_pos, head_dim / 2, theta,
                     cosc, sinc);
  return hipGetLastError();
}

constexpr int kMaxSplits = 64;

// Sum over z < splits of the float4 at src + z stride, in split order, with
// the loads of up to 8 splits issued before their adds.
__device__ __forceinline__ float4 sum_splits(const float* __restrict__ src, int splits, int64_t stride) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z0 = 0; z0 < splits; z0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int z = z0 + u < splits ? z0 + u : splits - 1;
      v[u] = *reinterpret_cast<const float4*>(src + (int64_t)z * stride);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (z0 + u >= splits) break;
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  return acc;
}

// out[q, c] (transpose: out[c, q]) = sum over z < splits of part[z][q, c],
// in split order, for q < rows, c < N (N a multiple of 4).  A block covers
// 16 rows x 64 columns (from q0, c0), thread t columns 4 (t & 15) .. +3 of
// row t >> 4, with the float4 loads of up to 8 splits in flight before their
// sums.  The transposed store goes through an LDS tile so that consecutive
// threads write consecutive q.
__device__ __forceinline__ void reduce_tile(const float* __restrict__ part, int splits, int64_t rows, int64_t N,
                                            int64_t part_stride, int transpose, float* __restrict__ out,
                                            int64_t c0, int64_t q0, float (*tile)[65]) {
  const int tid = threadIdx.x;
  const int cl = 4 * (tid & 15), rl = tid >> 4;
  const int64_t c = c0 + cl, q = q0 + rl;
  const bool ok = c < N && q < rows;
  // past the end: a valid element is read and nothing is stored
  const float* src = part + (ok ? q * N + c : 0);
  const float4 acc = sum_splits(src, splits, part_stride);
  if (!transpose) {
    if (ok) {
      float* d = out + q * N + c;
      d[0] = acc.x;
      d[1] = acc.y;
      d[2] = acc.z;
      d[3] = acc.w;
    }
    return;
  }
  float* trow = &tile[rl][cl];
  trow[0] = acc.x;
  trow[1] = acc.y;
  trow[2] = acc.z;
  trow[3] = acc.w;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * 256 + tid;
    const int cc = idx >> 4, qq = idx & 15;
    const int64_t qg = q0 + qq, cg = c0 + cc;
    if (qg < rows && cg < N) out[cg * rows + qg] = tile[qq][cc];
  }
}

__global__ void __launch_bounds__(256) reduce_splits_kernel(const float* __restrict__ part, int splits,
                                                            int64_t rows, int64_t N, int64_t part_stride,
                                                            int transpose, float* __restrict__ out) {
  __shared__ float tile[16][65];
  reduce_tile(part, splits, rows, N, part_stride, transpose, out, (int64_t)blockIdx.x * 64,
              (int64_t)blockIdx.y * 16, tile);
}

// the jobs' tiles, job by job (the job of a block: a scalar search)
__global__ void __launch_bounds__(256) reduce_batch_kernel(const ReduceBatch b) {
  __shared__ float tile[16][65];
  const int blk = blockIdx.x;
  int g = 0;
  for (int i = 1; i < b.n; ++i) g = blk >= b.j[i].block0 ? i : g;
  const ReduceJob& J = b.j[g];
  const int lb = blk - J.block0;
  reduce_tile(J.part, J.splits, J.rows, J.N, J.part_stride, J.transpose, J.out, (int64_t)(lb % J.tiles_n) * 64,
              (int64_t)(lb / J.tiles_n) * 16, tile);
}

hipError_t ReduceBatch::add(const float* part, int splits, int64_t rows, int64_t N, int64_t part_stride,
                            bool transpose, float* out) {
  if (rows <= 0 || N <= 0) return hipSuccess;  // nothing to do
  if (n >= kBatchJobsMax || splits < 1 || splits > kMaxSplits || N % 4 || part_stride % 4 ||
      reinterpret_cast<uintptr_t>(part) % 16)
    return hipErrorInvalidValue;
  const int64_t tn = (N + 63) / 64, tiles = tn * ((rows + 15) / 16);
  if (blocks + tiles > INT32_MAX) return hipErrorInvalidValue;
  j[n] = ReduceJob{part, out, rows, N, part_stride, splits, transpose ? 1 : 0, blocks, (int)tn};
  blocks += (int)tiles;
  ++n;
  return hipSuccess;
}

hipError_t launch_reduce_batch(const ReduceBatch& b, hipStream_t st) {
  if (b.n == 0 || b.blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_batch_kernel, dim3((unsigned)b.blocks), dim3(256), 0, st, b);
  return hipGetLastError();
}

hipError_t launch_reduce_splits(const float* part, int splits, int64_t rows, int64_t N, int64_t part_stride,
                                bool transpose, float* out, hipStream_t st) {
  if (rows <= 0 || N <= 0) return hipSuccess;
  if (splits < 1 || splits > kMaxSplits || N % 4 || part_stride % 4 ||
      reinterpret_cast<uintptr_t>(part) % 16)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((rows + 15) / 16));
  hipLaunchKernelGGL(reduce_splits_kernel, grid, dim3(256), 0, st, part, splits, rows, N, part_stride,
                     transpose ? 1 : 0, out);
  return hipGetLastError();
}

// Outputs of a contraction-split GEMM (few tokens): y[m, n] = sum over
// z < splits of part[z][m, n] in split order, then for q/k projections the
// RoPE rotation of the pairs (n, n + 64) of each 128-wide head (cos/sin row
// positions[m]), stored as bf16.  One thread per 4 consecutive columns (with
// RoPE: 4 columns of a head's first half and their 4 partners).
template <bool ROPE>
__global__ void __launch_bounds__(256) split_finish_kernel(const float* __restrict__ part, int splits,
                                                           int64_t part_stride, int64_t M, int64_t N,
                                                           uint16_t* __restrict__ out, int64_t ldo,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ cosc,
                                                           const float* __restrict__ sinc, int64_t max_pos) {
  const int64_t per_row = ROPE ? N / 8 : N / 4;
  const int64_t items = M * per_row;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < items; e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = e / per_row, q = e - m * per_row;
    const int64_t c = ROPE ? (q >> 4) * 128 + (q & 15) * 4 : q * 4;
    const float* src = part + m * N + c;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    for (int z = 0; z < splits; ++z) {
      const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)z * part_stride);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
      if constexpr (ROPE) {
        const float4 u = *reinterpret_cast<const float4*>(src + 64 + (int64_t)z * part_stride);
        b.x += u.x; b.y += u.y; b.z += u.z; b.w += u.w;
      }
    }
    uint16_t* dst = out + m * ldo + c;
    if constexpr (ROPE) {
      const int32_t ps = pos[m];
      const bool ok = rope_pos_ok(ps, max_pos);
      const int64_t prow = (int64_t)ps * 64 + (c & 127);
      const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 cs = ok ? *reinterpret_cast<const float4*>(cosc + prow) : zero;
      const float4 sn = ok ? *reinterpret_cast<const float4*>(sinc + prow) : zero;
      const float y1[4] = {a.x * cs.x - b.x * sn.x, a.y * cs.y - b.y * sn.y, a.z * cs.z - b.z * sn.z,
                           a.w * cs.w - b.w * sn.w};
      const float y2[4] = {b.x * cs.x + a.x * sn.x, b.y * cs.y + a.y * sn.y, b.z * cs.z + a.z * sn.z,
                           b.w * cs.w + a.w * sn.w};
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]));
      *reinterpret_cast<uint2*>(dst + 64) = make_uint2(pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]));
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
    }
  }
}

hipError_t launch_split_finish(const float* part, int splits, int64_t part_stride, int64_t M, int64_t N,
                               uint16_t* out, int64_t ldo, const int32_t* pos, const float* cosc, const float* sinc,
                               int64_t max_pos, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (splits < 1 || splits > kMaxSplits || N % 8 || ldo % 4 || part_stride % 4) return hipErrorInvalidValue;
  if (pos) {
    if (N % 128) return hipErrorInvalidValue;
    const int64_t items = M * (N / 8);
    hipLaunchKernelGGL(split_finish_kernel<true>, dim3(grid_for(items, 256)), dim3(256), 0, st, part, splits,
                       part_stride, M, N, out, ldo, pos, cosc, sinc, max_pos);
  } else {
    const int64_t items = M * (N / 4);
    hipLaunchKernelGGL(split_finish_kernel<false>, dim3(grid_for(items, 256)), dim3(256), 0, st, part, splits,
                       part_stride, M, N, out, ldo, pos, cosc, sinc, max_pos);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU elementwise passes (gate/up pairs whose shapes the fused whole-tile
// epilogue does not cover, and the backward): fp32 arithmetic on T values,
// silu(z) = z / (1 + e^-z), sigmoid s = 1 / (1 + e^-z).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, int64_t i) {
  if constexpr (sizeof(T) == 2)
    return static_cast<float>(__builtin_bit_cast(__bf16, reinterpret_cast<const uint16_t*>(p)[i]));
  else
    return p[i];
}

template <typename T>
__device__ __forceinline__ void st_elem(T* p, int64_t i, float v) {
  if constexpr (sizeof(T) == 2)
    reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
  else
    p[i] = v;
}

// H = silu(G) * U
template <typename T>
__global__ void swiglu_apply_kernel(const T* __restrict__ G, const T* __restrict__ U, T* __restrict__ H, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const float g = ld_elem(G, e), u = ld_elem(U, e);
    st_elem(H, e, g / (1.f + __expf(-g)) * u);
  }
}

// dG = dH U s (1 + G (1 - s)), dU = dH G s, s = sigmoid(G)
template <typename T>
__global__ void swiglu_grad_kernel(const T* __restrict__ dH, const T* __restrict__ G, const T* __restrict__ U,
                                   T* __restrict__ dG, T* __restrict__ dU, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const float h = ld_elem(dH, e), g = ld_elem(G, e), u = ld_elem(U, e);
    const float sg = 1.f / (1.f + __expf(-g));
    st_elem(dG, e, h * u * sg * (1.f + g * (1.f - sg)));
    st_elem(dU, e, h * g * sg);
  }
}

// dst += src
template <typename T>
__global__ void add_into_kernel(T* __restrict__ dst, const T* __restrict__ src, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
    st_elem(dst, e, ld_elem(dst, e) + ld_elem(src, e));
}

// bf16 forms of the three kernels above for n a multiple of 8 and 16-byte
// aligned arrays: 8 elements per thread and iteration through 16-byte
// accesses (2-byte accesses leave these HBM streams far below the memory's
// rate), the same arithmetic per element.
__device__ __forceinline__ void unpack_bf16x8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = __builtin_bit_cast(float, v[k] << 16);
    f[2 * k + 1] = __builtin_bit_cast(float, v[k] & 0xFFFF0000u);
  }
}

__global__ void swiglu_apply_bf16x8_kernel(const u32x4* __restrict__ G, const u32x4* __restrict__ U,
                                           u32x4* __restrict__ H, int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    float g[8], u[8];
    unpack_bf16x8(G[e], g);
    unpack_bf16x8(U[e], u);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = g[i] / (1.f + __expf(-g[i])) * u[i];
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
    H[e] = o;
  }
}

__global__ void swiglu_grad_bf16x8_kernel(const u32x4* __restrict__ dH, const u32x4* __restrict__ G,
                                          const u32x4* __restrict__ U, u32x4* __restrict__ dG,
                                          u32x4* __restrict__ dU, int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    float h[8], g[8], u[8];
    unpack_bf16x8(dH[e], h);
    unpack_bf16x8(G[e], g);
    unpack_bf16x8(U[e], u);
    float a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = 1.f / (1.f + __expf(-g[i]));
      a[i] = h[i] * u[i] * sg * (1.f + g[i] * (1.f - sg));
      b[i] = h[i] * g[i] * sg;
    }
    u32x4 og, ou;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      og[k] = pack_bf16x2(a[2 * k], a[2 * k + 1]);
      ou[k] = pack_bf16x2(b[2 * k], b[2 * k + 1]);
    }
    dG[e] = og;
    dU[e] = ou;
  }
}

__global__ void add_into_bf16x8_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    float a[8], b[8];
    unpack_bf16x8(dst[e], a);
    unpack_bf16x8(src[e], b);
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(a[2 * k] + b[2 * k], a[2 * k + 1] + b[2 * k + 1]);
    dst[e] = o;
  }
}

static bool vec8_ok(int elem_bytes, int64_t n, std::initializer_list<const void*> ps) {
  if (elem_bytes != 2 || n % 8) return false;
  for (const void* q : ps)
    if (reinterpret_cast<uintptr_t>(q) % 16) return false;
  return true;
}

hipError_t launch_swiglu_apply(int elem_bytes, const void* G, const void* U, void* H, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (vec8_ok(elem_bytes, n, {G, U, H}))
    hipLaunchKernelGGL(swiglu_apply_bf16x8_kernel, dim3(grid_for(n / 8, 256)), dim3(256), 0, st, (const u32x4*)G,
                       (const u32x4*)U, (u32x4*)H, n / 8);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(swiglu_apply_kernel<__bf16>, dim3(grid_for(n, 256)), dim3(256), 0, st,
                       (const __bf16*)G, (const __bf16*)U, (__bf16*)H, n);
  else
    hipLaunchKernelGGL(swiglu_apply_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, (const float*)G,
                       (const float*)U, (float*)H, n);
  return hipGetLastError();
}

hipError_t launch_swiglu_grad(int elem_bytes, const void* dH, const void* G, const void* U, void* dG, void* dU,
                              int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (vec8_ok(elem_bytes, n, {dH, G, U, dG, dU}))
    hipLaunchKernelGGL(swiglu_grad_bf16x8_kernel, dim3(grid_for(n / 8, 256)), dim3(256), 0, st, (const u32x4*)dH,
                       (const u32x4*)G, (const u32x4*)U, (u32x4*)dG, (u32x4*)dU, n / 8);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(swiglu_grad_kernel<__bf16>, dim3(grid_for(n, 256)), dim3(256), 0, st, (const __bf16*)dH,
                       (const __bf16*)G, (const __bf16*)U, (__bf16*)dG, (__bf16*)dU, n);
  else
    hipLaunchKernelGGL(swiglu_grad_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, (const float*)dH,
                       (const float*)G, (const float*)U, (float*)dG, (float*)dU, n);
  return hipGetLastError();
}

hipError_t launch_add_into(int elem_bytes, void* dst, const void* src, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (vec8_ok(elem_bytes, n, {dst, src}))
    hipLaunchKernelGGL(add_into_bf16x8_kernel, dim3(grid_for(n / 8, 256)), dim3(256), 0, st, (u32x4*)dst,
                       (const u32x4*)src, n / 8);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(add_into_kernel<__bf16>, dim3(grid_for(n, 256)), dim3(256), 0, st, (__bf16*)dst,
                       (const __bf16*)src, n);
  else
    hipLaunchKernelGGL(add_into_kernel<float>, dim3(grid_for(n, 256)), dim3(256), 0, st, (float*)dst,
                       (const float*)src, n);
  return hipGetLastError();
}

// The adapter's input under LoRA dropout: out = X where the keep bit is set,
// else 0 (exact: no scaling here).  One mask byte and 8 elements per thread
// and iteration; bit b of byte e keeps element 8 e + b.
__global__ void mask_copy_bf16_kernel(const u32x4* __restrict__ X, const uint8_t* __restrict__ keep,
                                      u32x4* __restrict__ out, int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t k = keep[e];
    u32x4 v = X[e];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] &= (((k >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) | (((k >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
    out[e] = v;
  }
}

__global__ void mask_copy_f32_kernel(const float4* __restrict__ X, const uint8_t* __restrict__ keep,
                                     float4* __restrict__ out, int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t k = keep[e];
    float4 a = X[2 * e], b = X[2 * e + 1];
    a.x = (k & 1u) ? a.x : 0.f;
    a.y = (k & 2u) ? a.y : 0.f;
    a.z = (k & 4u) ? a.z : 0.f;
    a.w = (k & 8u) ? a.w : 0.f;
    b.x = (k & 16u) ? b.x : 0.f;
    b.y = (k & 32u) ? b.y : 0.f;
    b.z = (k & 64u) ? b.z : 0.f;
    b.w = (k & 128u) ? b.w : 0.f;
    out[2 * e] = a;
    out[2 * e + 1] = b;
  }
}

hipError_t launch_mask_copy(int elem_bytes, const void* X, const uint8_t* keep, void* out, int64_t n,
                            hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(mask_copy_bf16_kernel, dim3(grid_for(n8, 256)), dim3(256), 0, st, (const u32x4*)X, keep,
                       (u32x4*)out, n8);
  else
    hipLaunchKernelGGL(mask_copy_f32_kernel, dim3(grid_for(n8, 256)), dim3(256), 0, st, (const float4*)X, keep,
                       (float4*)out, n8);
  return hipGetLastError();
}

// The dropout keep mask drawn on the device from Philox4x32-10 (J. K. Salmon
// et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11, section 4),
// so the backward regenerates the forward's mask from (seed, offset) instead
// of reading a stored one.  Element e of the flattened input takes word e & 3
// of the block with counter (lo32(e >> 2), hi32(e >> 2), o0, o1) under the key
// (k0, k1) and is kept iff that word >= thr (thr = floor(p 2^32)).
__device__ __forceinline__ void philox4x32_10(uint32_t& x0, uint32_t& x1, uint32_t& x2, uint32_t& x3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const uint64_t a = (uint64_t)0xD2511F53u * x0, b = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t y0 = (uint32_t)(b >> 32) ^ x1 ^ k0, y2 = (uint32_t)(a >> 32) ^ x3 ^ k1;
    x0 = y0;
    x1 = (uint32_t)b;
    x2 = y2;
    x3 = (uint32_t)a;
    k0 += 0x9E3779B9u;  // the key after the last round is unused
    k1 += 0xBB67AE85u;
  }
}

// One mask byte (8 elements, two Philox blocks) per thread and iteration:
// writes the packed byte (bit b keeps element 8 e + b) if keep is set and the
// masked copy of X (kept elements exact, the rest 0) if out is set.
template <int EB>
__global__ void dropout_philox_kernel(const void* __restrict__ X, void* __restrict__ out,
                                      uint8_t* __restrict__ keep, int64_t n8, uint32_t thr, uint32_t k0,
                                      uint32_t k1, uint32_t o0, uint32_t o1) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (int64_t)gridDim.x * blockDim.x) {
    uint32_t bits = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t g = 2 * (uint64_t)e + h;
      uint32_t x0 = (uint32_t)g, x1 = (uint32_t)(g >> 32), x2 = o0, x3 = o1;
      philox4x32_10(x0, x1, x2, x3, k0, k1);
      bits |= ((x0 >= thr ? 1u : 0u) | (x1 >= thr ? 2u : 0u) | (x2 >= thr ? 4u : 0u) | (x3 >= thr ? 8u : 0u))
              << (4 * h);
    }
    if (keep) keep[e] = (uint8_t)bits;
    if (!out) continue;
    if constexpr (EB == 2) {
      u32x4 v = static_cast<const u32x4*>(X)[e];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] &= (((bits >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u) | (((bits >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u);
      static_cast<u32x4*>(out)[e] = v;
    } else {
      const float4* x = static_cast<const float4*>(X);
      float4 a = x[2 * e], b = x[2 * e + 1];
      a.x = (bits & 1u) ? a.x : 0.f;
      a.y = (bits & 2u) ? a.y : 0.f;
      a.z = (bits & 4u) ? a.z : 0.f;
      a.w = (bits & 8u) ? a.w : 0.f;
      b.x = (bits & 16u) ? b.x : 0.f;
      b.y = (bits & 32u) ? b.y : 0.f;
      b.z = (bits & 64u) ? b.z : 0.f;
      b.w = (bits & 128u) ? b.w : 0.f;
      static_cast<float4*>(out)[2 * e] = a;
      static_cast<float4*>(out)[2 * e + 1] = b;
    }
  }
}

hipError_t launch_dropout_philox(int elem_bytes, const void* X, void* out, uint8_t* keep, int64_t n, uint32_t thr,
                                 uint64_t seed, uint64_t offset, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8 || (out && !X)) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32), o0 = (uint32_t)offset,
                 o1 = (uint32_t)(offset >> 32);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(dropout_philox_kernel<2>, dim3(grid_for(n8, 256)), dim3(256), 0, st, X, out, keep, n8, thr,
                       k0, k1, o0, o1);
  else
    hipLaunchKernelGGL(dropout_philox_kernel<4>, dim3(grid_for(n8, 256)), dim3(256), 0, st, X, out, keep, n8, thr,
                       k0, k1, o0, o1);
  return hipGetLastError();
}

constexpr int kMaxPanelSplits = 32;

// One 16-row x 64-column tile of the panel per workgroup: the fixed-order
// sum of the split partials (thread t: columns 4 (t & 15) .. +3 of row
// t >> 4, the loads of up to 8 splits in flight before their sums), the
// column scale, then the row-major and/or (through LDS) the transposed bf16
// stores.
__global__ void __launch_bounds__(256) panel_reduce_kernel(const float* __restrict__ part, int splits,
                                                           int64_t part_stride, int64_t ldp, int64_t rows, int64_t n,
                                                           ColScale scale, uint16_t* __restrict__ out, int64_t ldo,
                                                           uint16_t* __restrict__ outt, int64_t ldot) {
  __shared__ float tile[16][65];
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * 16, c0 = (int64_t)blockIdx.y * 64;
  const int cl = 4 * (tid & 15), rl = tid >> 4;
  const int64_t c = c0 + cl, q = q0 + rl;
  const bool ok = c < n && q < rows;
  float alpha[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    alpha[k] = scale.s[0];
#pragma unroll
    for (int i = kColScaleMax - 1; i >= 0; --i)
      if (i < scale.n && c + k < scale.end[i]) alpha[k] = scale.s[i];
  }
  // past the end: a valid element is read and nothing is stored
  const float4 acc = sum_splits(part + (ok ? q * ldp + c : 0), splits, part_stride);
  const float y[4] = {acc.x * alpha[0], acc.y * alpha[1], acc.z * alpha[2], acc.w * alpha[3]};
  if (out && ok) {
    uint2 pk;
    pk.x = (uint32_t)f2bf(y[0]) | ((uint32_t)f2bf(y[1]) << 16);
    pk.y = (uint32_t)f2bf(y[2]) | ((uint32_t)f2bf(y[3]) << 16);
    *reinterpret_cast<uint2*>(out + q * ldo + c) = pk;
  }
  if (!outt) return;
  float* trow = &tile[rl][cl];
  trow[0] = y[0];
  trow[1] = y[1];
  trow[2] = y[2];
  trow[3] = y[3];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * 256 + tid;
    const int cc = idx >> 4, qq = idx & 15;  // consecutive threads: consecutive rows of the transpose
    const int64_t qg = q0 + qq, cg = c0 + cc;
    if (qg < rows && cg < n) outt[cg * ldot + qg] = f2bf(tile[qq][cc]);
  }
}

hipError_t launch_panel_reduce(const float* part, int splits, int64_t part_stride, int64_t ldp, int64_t rows,
                               int64_t n, const ColScale& scale, uint16_t* out, int64_t ldo, uint16_t* outt,
                               int64_t ldot, hipStream_t st) {
  if (rows <= 0 || n <= 0) return hipSuccess;
  if (splits < 1 || splits > kMaxPanelSplits || scale.n < 1 || scale.n > kColScaleMax) return hipErrorInvalidValue;
  // float4 partial loads, 4-column bf16 stores
  if (n % 4 || ldp % 4 || part_stride % 4 || reinterpret_cast<uintptr_t>(part) % 16 ||
      (out && (ldo % 4 || reinterpret_cast<uintptr_t>(out) % 8)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 15) / 16), (unsigned)((n + 63) / 64));
  hipLaunchKernelGGL(panel_reduce_kernel, grid, dim3(256), 0, st, part, splits, part_stride, ldp, rows, n, scale, out,
                     ldo, outt, ldot);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
    p[e] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

struct Table16 {
  float v[16];
};

// W bf16 from NF4 codes with the NF4 GEMM load stage's own byte -> bf16x2
// routine: code dword d (8 elements, absmax block d / 8) to the 16-byte
// output chunk d.  Each wave takes 256 consecutive dwords, lane l
// the dwords l, l + 64, l + 128, l + 192 of them, so every load and every
// 16-byte store instruction covers one contiguous KB of its wave's range
// (one thread per four consecutive dwords had spread each store instruction
// over 4 KB, 32 cache lines).
__global__ void __launch_bounds__(256) nf4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ absmax, int64_t ndw,
                                                          Table16 tab, u32x4* __restrict__ out) {
  __shared__ float2 tab2[256];
  nf4_fill_tab2(tab2, tab.v, threadIdx.x, blockDim.x);
  __syncthreads();
  const uint32_t* src = reinterpret_cast<const uint32_t*>(codes);
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t d0 = wave * 256; d0 < ndw; d0 += waves * 256) {
    uint32_t c[4];
    float am[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t d = d0 + lane + 64 * k;
      c[k] = d < ndw ? src[d] : 0u;
      am[k] = d < ndw ? absmax[d >> 3] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t d = d0 + lane + 64 * k;
      if (d >= ndw) break;
      u32x4 o;
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = nf4_byte_to_bf16x2(tab2, c[k] >> (8 * b), am[k]);
      out[d] = o;
    }
  }
}

// W^T [cols, rows] bf16 straight from NF4 codes of W [rows, cols] (cols a
// multiple of 64): a 64 x 64 tile per workgroup, the load stage's own byte ->
// bf16x2 routine into LDS, then 16-byte stores of the transposed rows.
__global__ void __launch_bounds__(256) nf4_dequant_t_kernel(const uint8_t* __restrict__ codes,
                                                            const float* __restrict__ absmax, int64_t rows,
                                                            int64_t cols, Table16 tab, uint16_t* __restrict__ out) {
  __shared__ float2 tab2[256];
  __shared__ __attribute__((aligned(16))) uint32_t t[64][36];  // 64 rows x 64 bf16 (+ pad)
  nf4_fill_tab2(tab2, tab.v, threadIdx.x, blockDim.x);
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
  if (threadIdx.x < 128) {
    const int rr = threadIdx.x >> 1, half = threadIdx.x & 1;  // 32 elements = 16 code bytes
    const int64_t row = r0 + rr;
    u32x4 o[4] = {};
    if (row < rows) {
      const int64_t e0 = row * cols + c0 + 32 * half;  // first element (cols % 64 == 0: one absmax)
      const u32x4 c = *reinterpret_cast<const u32x4*>(codes + e0 / 2);
      const float am = absmax[e0 >> 6];
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) o[w][b] = nf4_byte_to_bf16x2(tab2, c[w] >> (8 * b), am);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<u32x4*>(&t[rr][16 * half + 4 * w]) = o[w];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 512; e += 256) {
    const int cc = e >> 3, qc = e & 7;  // output row c0 + cc, columns r0 + 8 qc .. +7
    const int64_t c = c0 + cc, r = r0 + 8 * qc;
    if (r >= rows) continue;
    const uint16_t* tt = reinterpret_cast<const uint16_t*>(&t[0][0]);
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = (uint32_t)tt[(8 * qc + 2 * k) * 72 + cc] | ((uint32_t)tt[(8 * qc + 2 * k + 1) * 72 + cc] << 16);
    *reinterpret_cast<u32x4*>(out + c * rows + r) = v;
  }
}

hipError_t launch_nf4_dequant_t(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                                const float* table16, uint16_t* out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 64 || rows % 8) return hipErrorInvalidValue;
  Table16 t;
  for (int i = 0; i < 16; ++i) t.v[i] = table16[i];
  const dim3 grid((unsigned)(cols / 64), (unsigned)((rows + 63) / 64));
  hipLaunchKernelGGL(nf4_dequant_t_kernel, grid, dim3(256), 0, st, codes, absmax, rows, cols, t, out);
  return hipGetLastError();
}

hipError_t launch_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n, const float* table16,
                              uint16_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 64) return hipErrorInvalidValue;
  Table16 t;
  for (int i = 0; i < 16; ++i) t.v[i] = table16[i];
  const int64_t ndw = n / 8;  // code dwords; one thread per four of them
  hipLaunchKernelGGL(nf4_dequant_kernel, dim3(grid_for((ndw + 3) / 4, 256)), dim3(256), 0, st, codes, absmax, ndw, t,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

// Dense bf16 MFMA rate of this chip under its own power and clock limits:
// each wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
// register operands (pseudo-random bf16 values in [-2, 2), four operand
// pairs in turn so the inputs keep changing), one wave per SIMD.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_rate_kernel(int iters, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h = (t * 0x9E3779B9u) ^ ((uint32_t)(i * 4 + e) * 0x85EBCA6Bu);
      h ^= h >> 15;
      h *= 0x2C1B3C6Du;
      h ^= h >> 12;
      // two bf16: random sign, exponent 126 or 127, random mantissa
      const uint32_t lo = ((h & 1u) << 15) | ((126u + ((h >> 1) & 1u)) << 7) | ((h >> 2) & 0x7Fu);
      const uint32_t hi = (((h >> 9) & 1u) << 15) | ((126u + ((h >> 10) & 1u)) << 7) | ((h >> 11) & 0x7Fu);
      w[e] = lo | (hi << 16);
    }
    if (i < 4)
      a[i] = __builtin_bit_cast(bf16x8, w);
    else
      b[i - 4] = __builtin_bit_cast(bf16x8, w);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][15];
  out[t] = sum;
}

hipError_t launch_mfma_rate(int iters, int blocks, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tiny fp32 problems: one launch per direction (tiny.h)
// ---------------------------------------------------------------------------
bool tiny_fits(int64_t M, int64_t K, int64_t N, int64_t r) {
  const int64_t mx = K > N ? K : N;
  return M >= 1 && r >= 1 && r <= tiny::MAX_R && M * r <= tiny::MAX_MR && K >= 1 && N >= 1 && mx <= 4096 &&
         M * r * mx <= (int64_t(1) << 21) && M * K * N <= (int64_t(1) << 25);
}

hipError_t launch_tiny(bool bwd, const float* X, const float* W, const float* A, const float* B, const float* G,
                       float* Y, float* dX, float* dA, float* dB, float* Ps, float* Qs, int64_t M, int64_t K,
                       int64_t N, int64_t r, float s, hipStream_t st) {
  if (!tiny_fits(M, K, N, r)) return hipErrorInvalidValue;
  if (bwd && (!Ps || !Qs)) return hipErrorInvalidValue;
  TinyArgs a;
  a.X = X; a.W = W; a.A = A; a.B = B; a.G = G;
  a.Y = Y; a.dX = dX; a.dA = dA; a.dB = dB; a.Ps = Ps; a.Qs = Qs;
  a.M = (int)M; a.K = (int)K; a.N = (int)N; a.r = (int)r; a.s = s;
  a.tiles_m = (int)((M + tiny::T - 1) / tiny::T);
  const int tk = (int)((K + tiny::T - 1) / tiny::T), tn = (int)((N + tiny::T - 1) / tiny::T);
  if (!bwd) {
    a.blocks_x = a.tiles_m * tn;
    a.blocks_a = 0;
    hipLaunchKernelGGL(tiny_fwd_f32_kernel, dim3((unsigned)a.blocks_x), dim3(tiny::NT), 0, st, a);
  } else {
    a.blocks_x = dX ? a.tiles_m * tk : 0;
    a.blocks_a = tk;
    hipLaunchKernelGGL(tiny_rank_f32_kernel, dim3((unsigned)(2 * a.tiles_m)), dim3(tiny::NT), 0, st, a);
    const hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
    hipLaunchKernelGGL(tiny_bwd_f32_kernel, dim3((unsigned)(a.blocks_x + tk + tn)), dim3(tiny::NT), 0, st, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// few-token fused forward
// ---------------------------------------------------------------------------
bool skinny_fits(int64_t M, int64_t K, int64_t N, int64_t r, int mode) {
  const int64_t lim = int64_t(1) << 30;  // the kernel's buffer offsets stay below
  return M >= 1 && M <= 64 && r >= 8 && r <= 64 && r % 8 == 0 && K % 8 == 0 && N * K * 2 < lim &&
         M * K * 2 < lim && r * K * 2 < lim && N * r * 2 < lim && (mode != sk::ROPE || N % 128 == 0);
}

namespace {
template <int MB, int NB, int RB, int MODE>
hipError_t run_skinny(const SkinnyArgs& a, hipStream_t st) {
  const int64_t blocks = MODE == sk::ROPE ? int64_t(a.N / 128) * 4 : (a.N + 16 * NB - 1) / (16 * NB);
  // waves per block: more waves keep more loads in flight per CU; the
  // partial sums (NW x MB (NB + RB) KiB of LDS) and registers bound it
  constexpr int E = MB * (NB + RB);
  constexpr int NW = E <= 4 ? 16 : (E <= 8 ? 8 : 4);
  hipLaunchKernelGGL((skinny_fwd_kernel<MB, NB, RB, MODE, NW>), dim3((unsigned)blocks), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

template <int MB, int RB>
hipError_t run_skinny_mode(const SkinnyArgs& a, int mode, hipStream_t st) {
  // 4 strips of 16 columns per block once the output is wide enough: fewer
  // blocks, so fewer re-reads of X from L2
  const bool wide = a.N >= 12288;
  if (mode == sk::ROPE) return run_skinny<MB, 2, RB, sk::ROPE>(a, st);
  return wide ? run_skinny<MB, 4, RB, sk::PLAIN>(a, st) : run_skinny<MB, 1, RB, sk::PLAIN>(a, st);
}
}  // namespace

template <int MB>
hipError_t few_launch(const FewArgs& a, int what, bool nf4, hipStream_t st) {
  if (what == 0) {
    // (row groups: one 16-row block of tokens per launch-1 block)
    if (a.pg > 1)
      hipLaunchKernelGGL(few_panel_kernel<1>, dim3(a.Sp * a.pg + a.Sq), dim3(few::NT), 0, st, a);
    else
      hipLaunchKernelGGL(few_panel_kernel<MB>, dim3(a.Sp + a.Sq), dim3(few::NT), 0, st, a);
  } else if (what == 1) {
    // the stream sums at most SMAX panel slabs
    if (a.Sp > (nf4 ? FewPanelPre<MB, few::NT4>::SMAX : FewPanelPre<MB, few::NT>::SMAX)) return hipErrorInvalidValue;
    if (nf4)
      hipLaunchKernelGGL((few_fwd_nf4_kernel<MB>), dim3((unsigned)a.nblk), dim3(few::NT4), 0, st, a);
    else
      hipLaunchKernelGGL((few_fwd_bf16_kernel<MB>), dim3((unsigned)a.nblk), dim3(few::NT), 0, st, a);
  } else {
    const dim3 grid((unsigned)a.nblk);
    if (nf4)
      hipLaunchKernelGGL((few_bwd_kernel<MB, true>), grid, dim3(few::NT), 0, st, a);
    else
      hipLaunchKernelGGL((few_bwd_kernel<MB, false>), grid, dim3(few::NT), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t few_dispatch(const FewArgs& a, int MB, int what, bool nf4, hipStream_t st) {
  if (a.M < 1 || a.M > 16 * MB || a.Mp != 16 * MB || a.r8 < 8 || a.r8 > few::MAXR || a.r8 % 8) return hipErrorInvalidValue;
  if (a.Sp < 1 || a.n_tiles < 1 || a.n_tiles > a.nblk || a.nkt < 1 || a.T != a.n_tiles * a.nkt || a.nblk < 1 ||
      a.nblk > few::GRID || a.nblk > a.T)
    return hipErrorInvalidValue;
  // launch 1's row groups: all rows per block, or one 16-row block each (P only)
  if (!(a.pg == 1 || (a.pg == MB && a.Sq == 0))) return hipErrorInvalidValue;
  // the W stream's tiles and stages cover its output columns and contraction
  // exactly (stages 128 deep in the NF4 forward, 64 otherwise)
  if (what > 0) {
    const int64_t ncols = what == 1 ? a.d_out : a.d_in, K = what == 1 ? a.d_in : a.d_out;
    if ((ncols + few::BN - 1) / few::BN != a.n_tiles || (int64_t)a.nkt * (what == 1 && nf4 ? 128 : 64) != K)
      return hipErrorInvalidValue;
  }
  switch (MB) {
    case 1: return few_launch<1>(a, what, nf4, st);
    case 2: return few_launch<2>(a, what, nf4, st);
    case 4: return few_launch<4>(a, what, nf4, st);
    case 8: return few_launch<8>(a, what, nf4, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_few_panel(const FewArgs& a, int MB, hipStream_t st) { return few_dispatch(a, MB, 0, false, st); }
hipError_t launch_few_reduce(const FewArgs& a, hipStream_t st) {
  if (a.Mp < 16 || a.r8 % 8 || a.Sp < 1 || a.Sq < 1) return hipErrorInvalidValue;
  const int nb = (a.Mp * a.r8 / 4 + few::NT - 1) / few::NT;
  hipLaunchKernelGGL(few_reduce_kernel, dim3(2 * nb), dim3(few::NT), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_few_fwd(const FewArgs& a, int MB, bool nf4, hipStream_t st) {
  return few_dispatch(a, MB, 1, nf4, st);
}
hipError_t launch_few_bwd(const FewArgs& a, int MB, bool nf4, hipStream_t st) {
  return few_dispatch(a, MB, 2, nf4, st);
}

hipError_t launch_skinny_fwd(const SkinnyArgs& a, int mode, hipStream_t st) {
  // 16 or 64 rows of X, rank up to 16 or 64 (rows past M and rank columns
  // past r read as zero)
  if (a.M <= 16) return a.r <= 16 ? run_skinny_mode<1, 1>(a, mode, st) : run_skinny_mode<1, 4>(a, mode, st);
  return a.r <= 16 ? run_skinny_mode<4, 1>(a, mode, st) : run_skinny_mode<4, 4>(a, mode, st);
}

}  // namespace lora
