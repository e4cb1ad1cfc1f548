// panel.h - the rank-r panels of the fused LoRA layer on gfx950:
//
//   out[m, q] = alpha * sum_k X[m, k] * R[q, k]      (q < r, padded to r8)
//
// with R = A for P = s X A^T (forward and the recomputation in the backward)
// and R = B^T for Q = s dY B.  The contraction is long (d_in or d_out) and the
// result narrow (r <= 64 per column tile), so the kernel is bound by streaming
// X once from HBM.  No LDS staging: every lane's 16-byte global load is
// directly its MFMA fragment (v_mfma_f32_16x16x32_bf16 takes 8 consecutive
// contraction elements of one row per lane), R stays hot in L2.  The eight
// waves of a workgroup take interleaved 32-element slices of the contraction
// for the same 32 rows and 64 rank columns, then add their partial tiles in
// LDS in a fixed order (deterministic).  Outputs: row-major [m_store, ldo]
// and/or transposed [r8, ldot], bf16; rows in [M, m_store) are written as 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace lora {

struct PanelArgs {
  const uint16_t* x;  // [M, K] bf16, row stride ldx
  int64_t ldx;
  const uint16_t* w;  // [n_valid, K] bf16, row stride ldw
  int64_t ldw;
  int64_t M, K, n_valid;
  int64_t m_store;    // rows of the outputs (>= M; the extra rows are zeros)
  int64_t n_store;    // rank columns written (r8)
  float alpha;
  uint16_t* out;      // row-major [m_store, ldo] or null
  int64_t ldo;
  uint16_t* outt;     // transposed [n_store, ldot] or null
  int64_t ldot;
};

namespace panel {
constexpr int FM = 2;      // 16-row blocks per workgroup (32 rows)
constexpr int FN = 4;      // 16-column blocks (64 rank columns)
constexpr int WAVES = 8;
constexpr int U = 4;       // contraction slices in flight per wave
constexpr int ROWS = 16 * FM, COLS = 16 * FN;
}  // namespace panel

template <int WAVES_ = panel::WAVES>
__global__ void __launch_bounds__(64 * WAVES_) panel_kernel(const PanelArgs p) {
  using namespace panel;
  __shared__ float red[WAVES][ROWS][COLS + 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * ROWS;
  const int64_t n0 = (int64_t)blockIdx.y * COLS;
  const int64_t nkk = (p.K + 31) / 32;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xr[FM];
  bool xok[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = m0 + 16 * i + l16;
    xok[i] = row < p.M;
    xr[i] = p.x + (xok[i] ? row : 0) * p.ldx + 8 * g;
  }
  const uint16_t* wr[FN];
  bool wok[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t q = n0 + 16 * j + l16;
    wok[j] = q < p.n_valid;
    wr[j] = p.w + (wok[j] ? q : 0) * p.ldw + 8 * g;
  }
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  for (int64_t kk0 = w; kk0 < nkk; kk0 += (int64_t)WAVES * U) {
    u32x4 a[U][FM], b[U][FN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kk = kk0 + (int64_t)u * WAVES;
      const int64_t k = kk * 32 + 8 * g;  // this lane's 8 contraction elements
      const bool kok = kk < nkk && k < p.K;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[u][i] = (kok && xok[i]) ? *reinterpret_cast<const u32x4*>(xr[i] + kk * 32) : zero4;
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b[u][j] = (kok && wok[j]) ? *reinterpret_cast<const u32x4*>(wr[j] + kk * 32) : zero4;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][i]),
                                                              __builtin_bit_cast(bf16x8, b[u][j]), acc[i][j], 0,
                                                              0, 0);
  }

  // partial tiles -> LDS; acc[i][j][v] is (row 16i + 4g + v, column 16j + l16)
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][16 * i + 4 * g + v][16 * j + l16] = acc[i][j][v];
  __syncthreads();

  // fixed-order sum over the waves, then the stores
  constexpr int NT = 64 * WAVES;
  if (p.out) {
    for (int e = tid; e < ROWS * COLS; e += NT) {
      const int row = e / COLS, col = e % COLS;
      const int64_t gm = m0 + row, gq = n0 + col;
      if (gm >= p.m_store || gq >= p.n_store) continue;
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) s += red[ww][row][col];
      p.out[gm * p.ldo + gq] = f2bf(s * p.alpha);
    }
  }
  if (p.outt) {
    for (int e = tid; e < ROWS * COLS; e += NT) {
      const int col = e / ROWS, row = e % ROWS;  // consecutive threads: consecutive rows of Pt
      const int64_t gm = m0 + row, gq = n0 + col;
      if (gm >= p.m_store || gq >= p.n_store) continue;
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) s += red[ww][row][col];
      p.outt[gq * p.ldot + gm] = f2bf(s * p.alpha);
    }
  }
}

}  // namespace lora
