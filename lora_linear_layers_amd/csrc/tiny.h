// tiny.h - the fp32 LoRA layer for tiny problems in one launch per direction
// (page "UnSloth加速微调体验：在LoRA基础上再提速3倍的秘密", sections 算子融合 and
// 反向传播优化):
//
//     forward   Y  = X W^T + P_s B^T,        P_s = s X A^T
//     backward  dX = G W + Q_s A,            Q_s = s G B
//               dA = Q_s^T X,   dB = G^T P_s
//
// Below a few million multiply-adds the split kernels are all launch and
// pipeline fill (the fp32 forward took two launches, the backward eight), so
// here every output tile is one block.  The forward's Y tiles form the rank-r
// rows of their own 32 tokens in the same contraction loop as the base
// product (the two share its left operand tiles): one launch.  The backward
// forms P_s and Q_s of every token first (launch 1, into the workspace), then
// the dX, dA and dB tiles in one launch.  All products go through LDS
// stages of 128 contraction steps with fp32 fused multiply-adds, the next
// stage's operands in flight while the current one is multiplied.  Every sum
// runs in one fixed order (each wave its quarter of every stage in ascending
// order, the four waves' sums added in wave order, the rank term after the
// base term), so results do not depend on the grid and repeat bit for bit.
// Rows and columns past the ends load as zeros and are not stored.  No MFMA:
// at these sizes the work is a few thousand FMAs per thread and the launches
// are the cost (the 128-token, 256 -> 256, r 8 layer: 34 us of kernel time
// per forward + backward against 100 us in the ten launches of the generic
// fp32 GEMMs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

namespace tiny {
constexpr int T = 32;         // output tile edge
constexpr int NT = 256;       // threads per block
constexpr int MAX_R = 32;     // rank limit
constexpr int KC = 128;       // contraction steps per LDS stage (32 per wave)
constexpr int LP = T + 4;     // L row pitch: rows stay 16-byte aligned, column writes spread over banks
constexpr int MAX_MR = 4096;  // M r limit (bounds the dA / dB blocks' contraction over the tokens)
// a stage's operand tiles, contraction-major: L [KC][32 rows] (padded), R and
// R2 [KC][32 columns]; R also holds the waves' partial tiles at the end
struct Tiles {
  __attribute__((aligned(16))) float L[KC][LP];
  __attribute__((aligned(16))) float R[KC][T];
  __attribute__((aligned(16))) float R2[KC][T];
};
static_assert(KC * T >= 4 * T * T, "R holds the four waves' partial tiles");
static_assert(KC == 4 * 32, "a wave takes 32 steps of a stage");
}  // namespace tiny

struct TinyArgs {
  const float *X, *W, *A, *B, *G;
  float *Y, *dX, *dA, *dB;
  float *Ps, *Qs;  // backward: the rank rows [M, r] (workspace)
  int M, K, N, r;  // tokens, d_in, d_out, rank
  float s;
  int tiles_m;     // ceil(M / 32)
  int blocks_x;    // blocks of the Y (forward) or dX (backward) tiles
  int blocks_a;    // backward: blocks of the dA column tiles (then the dB row tiles)
};

// operand loads through the global address space (a generic pointer would
// make them flat loads, which the LDS waits of the tile loop also wait for)
__device__ inline float tiny_ld(const float* p, int64_t i) {
  return ((const __attribute__((address_space(1))) float*)p)[i];
}

// One 32 x 32 tile of a product over a contraction of length kn, staged
// through LDS KC contraction steps at a time, the next stage's operands loaded
// into registers while this one is multiplied.  Result for thread t
// (ti = t / 8, tj = 4 (t % 8)): acc[c] += sum_k L(ti, k) R(k, tj + c), and,
// when TWO, acc2[c] += sum_k L(ti, k) R2(k, tj + c) from the same L tiles (the
// rank-r panel that shares the main product's left operand).  lf(u, k) /
// rf(k, v) / rf2(k, v) return the operands (zero outside their matrices); LT:
// L is read along u (consecutive threads take consecutive u, for a
// transposed source).
//
// Inside a stage, wave w takes the steps 32 w .. 32 w + 31 over the whole
// tile, lane l the 4 x 4 outputs of rows 4 (l / 8) .. + 3 and columns
// 4 (l % 8) .. + 3, one 16-byte read of L (stored k-major) and one of R per
// step for 16 FMAs; the four waves' sums then meet in LDS, added in wave
// order.  Every sum has one fixed order.
template <bool TWO, bool LT, class LF, class RF, class RF2>
__device__ inline void tiny_mm(int kn, LF lf, RF rf, RF2 rf2, tiny::Tiles& sm, float (&acc)[4], float (&acc2)[4]) {
  using tiny::KC;
  constexpr int PER = tiny::T * KC / tiny::NT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ri = 4 * (lane >> 3), cj = 4 * (lane & 7);
  float lv[PER], rv[PER], r2v[PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (int)threadIdx.x + i * tiny::NT;
      if (LT) {
        const int u = e & 31, k = e >> 5;
        lv[i] = k0 + k < kn ? lf(u, k0 + k) : 0.f;
      } else {
        const int u = e / KC, k = e % KC;
        lv[i] = k0 + k < kn ? lf(u, k0 + k) : 0.f;
      }
      const int k = e >> 5, v = e & 31;
      rv[i] = k0 + k < kn ? rf(k0 + k, v) : 0.f;
      if (TWO) r2v[i] = k0 + k < kn ? rf2(k0 + k, v) : 0.f;
    }
  };
  float pa[4][4] = {}, pb[4][4] = {};
  fetch(0);
  for (int k0 = 0; k0 < kn; k0 += KC) {
    __syncthreads();  // every wave done with the previous stage's tiles
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (int)threadIdx.x + i * tiny::NT;
      if (LT)
        sm.L[e >> 5][e & 31] = lv[i];
      else
        sm.L[e % KC][e / KC] = lv[i];
      sm.R[e >> 5][e & 31] = rv[i];
      if (TWO) sm.R2[e >> 5][e & 31] = r2v[i];
    }
    __syncthreads();
    if (k0 + KC < kn) fetch(k0 + KC);
    const int steps = kn - k0 < KC ? kn - k0 : KC;
    const int kb = 32 * wave, ke = kb + 32 < steps ? kb + 32 : steps;
    // 4 steps' 16-byte reads issued together, then their 64 (or 128) FMAs
    for (int k4 = kb; k4 < ke; k4 += 4) {
      float4 l[4], rr[4], r2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        l[u] = *reinterpret_cast<const float4*>(&sm.L[k4 + u][ri]);
        rr[u] = *reinterpret_cast<const float4*>(&sm.R[k4 + u][cj]);
        if (TWO) r2[u] = *reinterpret_cast<const float4*>(&sm.R2[k4 + u][cj]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float lx[4] = {l[u].x, l[u].y, l[u].z, l[u].w};
        const float rx[4] = {rr[u].x, rr[u].y, rr[u].z, rr[u].w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) pa[a][b] = __builtin_fmaf(lx[a], rx[b], pa[a][b]);
        if (TWO) {
          const float r2x[4] = {r2[u].x, r2[u].y, r2[u].z, r2[u].w};
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) pb[a][b] = __builtin_fmaf(lx[a], r2x[b], pb[a][b]);
        }
      }
    }
  }
  // the waves' partial tiles meet in LDS (the stage tiles are free after the
  // barrier); thread t adds its 4 outputs over the waves in order
  const int ti = threadIdx.x >> 3, tj = (threadIdx.x & 7) * 4;
  auto reduce = [&](float (&part)[4][4], float (&out)[4]) {
    __syncthreads();  // every wave done reading the stage tiles
    float* red = &sm.R[0][0];  // [4 waves][32][32]
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(red + (wave * 32 + ri + a) * 32 + cj) =
          make_float4(part[a][0], part[a][1], part[a][2], part[a][3]);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 v = *reinterpret_cast<const float4*>(red + (w * 32 + ti) * 32 + tj);
      out[0] += v.x;
      out[1] += v.y;
      out[2] += v.z;
      out[3] += v.w;
    }
  };
  reduce(pa, acc);
  if (TWO) reduce(pb, acc2);
}

__global__ void __launch_bounds__(tiny::NT) tiny_fwd_f32_kernel(const TinyArgs a) {
  using namespace tiny;
  __shared__ Tiles sm;
  __shared__ float Ps[T * MAX_R];
  const int tm = (int)blockIdx.x % a.tiles_m, tn = (int)blockIdx.x / a.tiles_m;
  const int i0 = tm * T, j0 = tn * T;
  const int ti = threadIdx.x >> 3, tj = (threadIdx.x & 7) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, pv[4] = {0.f, 0.f, 0.f, 0.f};
  // Y tile = X[i0.., :] W[j0.., :]^T and the panel X[i0.., :] A^T on the same X tiles
  tiny_mm<true, false>(
      a.K, [&](int u, int k) { return i0 + u < a.M ? tiny_ld(a.X, (int64_t)(i0 + u) * a.K + k) : 0.f; },
      [&](int k, int v) { return j0 + v < a.N ? tiny_ld(a.W, (int64_t)(j0 + v) * a.K + k) : 0.f; },
      [&](int k, int v) { return v < a.r ? tiny_ld(a.A, (int64_t)v * a.K + k) : 0.f; }, sm, acc, pv);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (tj + c < a.r) Ps[ti * a.r + tj + c] = a.s * pv[c];
  __syncthreads();  // every wave done reading R
  // B rows of the tile's columns into R[j][q]
  for (int e = threadIdx.x; e < T * T; e += NT) {
    const int jj = e >> 5, q = e & 31;
    sm.R[jj][q] = (j0 + jj < a.N && q < a.r) ? tiny_ld(a.B, (int64_t)(j0 + jj) * a.r + q) : 0.f;
  }
  __syncthreads();
  if (i0 + ti >= a.M) return;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = j0 + tj + c;
    if (j >= a.N) continue;
    float v = acc[c];
    for (int q = 0; q < a.r; ++q) v = __builtin_fmaf(Ps[ti * a.r + q], sm.R[tj + c][q], v);
    a.Y[(int64_t)(i0 + ti) * a.N + j] = v;
  }
}

// Backward launch 1: the rank rows of 32 tokens per block, P_s = s X A^T
// (blocks [0, tiles_m)) and Q_s = s G B (the next tiles_m), into Ps / Qs [M, r]
__global__ void __launch_bounds__(tiny::NT) tiny_rank_f32_kernel(const TinyArgs a) {
  using namespace tiny;
  __shared__ Tiles sm;
  const int b = (int)blockIdx.x;
  const bool is_q = b >= a.tiles_m;
  const int m0 = (is_q ? b - a.tiles_m : b) * T;
  const int ti = threadIdx.x >> 3, tj = (threadIdx.x & 7) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f}, none2[4];
  auto none = [](int, int) { return 0.f; };
  if (is_q)
    tiny_mm<false, false>(
        a.N, [&](int u, int j) { return m0 + u < a.M ? tiny_ld(a.G, (int64_t)(m0 + u) * a.N + j) : 0.f; },
        [&](int j, int q) { return q < a.r ? tiny_ld(a.B, (int64_t)j * a.r + q) : 0.f; }, none, sm, v, none2);
  else
    tiny_mm<false, false>(
        a.K, [&](int u, int k) { return m0 + u < a.M ? tiny_ld(a.X, (int64_t)(m0 + u) * a.K + k) : 0.f; },
        [&](int k, int q) { return q < a.r ? tiny_ld(a.A, (int64_t)q * a.K + k) : 0.f; }, none, sm, v, none2);
  if (m0 + ti >= a.M) return;
  float* out = is_q ? a.Qs : a.Ps;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (tj + c < a.r) out[(int64_t)(m0 + ti) * a.r + tj + c] = a.s * v[c];
}

// Backward launch 2: blocks [0, blocks_x): dX tiles; [blocks_x, blocks_x +
// blocks_a): dA column tiles; the rest: dB row tiles
__global__ void __launch_bounds__(tiny::NT) tiny_bwd_f32_kernel(const TinyArgs a) {
  using namespace tiny;
  __shared__ Tiles sm;
  __shared__ float Qr[T * MAX_R];
  int b = (int)blockIdx.x;
  const int ti = threadIdx.x >> 3, tj = (threadIdx.x & 7) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, none2[4];
  auto none = [](int, int) { return 0.f; };
  if (b < a.blocks_x) {
    const int i0 = (b % a.tiles_m) * T, k0 = (b / a.tiles_m) * T;
    // the tile rows' Q_s (read after the loop's barriers)
    for (int e = threadIdx.x; e < T * a.r; e += NT)
      Qr[e] = i0 + e / a.r < a.M ? tiny_ld(a.Qs, (int64_t)i0 * a.r + e) : 0.f;
    // dX tile = G[i0.., :] W[:, k0..]
    tiny_mm<false, false>(
        a.N, [&](int u, int j) { return i0 + u < a.M ? tiny_ld(a.G, (int64_t)(i0 + u) * a.N + j) : 0.f; },
        [&](int j, int v) { return k0 + v < a.K ? tiny_ld(a.W, (int64_t)j * a.K + k0 + v) : 0.f; }, none, sm, acc, none2);
    __syncthreads();  // every wave done reading R
    // A columns of the tile into R[q][k]
    for (int e = threadIdx.x; e < T * T; e += NT) {
      const int q = e >> 5, kk = e & 31;
      sm.R[q][kk] = (q < a.r && k0 + kk < a.K) ? tiny_ld(a.A, (int64_t)q * a.K + k0 + kk) : 0.f;
    }
    __syncthreads();
    if (i0 + ti >= a.M) return;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = k0 + tj + c;
      if (k >= a.K) continue;
      float v = acc[c];
      for (int q = 0; q < a.r; ++q) v = __builtin_fmaf(Qr[ti * a.r + q], sm.R[q][tj + c], v);
      a.dX[(int64_t)(i0 + ti) * a.K + k] = v;
    }
    return;
  }
  b -= a.blocks_x;
  if (b < a.blocks_a) {
    // dA[q][k0..] = sum_t Q_s[t][q] X[t][k0..]: L(q, t) = Q_s read transposed
    const int k0 = b * T;
    tiny_mm<false, true>(
        a.M, [&](int q, int t) { return q < a.r ? tiny_ld(a.Qs, (int64_t)t * a.r + q) : 0.f; },
        [&](int t, int v) { return k0 + v < a.K ? tiny_ld(a.X, (int64_t)t * a.K + k0 + v) : 0.f; }, none, sm, acc, none2);
    if (ti >= a.r) return;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (k0 + tj + c < a.K) a.dA[(int64_t)ti * a.K + k0 + tj + c] = acc[c];
    return;
  }
  {
    // dB[j0 + u][q] = sum_t G[t][j0 + u] P_s[t][q]: L(u, t) = G read transposed
    const int j0 = (b - a.blocks_a) * T;
    tiny_mm<false, true>(
        a.M, [&](int u, int t) { return j0 + u < a.N ? tiny_ld(a.G, (int64_t)t * a.N + j0 + u) : 0.f; },
        [&](int t, int q) { return q < a.r ? tiny_ld(a.Ps, (int64_t)t * a.r + q) : 0.f; }, none, sm, acc, none2);
    if (j0 + ti >= a.N) return;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (tj + c < a.r) a.dB[(int64_t)(j0 + ti) * a.r + tj + c] = acc[c];
  }
}

}  // namespace lora
