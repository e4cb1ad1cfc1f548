// skinny.h - the fused LoRA forward for few tokens (M <= 64) in ONE launch:
//
//     Y = X W^T + bf16(s X A^T) B^T        (page "UnSloth加速微调体验…",
//                                          section 算子融合)
//
// with an optional RoPE epilogue (section RoPE缓存集成).
//
// With few tokens the layer is a stream of W: every other operand (X, A, B)
// is a few hundred KB and stays in L2.  The split-contraction path needs
// four launches (panel partials, their reduction, GEMM partials, the finish);
// each costs several microseconds of launch and drain, more than streaming a
// 4096 x 4096 W takes.  Here a block owns a strip of output columns for all
// M rows and the whole contraction, so no partials leave the block:
//
//   * NW waves (16, 8 or 4: as many as the registers and the LDS for the
//     partial sums allow) split the contraction; each lane loads its MFMA
//     fragments straight from global memory into registers (16 bytes of a
//     row per lane; W from HBM, X and A from L2), D steps ahead, and runs
//     v_mfma_f32_16x16x32_bf16 on [X] x [W strip | A]^T: the strip's outputs
//     and the block's own copy of the rank-r panel X A^T (a few MFMAs per
//     step; recomputing it per block is cheaper than another launch).
//   * The waves' parts meet in LDS; P = bf16(s X A^T) is rounded where the split
//     path rounds it, goes back through LDS into the MFMA's A layout, and
//     P B^T is added with one more MFMA pass over r.
//   * Epilogue: bf16 store, or RoPE on column pairs (c, c + 64): a RoPE
//     block's two 16-column strips lie 64 apart in one head.
//
// Measured on MI355X (4096 x 4096 W, 16 tokens): 17-19 us per call against
// 33 us for the four launches of the split path.  What bounds it: the X and A
// fragments are 16 rows x 64 bytes per load instruction, which from L2 moves
// about 6.8 TB/s over the chip (contiguous loads: about 23), so the X and A
// re-reads, not W, set the pace.  An NF4 form of this kernel (codes and
// absmax as the W fragment, table lookups in LDS) was slower than the split
// path's NF4 load stage and is not built.
//
// MFMA 16x16x32 layouts: A lane l holds row l % 16, contraction
// 8 (l / 16) .. +7; B lane l holds column l % 16, the same contraction; the
// 4 results of lane l are rows 4 (l / 16) + v, column l % 16.
#pragma once

#include <type_traits>

#include "gemm.h"

namespace lora {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace sk {
enum Mode : int { PLAIN = 0, ROPE = 1 };
constexpr int BIG = 0x40000000;        // buffer resource size (offsets stay below)
constexpr uint32_t OOB = 0x40000000u;  // lane offset that reads zero
}  // namespace sk

// f(integral_constant<int, d>) for d = 0 .. D-1, in order (slot indices stay
// compile-time constants, so the fragment arrays stay in registers)
template <class F, int... ds>
__device__ __forceinline__ void sk_for_slots(F&& f, std::integer_sequence<int, ds...>) {
  (f(std::integral_constant<int, ds>{}), ...);
}

struct SkinnyArgs {
  const uint16_t* X;  // [M, K] bf16, row stride ldx
  int64_t ldx;
  const uint16_t* W;  // [N, K] bf16, row stride ldw
  int64_t ldw;
  const uint16_t* A;  // [r, K] bf16
  const uint16_t* B;  // [N, r] bf16
  uint16_t* Y;        // [M, N] bf16
  int M, N, K, r;
  float s;
  const int32_t* pos;  // ROPE: position of each row; cos / sin rows of 64
  const float* cosc;
  const float* sinc;
  int64_t max_pos;     // rows of the cos / sin cache
};

// MB: 16-row blocks of X (M <= 16 MB); NB: 16-column strips per block; RB:
// 16-wide blocks of the rank (r <= 16 RB); MODE: sk::Mode; NW: waves.
template <int MB, int NB, int RB, int MODE, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
skinny_fwd_kernel(const SkinnyArgs p) {
  static_assert(MODE != sk::ROPE || NB == 2, "a RoPE block holds the two halves of 16 head pairs");
  static_assert(NW == 4 || NW == 8 || NW == 16, "4, 8 or 16 waves");
  static_assert(NW >= MB, "one finishing wave per 16-row block");
  constexpr int NT = 64 * NW;
  // prefetch depth (steps of 32 contraction elements), bounded by the
  // registers a wave has at NW / 4 waves per SIMD
  constexpr int REGS = (MB + RB + NB) * 4;
  constexpr int BUDGET = NW == 16 ? 48 : (NW == 8 ? 112 : 160);
  constexpr int D0 = BUDGET / REGS;
  constexpr int D = D0 > 8 ? 8 : (D0 < 2 ? 2 : D0);
  constexpr int RK = (16 * RB + 31) / 32;  // k32 steps over the rank
  constexpr int RED = NW * MB * (NB + RB) * 4 * 64 * 4;  // bytes of partial sums

  __shared__ __attribute__((aligned(16))) char smem[RED + 4 * 16 * 16 * RB * 2];
  float* red = reinterpret_cast<float*>(smem);
  uint16_t* plds = reinterpret_cast<uint16_t*>(smem + RED);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;

  // the block's strips: contiguous 16 NB columns, or (RoPE) n0 and n0 + 64
  int n0;
  if constexpr (MODE == sk::ROPE)
    n0 = 128 * (int)(blockIdx.x >> 2) + 16 * (int)(blockIdx.x & 3);
  else
    n0 = 16 * NB * (int)blockIdx.x;
  auto col0 = [&](int j) { return MODE == sk::ROPE ? n0 + 64 * j : n0 + 16 * j; };

  // the wave's part of the contraction, in steps of 32
  const int nks = (p.K + 31) / 32;
  const int qs = (nks + NW - 1) / NW;
  const int sbeg = wave * qs;
  const int send = sbeg + qs < nks ? sbeg + qs : nks;

  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.X), (short)0, sk::BIG, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.A), (short)0, sk::BIG, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.W), (short)0, sk::BIG, 0x00020000);

  // per-slot fragments (bf16x8 as 4 dwords)
  u32x4 xf[D][MB], af[D][RB], wf[D][NB];
  auto load = [&](int st, auto slot_c) {
    constexpr int d = decltype(slot_c)::value;
    const bool live = st >= sbeg && st < send;
    const int k = 32 * st + 8 * g;  // the lane's first contraction element
    const bool kin = live && k < p.K;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int row = 16 * mb + l16;
      const uint32_t o = kin && row < p.M ? (uint32_t)((row * p.ldx + k) * 2) : sk::OOB;
      xf[d][mb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)o, 0, 0));
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = 16 * rb + l16;
      const uint32_t o = kin && row < p.r ? (uint32_t)((row * (int64_t)p.K + k) * 2) : sk::OOB;
      af[d][rb] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)o, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t n = col0(j) + l16;
      const uint32_t o = kin && n < p.N ? (uint32_t)((n * p.ldw + k) * 2) : sk::OOB;
      wf[d][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)o, 0, 0));
    }
  };

  f32x4 ay[MB][NB], ap[MB][RB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int j = 0; j < NB; ++j) ay[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ap[mb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](auto slot_c) {
    constexpr int d = decltype(slot_c)::value;
    bf16x8 wv[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) wv[j] = __builtin_bit_cast(bf16x8, wf[d][j]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8 xv = __builtin_bit_cast(bf16x8, xf[d][mb]);
#pragma unroll
      for (int j = 0; j < NB; ++j) ay[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, wv[j], ay[mb][j], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        ap[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8, af[d][rb]), ap[mb][rb],
                                                             0, 0, 0);
    }
  };

  // software pipeline over the quarter: slot d holds step i + d; steps past
  // the quarter load zeros (out-of-range offsets), so a whole number of
  // D-step rounds runs and their MFMAs add nothing
  sk_for_slots([&](auto dc) { load(sbeg + decltype(dc)::value, dc); }, std::make_integer_sequence<int, D>{});
  for (int i = sbeg; i < send; i += D)
    sk_for_slots(
        [&](auto dc) {
          compute(dc);
          load(i + decltype(dc)::value + D, dc);
        },
        std::make_integer_sequence<int, D>{});

  // ---- the waves' parts meet in LDS ----
  // red[(w * MB (NB + RB) + e) * 4 + v][lane], e: Y blocks then P blocks
  constexpr int E = MB * (NB + RB);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((wave * E + mb * (NB + RB) + j) * 4 + v) * 64 + lane] = ay[mb][j][v];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[((wave * E + mb * (NB + RB) + NB + rb) * 4 + v) * 64 + lane] = ap[mb][rb][v];
  }
  __syncthreads();
  if (wave >= MB) return;
  // wave w finishes rows 16 w .. 16 w + 15
  const int mb = wave;
  f32x4 y[NB], pp[RB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += red[((w * E + mb * (NB + RB) + j) * 4 + v) * 64 + lane];
      y[j][v] = a;
    }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += red[((w * E + mb * (NB + RB) + NB + rb) * 4 + v) * 64 + lane];
      pp[rb][v] = a;
    }
  // P = bf16(s X A^T), rows 4 g + v, column 16 rb + l16 of this wave's 16 rows,
  // into LDS [16][16 RB] and back in the A layout (row l16, rank 8 g ..)
  uint16_t* pw = plds + wave * 16 * 16 * RB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) pw[(4 * g + v) * (16 * RB) + 16 * rb + l16] = f2bf(p.s * pp[rb][v]);
  // (the wave reads back only what it wrote; LDS operations of a wave
  // complete in order)
  const __amdgpu_buffer_rsrc_t rbb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.B), (short)0, sk::BIG, 0x00020000);
#pragma unroll
  for (int kr = 0; kr < RK; ++kr) {
    const int c = 32 * kr + 8 * g;  // the lane's first rank column
    u32x4 pv = {0u, 0u, 0u, 0u};
    if (c < 16 * RB) pv = *reinterpret_cast<const u32x4*>(pw + l16 * (16 * RB) + c);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t n = col0(j) + l16;
      const uint32_t o = (n < p.N && c < p.r) ? (uint32_t)((n * p.r + c) * 2) : sk::OOB;
      const u32x4 bv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rbb, (int)o, 0, 0));
      y[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pv), __builtin_bit_cast(bf16x8, bv),
                                                     y[j], 0, 0, 0);
    }
  }

  // ---- epilogue: y[j][v] = Y[16 mb + 4 g + v, col0(j) + l16] ----
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 16 * mb + 4 * g + v;
    if (row >= p.M) continue;
    if constexpr (MODE == sk::ROPE) {
      const int f = (n0 & 127) + l16;  // frequency index (< 64) of the pair
      const int32_t ps = p.pos[row];
      const bool ok = rope_pos_ok(ps, p.max_pos);
      const int64_t cr = ok ? (int64_t)ps * 64 + f : 0;
      const float cs = ok ? p.cosc[cr] : 0.f, sn = ok ? p.sinc[cr] : 0.f;
      const float z1 = y[0][v], z2 = y[1][v];
      p.Y[(int64_t)row * p.N + n0 + l16] = f2bf(z1 * cs - z2 * sn);
      p.Y[(int64_t)row * p.N + n0 + 64 + l16] = f2bf(z2 * cs + z1 * sn);
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = col0(j) + l16;
        if (n < p.N) p.Y[(int64_t)row * p.N + n] = f2bf(y[j][v]);
      }
    }
  }
}

}  // namespace lora
