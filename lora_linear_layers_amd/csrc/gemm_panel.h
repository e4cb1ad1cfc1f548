// gemm_panel.h - the rank-r panel GEMM: fp32 split partials of X R^T for a
// tall X [M, K] (bf16, row-major) and a short R [r, K] (the adapter's A, a
// group's stacked A's, or B^T for the backward's dY B), the first step of
// both the forward (X A^T) and the backward's recompute and dY B (page
// "UnSloth加速微调体验…", sections 算子融合 and 反向传播优化).
//
// The work is a stream of X: 2 r FLOP per element read, far below the
// machine balance, so the kernel is built for HBM bandwidth (on MI355X a
// plain streaming read reaches about 6.1 TB/s, from L2 about 21 TB/s through
// the LDS DMA path).  A BM-row tile covers every panel column (BN = 64, 128
// or 256 >= r), so X is read exactly once; global tiles go straight to LDS
// (buffer_load_dwordx4 ... lds, 8 rows x 128 bytes per instruction) through a
// ring of NS stages issued NS - 1 stages ahead, 100+ KB in flight per CU.
// The contraction is split over gridDim / tiles_m blocks per row tile; split
// z writes its fp32 partial to C + z part_stride (rows at or past m_store and
// columns at or past n_store are not written), and panel_reduce_kernel sums
// the splits in order.  BM = 128 (launch.h): against 64 it halves the re-reads
// of R (from L2) per byte of X, against 256 it halves the splits, so the
// fp32 partials and the per-block pipeline fill; measured on the Llama-3-8B
// MLP panels the three differ by 5 %, 128 first.
//
// Stage t (64-deep): wait for this wave's DMAs of stage t (vmcnt: stages
// t+1 .. t+NS-2 may still fly), barrier (every wave's stage t landed, every
// wave done with stage t-1), issue stage t+NS-1 into stage t-1's slot, then
// four contraction steps.  Stages past the end issue DMAs at an out-of-range
// offset (zeros into a free slot), so every wait has the same count; the
// kernel waits for them before it ends.  Rows at or past m_load and
// contraction chunks at or past the split's end read zero the same way.
//
// Waves: 4 x 1 over a 256-row tile, else 2 x 2; each wave's part is FM x FN
// blocks of v_mfma_f32_32x32x16_bf16.  LDS rows are 128 bytes with 16-byte
// chunk c at chunk c ^ ((row >> 1) & 7); DMA instruction i of wave w moves
// rows 8 (i + IW w) + lane / 8 (IW instructions per wave, even), the lane
// landing at physical chunk lane & 7, i.e. logical chunk
// (lane & 7) ^ ((lane >> 4) | 4 (i & 1)) (the same lane mapping as the
// whole-tile NT kernel).
#pragma once

#include <type_traits>

#include "gemm_w4.h"

namespace lora {

namespace pdma {
constexpr int BK = 64, NT = 256;
template <int BM, int BN>
struct Cfg {
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NS0 = (160 * 1024) / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;  // ring stages
  static constexpr int IA = BM / 8 / 4;         // A instructions per wave
  static constexpr int IB = BN / 8 / 4;         // B instructions per wave
  static constexpr int PER = IA + IB;           // DMAs per wave per stage
  // waves: 4 x 1 over 256 rows, else 2 x 2
  static constexpr int WM = BM == 256 ? 4 : 2, WN = 4 / WM;
  static constexpr int FM = BM / WM / 32, FN = BN / WN / 32;  // MFMA blocks per wave
  static_assert(IA % 2 == 0 && IB % 2 == 0, "row parity pattern of the DMA lane mapping");
  static_assert(FM >= 1 && FN >= 1, "wave tile of at least one 32 x 32 block");
};

constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }
}  // namespace pdma

template <int BM, int BN>
__global__ void __launch_bounds__(pdma::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
panel_dma_kernel(const GemmArgs p) {
  using namespace pdma;
  using C = Cfg<BM, BN>;
  constexpr int NS = C::NS, LEAD = NS - 1, FM = C::FM, FN = C::FN;
  constexpr int A_BYTES = C::A_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STAGE];
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int mt = (int)(blockIdx.x % p.tiles_m), z = (int)(blockIdx.x / p.tiles_m);
  const int64_t m0 = (int64_t)mt * BM;
  const int64_t kbeg = (int64_t)z * p.k_split;
  const int64_t kend = kbeg + p.k_split < p.K1 ? kbeg + p.k_split : p.K1;
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;

  // ---- DMA addressing ----
  const int dr = lane >> 3;
  const int dce = (lane & 7) ^ (lane >> 4), dco = (lane & 7) ^ ((lane >> 4) | 4);
  const char* ga = reinterpret_cast<const char*>(p.a1) + (m0 * p.lda1 + kbeg) * 2;
  const int klen = (int)(kend - kbeg);
  const int64_t mrem = p.m_load - m0;  // rows of X left from the tile's first
  // B instruction i moves the 8 tile rows 8 (i + IB w) ..: their source (one
  // of the group's R's, or b1), the source's row of tile row 0 (rb_off) and
  // its row count (rb_lim), fixed for the whole kernel and uniform per wave
  const char* gb[C::IB];
  int rb_off[C::IB], rb_lim[C::IB];
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    const int row8 = 8 * (i + C::IB * wave);
    const void* src = p.b1;
    int off = 0, lim = (int)p.n_load;
    for (int g = 0; g < p.n_src; ++g)
      if (row8 >= p.rs_beg[g]) {
        src = p.rs[g];
        off = p.rs_beg[g];
        lim = p.rs_rows[g];
      }
    gb[i] = reinterpret_cast<const char*>(src) + kbeg * 2;
    rb_off[i] = off;
    rb_lim[i] = lim;
  }
  // A instruction i: rows 8 (i + IA w) + dr; B instruction i: 8 (i + IB w) + dr
  // of the tile, row - rb_off[i] of its source
  auto dma = [&](int u, int s, int op, int i) {
    const int odd = i & 1;
    const int dc = odd ? dco : dce;
    const int row = 8 * (i + (op == 0 ? C::IA : C::IB) * wave) + dr - (op == 0 ? 0 : rb_off[i]);
    const int64_t ld = op == 0 ? p.lda1 : p.ldb1;
    const int kk = u * BK + 8 * dc;
    const bool ok = kk < klen && row < (op == 0 ? mrem : (int64_t)rb_lim[i]);
    uint32_t vo = ok ? (uint32_t)(row * ld * 2 + kk * 2) : w4::OOB;
    asm volatile("" : "+v"(vo));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(op == 0 ? ga : gb[i]), (short)0, w4::BIG, 0x00020000);
    char* dst = smem + s * C::STAGE + (op == 0 ? 0 : A_BYTES) + (8 * (i + (op == 0 ? C::IA : C::IB) * wave)) * 128;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)vo, 0, 0,
                                             0);
  };
  auto issue = [&](int u) {
    const int s = u % NS;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) dma(u, s, 0, i);
#pragma unroll
    for (int i = 0; i < C::IB; ++i) dma(u, s, 1, i);
  };

  // ---- fragments ----
  const int swz = (l32 >> 1) & 7;
  const uint32_t ra = (uint32_t)(wm * (BM / C::WM) + l32) * 128;
  const uint32_t rb = (uint32_t)A_BYTES + (uint32_t)(wn * (BN / C::WN) + l32) * 128;
  bf16x8 fa[2][FM], fb[2][FN];
  auto rd = [&](int s, int st, auto fsel) {
    constexpr int f = decltype(fsel)::value;
    const uint32_t c = (uint32_t)(((2 * st + hh) ^ swz) << 4);
    const char* base = smem + s * C::STAGE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[f][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + ra + c + i * 32 * 128));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[f][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + rb + c + j * 32 * 128));
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto step = [&](auto fsel) {
    constexpr int f = decltype(fsel)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][i], fb[f][j], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < LEAD; ++u) issue(u);
    for (int t = 0; t < nk; ++t) {
      const int s = t % NS;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::PER * (LEAD - 1)));
      lds_barrier();
      issue(t + LEAD);  // into stage t-1's slot; zeros past the end
      rd(s, 0, I0{});
      rd(s, 1, I1{});
      step(I0{});
      rd(s, 2, I0{});
      step(I1{});
      rd(s, 3, I1{});
      step(I0{});
      step(I1{});
    }
    // the DMAs issued past the end must land before the block's LDS is freed
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  // fp32 partial: acc[i][j][v] = C[m0 + wm BM / WM + 32 i + 8 (v / 4) + 4 hh + v % 4,
  //                                  wn BN / WN + 32 j + l32]
  float* out = reinterpret_cast<float*>(p.c) + (int64_t)z * p.part_stride;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + wm * (BM / C::WM) + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (row >= p.m_store) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn * (BN / C::WN) + 32 * j + l32;
        if (col < p.n_store) out[row * p.ldc + col] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------------------
// Token-split partials of the adapters' gradients for up to 128 rows of C
// (BR = 64: one adapter's rank; BR = 128: a group's stacked ranks):
// C = Aop Bop over a range of tokens, Aop [R, M] the transposed panel (P^T
// for dB^T = P^T G, Q^T for dA = Q^T X; rows contiguous along the tokens),
// Bop [M, N] the tall operand
// (G or X, rows contiguous along N): page "UnSloth加速微调体验…", section
// 反向传播优化.  Like the panel, a stream of the tall operand, so the same
// design: a 256-column tile holds every row of C (R <= BR), so G or X
// is read once (64-row tiles read it twice: 176 -> 146 us for a 128-row dA
// over an 8192 x 4096 X); both operands go to LDS by DMA through an NS-stage ring;
// split z covers tokens [z k_split, ..) and writes its fp32 partial at
// C + z part_stride (reduce_splits_kernel sums them in order).
//
// Bop is contraction-major, so its MFMA fragments come from LDS through
// ds_read_b64_tr_b16 (the transposing LDS read): the stage's 64 token rows
// of 512 bytes hold 16-byte chunk c of row k at chunk c ^ 2 f(k),
// f(k) = (k & 3) | ((k >> 1) & 4) (the NN whole-tile kernel's layout,
// conflict-free for those reads).  DMA instruction i of wave w moves token
// rows 16 w + 2 i + lane / 32, the lane landing at physical chunk lane & 31,
// i.e. logical chunk (lane & 31) ^ 2 f(row).  Aop rows go as in the panel
// kernel.  Wave w computes columns 64 w .. 64 w + 63 against all BR rows.
namespace sdma {
constexpr int BN = 256, BK = 64, NT = 256;
constexpr int B_BYTES = BK * BN * 2;  // 64 token rows of 512 bytes
template <int BR, int NS_>
struct Cfg {
  static constexpr int A_BYTES = BR * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NS = NS_;  // ring stages
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "the ring fits the LDS");
  static constexpr int IA = BR / 8 / 4;  // Aop instructions per wave
  static constexpr int IB = BK / 2 / 4;  // Bop instructions per wave
  static constexpr int PER = IA + IB;
  static constexpr int FM = BR / 32, FN = 2;
  static_assert(IA % 2 == 0, "row parity pattern of the Aop lane mapping");
};
}  // namespace sdma

template <int BR, int NS_>
__global__ void __launch_bounds__(sdma::NT) __attribute__((amdgpu_waves_per_eu(1, 2)))
splitnn_dma_kernel(const GemmArgs p) {
  using namespace sdma;
  using C = Cfg<BR, NS_>;
  constexpr int NS = C::NS, LEAD = NS - 1, FM = C::FM, FN = C::FN;
  constexpr int A_BYTES = C::A_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[NS * C::STAGE];
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  // grid (column tiles, splits): both coordinates are workgroup ids, so
  // scalar; the DMA resources built from them must be (a coordinate left
  // in vector registers, as a division of a flat id leaves it, makes the
  // compiler wrap every DMA in a loop over the lanes' values)
  const int nt = (int)blockIdx.x, z = (int)blockIdx.y;
  const int64_t n0 = (int64_t)nt * BN;
  const int64_t kbeg = (int64_t)z * p.k_split;
  const int64_t kend = kbeg + p.k_split < p.K1 ? kbeg + p.k_split : p.K1;
  const int nk = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
  const int klen = (int)(kend - kbeg);

  // ---- DMA addressing ----
  const int dce = (lane & 7) ^ (lane >> 4), dco = (lane & 7) ^ ((lane >> 4) | 4);
  const char* ga = reinterpret_cast<const char*>(p.a1) + kbeg * 2;                   // Aop [R, ld] at token kbeg
  const char* gb = reinterpret_cast<const char*>(p.b1) + (kbeg * p.ldb1 + n0) * 2;  // Bop token row kbeg, column n0
  const int64_t ncols = p.n_load - n0;  // columns of Bop left from n0
  auto dma_a = [&](int u, int s, int i) {
    const int dc = (i & 1) ? dco : dce;
    const int row = 8 * (i + C::IA * wave) + (lane >> 3);
    const int kk = u * BK + 8 * dc;
    const bool ok = kk < klen && row < p.m_load;
    uint32_t vo = ok ? (uint32_t)(row * p.lda1 * 2 + kk * 2) : w4::OOB;
    asm volatile("" : "+v"(vo));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(ga), (short)0, w4::BIG, 0x00020000);
    char* dst = smem + s * C::STAGE + (8 * (i + C::IA * wave)) * 128;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)vo, 0, 0,
                                             0);
  };
  auto dma_b = [&](int u, int s, int i) {
    const int k = 16 * wave + 2 * i + (lane >> 5);  // token row within the stage
    const int f = (k & 3) | ((k >> 1) & 4);
    const int c = (lane & 31) ^ (2 * f);  // logical 16-byte chunk
    const bool ok = u * BK + k < klen && 8 * c < ncols;
    uint32_t vo = ok ? (uint32_t)(((int64_t)(u * BK + k) * p.ldb1 + 8 * c) * 2) : w4::OOB;
    asm volatile("" : "+v"(vo));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(gb), (short)0, w4::BIG, 0x00020000);
    char* dst = smem + s * C::STAGE + A_BYTES + (16 * wave + 2 * i) * 512;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, (int)vo, 0, 0,
                                             0);
  };
  auto issue = [&](int u) {
    const int s = u % NS;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) dma_a(u, s, i);
#pragma unroll
    for (int i = 0; i < C::IB; ++i) dma_b(u, s, i);
  };

  // ---- fragments ----
  // Aop: row 32 i + l32, tokens 16 st + 8 hh .. +7 (chunk 2 st + hh)
  const int swz = (l32 >> 1) & 7;
  const uint32_t ra = (uint32_t)l32 * 128;
  // Bop through ds_read_b64_tr_b16: within each 16-lane group, lane i receives
  // element (4 q + i / 4, i % 4) of the group's 4 x 4 loads, so pointing lane
  // i at token row k0 + i / 4 and columns c0 + 4 (i % 4) .. +3 hands it token
  // rows k0 .. k0 + 3 of column c0 + i.  Lane l of the 32x32x16 fragment needs
  // column 32 j + l % 32 and tokens 8 (l / 32) .. +7 of step st: group
  // gq = l >> 4 takes columns 32 j + 16 (gq & 1) and token rows
  // 16 st + 8 (gq >> 1) + 4 h, h < 2, whose swizzle is f = ((l & 15) >> 2) | 4 (gq >> 1).
  uint32_t nn_r[FN];
  {
    const int gq = lane >> 4, i16 = lane & 15;
    const int f = (i16 >> 2) | ((gq >> 1) << 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int chunk = (64 * wave + 32 * j + 16 * (gq & 1) + 4 * (i16 & 3)) >> 3;
      nn_r[j] = (uint32_t)A_BYTES + (uint32_t)(8 * (gq >> 1) + (i16 >> 2)) * 512 +
                (uint32_t)((chunk ^ (2 * f)) << 4) + (uint32_t)((i16 & 1) << 3);
    }
  }
  bf16x8 fa[2][FM], fb[2][FN];
  auto rd = [&](int s, int st, auto fsel) {
    constexpr int fi = decltype(fsel)::value;
    const char* base = smem + s * C::STAGE;
    const uint32_t c = (uint32_t)(((2 * st + hh) ^ swz) << 4);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[fi][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + ra + c + i * 32 * 128));
    // (the transposing reads in one asm batch: the builtin form would make
    // the compiler wait for every DMA of the ring in flight first)
    u32x2 ad[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) ad[j][hq] = lds_addr(base + nn_r[j] + (16 * st + 4 * hq) * 512);
    lds_tr_frags<FN>(fb[fi], ad);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  auto step = [&](auto fsel) {
    constexpr int fi = decltype(fsel)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fi][i], fb[fi][j], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < LEAD; ++u) issue(u);
    for (int t = 0; t < nk; ++t) {
      const int s = t % NS;
      __builtin_amdgcn_s_waitcnt(pdma::vmcnt_imm(C::PER * (LEAD - 1)));
      lds_barrier();
      issue(t + LEAD);  // into stage t-1's slot; zeros past the end
      rd(s, 0, I0{});
      rd(s, 1, I1{});
      step(I0{});
      rd(s, 2, I0{});
      step(I1{});
      rd(s, 3, I1{});
      step(I0{});
      step(I1{});
    }
    // the DMAs issued past the end must land before the block's LDS is freed
    __builtin_amdgcn_s_waitcnt(pdma::vmcnt_imm(0));
  }

  // fp32 partial: acc[i][j][v] = C[32 i + 8 (v / 4) + 4 hh + v % 4, n0 + 64 w + 32 j + l32]
  float* out = reinterpret_cast<float*>(p.c) + (int64_t)z * p.part_stride;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
      if (row >= p.m_store) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + 64 * wave + 32 * j + l32;
        if (col < p.n_store) out[row * p.ldc + col] = acc[i][j][v];
      }
    }
}

}  // namespace lora
