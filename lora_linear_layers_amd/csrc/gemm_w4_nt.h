// gemm_w4_nt.h - the whole-tile NT GEMM: C = alpha (A1 B1^T + A2 B2^T), both
// operands row-major with the contraction contiguous ([X | sXA^T] [W | B]^T of
// the forward, [G | sGB] [W^T | A^T]^T of the input gradient through W^T;
// page "UnSloth加速微调体验…", section 算子融合), 256 x 256 tiles, 4 waves of
// 128 x 128, 64-deep contraction stages.
//
// Global tiles go straight to LDS: buffer_load_dwordx4 with the lds flag
// writes each lane's 16 bytes at M0 + 16 lane with no register staging and
// no LDS write instruction.  One instruction moves 8 rows x 128 bytes, whole
// cache lines (measured on MI355X: 64-byte row pieces, as a 32-deep stage
// reads them, cost about 10% of the GEMM's time).
//
// LDS is a ring of 5 slots of 32 KiB, each one operand tile of a stage (256
// rows x 128 bytes): A of stage t in slot 2t mod 5, B in slot 2t+1 mod 5.
// Stage t runs four contraction steps of 16 MFMAs:
//   step 0: reads of step 1's fragments; DMA of half of A(t+2)
//   step 1: reads of step 2's fragments; DMA of the other half of A(t+2)
//   step 2: reads of step 3's fragments
//   wait for this wave's DMAs of stage t+1 (vmcnt), barrier
//   step 3: reads of stage t+1's step-0 fragments; DMA of B(t+2)
// A(t+2) goes to slot 2t+4 = slot of B(t-1), free since the barrier of stage
// t-1; B(t+2) to slot 2t+5 = slot of A(t), free since the barrier just
// passed (every read of stage t happened before it).  vmcnt counts a wave's
// own DMAs, which complete in order: at stage t's wait only A(t+2) (8) may
// still fly.  One barrier per 64-deep stage.
//
// Slot layout: row r at byte 128 r, logical 16-byte chunk c at physical chunk
// c ^ ((r >> 1) & 7).  DMA instruction i (< 8) of wave w moves rows
// 64 w + 8 i + lane / 8; the lane lands at physical chunk lane & 7, so it
// fetches logical chunk (lane & 7) ^ ((lane >> 4) | 4 (i & 1)).  Fragment
// reads (32 rows l32 of a block, chunk 2 s + l / 32) are conflict-free (a CPU
// model of the banks checks every lane).
//
// Group (EPI_GROUP): the forward GEMMs of several projections of one X in
// one launch.  Each block first finds its member (blocks [mem_tile0[g],
// mem_tile0[g + 1]), a scalar search over the kernel arguments) and takes
// that member's W, B, panel columns, rank, output and epilogue (RoPE or
// store); the main loop is the single GEMM's.  q, k and v of an attention
// block at 8192 tokens: 512 + 128 + 128 tiles in one launch instead of 512
// whole tiles plus two 128 x 128-tile launches.
//
// SwiGLU (EPI_SWIGLU): B-tile rows 32 b .. 32 b + 31 come from the gate's
// weight for even b and from the up's for odd b, rows n0 / 2 + 32 (b / 2) +
// .. of each, so MFMA blocks j = 0, 2 of a wave hold gate outputs and
// j = 1, 3 the up outputs of the same columns.  Wave w's B instructions
// i < 4 move gate rows n0 / 2 + 32 w + 8 i + lane / 8, i >= 4 the same rows
// of the up weight.  In the rank segment, columns [0, k2_split) belong to the
// gate's B and [k2_split, K2) to the up's (its own columns from 0).
#pragma once

#include <type_traits>

#include "gemm_w4.h"

namespace lora {

namespace w4nt {
constexpr int BK = 64;
constexpr int SLOT = w4::BM * 128;  // one operand tile of a stage
constexpr int NSLOT = 5;
constexpr int LDS = NSLOT * SLOT;
static_assert(w4::BM == w4::BN, "A and B tiles share the slot size");
static_assert(LDS >= 2 * w4::BM * 64 * 4, "the RoPE epilogue stages its cos/sin rows in the ring");

// s_waitcnt immediate: vmcnt = n (0..63), expcnt and lgkmcnt unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }
}  // namespace w4nt

typedef __attribute__((address_space(3))) void lds_void_t;

template <int EPI>
__global__ void __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_w4_nt_kernel(const GemmArgs p) {
  using namespace w4;
  using w4nt::NSLOT;
  using w4nt::SLOT;
  using w4nt::vmcnt_imm;
  constexpr int BKS = w4nt::BK;
  static_assert(EPI == EPI_STORE || EPI == EPI_ROPE || EPI == EPI_SWIGLU || EPI == EPI_GROUP,
                "store, RoPE, SwiGLU or group epilogue");
  constexpr bool SW = EPI == EPI_SWIGLU;
  constexpr bool GR = EPI == EPI_GROUP;
  __shared__ __attribute__((aligned(1024))) char smem[w4nt::LDS];
  // keep the MFMA accumulators in the accumulation registers
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  // the block's GEMM: one projection, or (group) the member whose tiles hold
  // this block, all of its parameters uniform
  int bid = blockIdx.x;
  const void* pa2 = p.a2;
  const void* pb1 = p.b1;
  const void* pb2 = p.b2;
  int64_t ldb2 = p.ldb2, K2 = p.K2;
  void* pc = p.c;
  int64_t ldc = p.ldc;
  int rope = 0;
  if constexpr (GR) {
    int g = 0;
    for (int i = 1; i < p.n_mem; ++i) g = bid >= p.mem_tile0[i] ? i : g;
    bid -= p.mem_tile0[g];
    pa2 = p.mem_a2[g];
    pb1 = p.mem_b1[g];
    pb2 = p.mem_b2[g];
    ldb2 = p.mem_ldb2[g];
    K2 = p.mem_k2[g];
    pc = p.mem_c[g];
    ldc = p.mem_ldc[g];
    rope = p.mem_rope[g];
  }
  const int64_t m0 = (int64_t)(bid % p.tiles_m) * BM;
  const int64_t n0 = (int64_t)(bid / p.tiles_m) * BN;
  const int nk1 = (int)(p.K1 / BKS);
  const int nk = nk1 + (int)((K2 + BKS - 1) / BKS);

  // ---- DMA addressing ----
  // dr: the lane's row within an instruction's 8; dce / dco: its logical
  // chunk for even / odd instructions.  Offsets of instruction 0 (even) and
  // 1 (odd); instruction i adds (i >> 1) * is (SwiGLU B: ((i & 3) >> 1) * is,
  // the weight chosen by i >> 2).
  const int dr = lane >> 3;
  const int dce = (lane & 7) ^ (lane >> 4), dco = (lane & 7) ^ ((lane >> 4) | 4);
  const int64_t nb0 = SW ? n0 / 2 : n0;  // first weight row of the tile
  const int rowa = 64 * wave + dr;
  const int rowb = SW ? 32 * wave + dr : 64 * wave + dr;
  const char* ga1 = reinterpret_cast<const char*>(p.a1) + m0 * p.lda1 * 2;
  const char* ga2 = reinterpret_cast<const char*>(pa2) + m0 * p.lda2 * 2;
  const char* gb1 = reinterpret_cast<const char*>(pb1) + nb0 * p.ldb1 * 2;
  const char* gb2 = reinterpret_cast<const char*>(pb2) + nb0 * ldb2 * 2;
  const char* gb1u = SW ? reinterpret_cast<const char*>(p.b1u) + nb0 * p.ldb1 * 2 : gb1;
  const char* gb2u = SW ? reinterpret_cast<const char*>(p.b2u) + nb0 * p.ldb2u * 2 : gb2;
  // row parts of the lane offsets (+ 8 rows for odd instructions)
  const uint32_t ra1 = (uint32_t)(rowa * p.lda1 * 2), ra2 = (uint32_t)(rowa * p.lda2 * 2);
  const uint32_t rb1 = (uint32_t)(rowb * p.ldb1 * 2), rb2 = (uint32_t)(rowb * ldb2 * 2);
  const uint32_t rb2u = SW ? (uint32_t)(rowb * p.ldb2u * 2) : 0u;
  const uint32_t va1[2] = {ra1 + (uint32_t)(dce * 16), ra1 + (uint32_t)(8 * p.lda1 * 2 + dco * 16)};
  const uint32_t vb1[2] = {rb1 + (uint32_t)(dce * 16), rb1 + (uint32_t)(8 * p.ldb1 * 2 + dco * 16)};
  // strides between a wave's instruction pairs, pinned in scalar registers
  const uint32_t isa1 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda1 * 2));
  const uint32_t isa2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda2 * 2));
  const uint32_t isb1 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb1 * 2));
  const uint32_t isb2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * ldb2 * 2));
  const uint32_t isb2u = SW ? __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb2u * 2)) : 0u;
  const uint32_t oda2 = (uint32_t)(8 * p.lda2 * 2), odb2 = (uint32_t)(8 * ldb2 * 2);
  const uint32_t odb2u = SW ? (uint32_t)(8 * p.ldb2u * 2) : 0u;
  const int k2 = __builtin_amdgcn_readfirstlane((int)K2);
  const int k2s = SW ? __builtin_amdgcn_readfirstlane((int)p.k2_split) : 0;

  // One DMA: stage u, operand op (0 A, 1 B), instruction i (< 8), slot s.
  // SEG2: u is a stage of the rank segment, whose chunks at or past K2 come
  // back as zero through an out-of-range offset.
  auto dma = [&](int u, int s, int op, int i, auto seg2_c) {
    constexpr bool SEG2 = decltype(seg2_c)::value;
    const bool up = SW && op == 1 && i >= 4;
    const int odd = i & 1;
    const int pair = (SW && op == 1) ? ((i & 3) >> 1) : (i >> 1);
    const int dc = odd ? dco : dce;
    const char* base;
    uint32_t vo, is;
    if constexpr (!SEG2) {
      base = (op == 0 ? ga1 : (up ? gb1u : gb1)) + (int64_t)u * (BKS * 2);
      vo = op == 0 ? va1[odd] : vb1[odd];
      is = op == 0 ? isa1 : isb1;
    } else {
      const int tt = u - nk1;
      const int kk = tt * BKS + 8 * dc;  // the lane's first rank column
      const uint32_t kc = (uint32_t)(tt * BKS * 2 + dc * 16);
      if (op == 0) {
        base = ga2;
        vo = kk < k2 ? ra2 + (odd ? oda2 : 0u) + kc : w4::OOB;
        is = isa2;
      } else if (!SW) {
        base = gb2;
        vo = kk < k2 ? rb2 + (odd ? odb2 : 0u) + kc : w4::OOB;
        is = isb2;
      } else if (!up) {
        base = gb2;
        vo = kk < k2s ? rb2 + (odd ? odb2 : 0u) + kc : w4::OOB;
        is = isb2;
      } else {
        base = gb2u;
        vo = kk >= k2s && kk < k2 ? rb2u + (odd ? odb2u : 0u) + (uint32_t)((kk - k2s) * 2) : w4::OOB;
        is = isb2u;
      }
    }
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, BIG, 0x00020000);
    char* dst = smem + s * SLOT + (8 * wave + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, (int)(vo + (uint32_t)pair * is), 0, 0, 0);
  };

  // ---- fragments ----
  // A rows wm*TM + 32 blk + l32 and B rows wn*TN + 32 blk + l32 all have
  // (row >> 1) & 7 = (l32 >> 1) & 7.
  const uint32_t ra = (uint32_t)(wm * TM + l32) * 128;
  const uint32_t rb = (uint32_t)(wn * TN + l32) * 128;
  const int swz = (l32 >> 1) & 7;
  bf16x8 fa[2][FM], fb[2][FN];
  // read k of step s (k < 4: A block k from slot sa, else B block k - 4 from
  // slot sb) into set f
  auto rd1 = [&](int sa, int sb, int s, auto fsel, int k) {
    constexpr int f = decltype(fsel)::value;
    const uint32_t c = (uint32_t)(((2 * s + hh) ^ swz) << 4);
    if (k < FM)
      fa[f][k] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(smem + sa * SLOT + ra + c + k * 32 * 128));
    else
      fb[f][k - FM] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(smem + sb * SLOT + rb + c + (k - FM) * 32 * 128));
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // MFMA number q (0..15) of a contraction step: block (q / 4, q % 4)
  auto mf = [&](auto fsel, int q) {
    constexpr int f = decltype(fsel)::value;
    acc[q >> 2][q & 3] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][q >> 2], fb[f][q & 3], acc[q >> 2][q & 3], 0, 0, 0);
  };
  // issue-order fence: nothing is scheduled across it
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  if (nk > 0) {
    // prologue: stages 0 and 1 in flight (slots 0 .. 3); wait for stage 0
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u < nk) {
#pragma unroll
        for (int op = 0; op < 2; ++op)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (u < nk1)
              dma(u, 2 * u + op, op, i, F_{});
            else
              dma(u, 2 * u + op, op, i, T_{});
          }
      }
    }
    if (nk >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 8; ++k) rd1(0, 1, 0, I0{}, k);

    // One stage.  ISSUE: 0 none, 1 stage t+2 of the main segment, 2 of the
    // rank segment.  NEXT: stage t+1 exists.
    auto stage = [&](int t, auto issue_c, auto next_c) {
      constexpr int ISSUE = decltype(issue_c)::value;
      constexpr bool NEXT = decltype(next_c)::value;
      using S2 = std::integral_constant<bool, ISSUE == 2>;
      const int sa = (2 * t) % NSLOT, sb = (2 * t + 1) % NSLOT;
      const int na = (2 * t + 2) % NSLOT, nb = (2 * t + 3) % NSLOT;
      const int fa2 = (2 * t + 4) % NSLOT;  // A(t+2): the slot of B(t-1)
      const int fb2 = sa;                   // B(t+2): the slot of A(t)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I0{}, q);
        if (q < 8)
          rd1(sa, sb, 1, I1{}, q);
        else if (ISSUE && (q & 1) == 0)
          dma(t + 2, fa2, 0, (q - 8) >> 1, S2{});
        fence();
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I1{}, q);
        if (q < 8)
          rd1(sa, sb, 2, I0{}, q);
        else if (ISSUE && (q & 1) == 0)
          dma(t + 2, fa2, 0, 4 + ((q - 8) >> 1), S2{});
        fence();
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I0{}, q);
        if (q < 8) rd1(sa, sb, 3, I1{}, q);
        fence();
      }
      // stage t+1 has landed (only A(t+2) may still fly), and every wave is
      // done with stage t's slots
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(ISSUE ? 8 : 0));
      lds_barrier();
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I1{}, q);
        if (q < 8) {
          if (NEXT) rd1(na, nb, 0, I0{}, q);
        } else if (ISSUE) {
          dma(t + 2, fb2, 1, q - 8, S2{});
        }
        fence();
      }
    };
    using N0 = std::integral_constant<int, 0>;
    using N1 = std::integral_constant<int, 1>;
    using N2 = std::integral_constant<int, 2>;
    int t = 0;
    for (; t + 2 < nk1; ++t) stage(t, N1{}, T_{});
    for (; t + 2 < nk; ++t) stage(t, N2{}, T_{});
    if (t + 1 < nk) stage(t++, N0{}, T_{});
    stage(t, N0{}, F_{});
  }

  // (the RoPE epilogue reuses the ring for its cos/sin rows after a barrier)
  if constexpr (GR) {
    if (rope)
      w4_epilogue<EPI_ROPE>(p, acc, smem, m0, n0, pc, ldc);
    else
      w4_epilogue<EPI_STORE>(p, acc, smem, m0, n0, pc, ldc);
  } else {
    w4_epilogue<EPI>(p, acc, smem, m0, n0, pc, ldc);
  }
}

}  // namespace lora
