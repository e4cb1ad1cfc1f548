// gemm_w4_nt.h - the whole-tile NT GEMM: C = alpha (A1 B1^T + A2 B2^T), both
// operands row-major with the contraction contiguous ([X | sXA^T] [W | B]^T of
// the forward, [G | sGB] [W^T | A^T]^T of the input gradient through W^T;
// page "UnSloth加速微调体验…", section 算子融合), 256 x 256 tiles, 4 waves of
// 128 x 128, 32-deep contraction stages.
//
// Global tiles go straight to LDS: buffer_load_dwordx4 with the lds flag
// writes each lane's 16 bytes at M0 + 16 lane of the LDS with no register
// staging and no LDS write instruction, so the LDS port serves only the
// fragment reads and the DMA stream.  The DMA runs LEAD = 3 stages ahead
// through a ring of 4 LDS buffers of 32 KiB (A 256 rows x 64 bytes, then B):
// measured on MI355X, a lead of 2 leaves the waves waiting on HBM latency, a
// lead of 4 (five buffers, all 160 KiB) gains nothing over 3.
//
// Stage t, ring buffer t % 4, two contraction steps of 16 MFMAs each:
//   step 0: MFMAs of step 0; the 8 fragment reads of step 1 (after the first
//           8 MFMAs), then 4 DMAs of stage t+3's A tile into buffer (t+3) % 4
//   wait for stage t+1's DMAs (vmcnt), barrier
//   step 1: MFMAs of step 1; the 8 reads of stage t+1's step-0 fragments,
//           then 4 DMAs of stage t+3's B tile
// Buffer (t+3) % 4 = (t-1) % 4 was last read in stage t-1's step 0, which
// every wave finished before the barrier of stage t-1, so the DMA may
// overwrite it.  vmcnt counts a wave's own DMAs, completed in order: at
// stage t's barrier stages t+2 (8) and t+3's A (4) may still fly.
//
// DMA lane mapping: instruction i (< 4) of wave w moves tile rows
// 16 (4 w + i) + lane / 4, lane lands at byte 16 lane of the instruction's
// 1 KiB block, i.e. row 16 (4 w + i) + lane / 4, physical chunk lane & 3.
// The LDS row holds logical 16-byte chunk c at physical chunk
// c ^ ((row >> 2) & 3), so the lane fetches logical chunk
// (lane & 3) ^ ((lane >> 4) & 3).  A fragment read (32 rows, one chunk each,
// rows l32 of a 32-row block) then touches 8 rows per bank group and is
// conflict-free (checked for every lane by a CPU model of the banks).
//
// SwiGLU (EPI_SWIGLU): B-tile rows 32 b .. 32 b + 31 come from the gate's
// weight for even b and from the up's for odd b, rows n0 / 2 + 32 (b / 2) +
// .. of each, so MFMA blocks j = 0, 2 of a wave hold gate outputs and
// j = 1, 3 the up outputs of the same columns.  Wave w's B instructions
// i = 0, 1 move gate rows n0 / 2 + 32 w + 16 i + lane / 4, i = 2, 3 the same
// rows of the up weight.  In the rank segment, columns [0, k2_split) belong
// to the gate's B and [k2_split, K2) to the up's (its own columns from 0).
#pragma once

#include <type_traits>

#include "gemm_w4.h"

namespace lora {

namespace w4nt {
constexpr int BK = 32;
constexpr int A_BYTES = w4::BM * 64, B_BYTES = w4::BN * 64, STAGE = A_BYTES + B_BYTES;
constexpr int NBUF = 4, LEAD = NBUF - 1;
constexpr int LDS = NBUF * STAGE;
static_assert(LDS >= 2 * w4::BM * 64 * 4, "the RoPE epilogue stages its cos/sin rows in the ring");

// s_waitcnt immediate: vmcnt = n (0..63), expcnt and lgkmcnt unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }
}  // namespace w4nt

typedef __attribute__((address_space(3))) void lds_void_t;

template <int EPI>
__global__ void __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_w4_nt_kernel(const GemmArgs p) {
  using namespace w4;
  using w4nt::A_BYTES;
  using w4nt::LEAD;
  using w4nt::NBUF;
  using w4nt::STAGE;
  using w4nt::vmcnt_imm;
  constexpr int BKS = w4nt::BK;
  static_assert(EPI == EPI_STORE || EPI == EPI_ROPE || EPI == EPI_SWIGLU, "store, RoPE or SwiGLU epilogue");
  constexpr bool SW = EPI == EPI_SWIGLU;
  __shared__ __attribute__((aligned(1024))) char smem[w4nt::LDS];
  // keep the MFMA accumulators in the accumulation registers
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int bid = blockIdx.x;
  const int64_t m0 = (int64_t)(bid % p.tiles_m) * BM;
  const int64_t n0 = (int64_t)(bid / p.tiles_m) * BN;
  const int nk1 = (int)(p.K1 / BKS);
  const int nk = nk1 + (int)((p.K2 + BKS - 1) / BKS);

  // ---- DMA addressing ----
  // dr: the lane's row within an instruction's 16, dc: its logical chunk.
  // Row offsets of instruction 0; instruction i adds i * is (SwiGLU B:
  // (i & 1) * is, the weight chosen by i >> 1).
  const int dr = lane >> 2, dc = (lane & 3) ^ ((lane >> 4) & 3);
  const int64_t nb0 = SW ? n0 / 2 : n0;  // first weight row of the tile
  const int rowa = 64 * wave + dr;
  const int rowb = SW ? 32 * wave + dr : 64 * wave + dr;
  const char* ga1 = reinterpret_cast<const char*>(p.a1) + m0 * p.lda1 * 2;
  const char* ga2 = reinterpret_cast<const char*>(p.a2) + m0 * p.lda2 * 2;
  const char* gb1 = reinterpret_cast<const char*>(p.b1) + nb0 * p.ldb1 * 2;
  const char* gb2 = reinterpret_cast<const char*>(p.b2) + nb0 * p.ldb2 * 2;
  const char* gb1u = SW ? reinterpret_cast<const char*>(p.b1u) + nb0 * p.ldb1 * 2 : gb1;
  const char* gb2u = SW ? reinterpret_cast<const char*>(p.b2u) + nb0 * p.ldb2u * 2 : gb2;
  const uint32_t va1 = (uint32_t)(rowa * p.lda1 * 2 + dc * 16);
  const uint32_t va2 = (uint32_t)(rowa * p.lda2 * 2 + dc * 16);
  const uint32_t vb1 = (uint32_t)(rowb * p.ldb1 * 2 + dc * 16);
  const uint32_t vb2 = (uint32_t)(rowb * p.ldb2 * 2 + dc * 16);
  const uint32_t vb2u = SW ? (uint32_t)(rowb * p.ldb2u * 2) : 0u;
  // strides between a wave's instructions, pinned in scalar registers
  const uint32_t isa1 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda1 * 2));
  const uint32_t isa2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda2 * 2));
  const uint32_t isb1 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb1 * 2));
  const uint32_t isb2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb2 * 2));
  const uint32_t isb2u = SW ? __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb2u * 2)) : 0u;
  const int k2 = __builtin_amdgcn_readfirstlane((int)p.K2);
  const int k2s = SW ? __builtin_amdgcn_readfirstlane((int)p.k2_split) : 0;

  // One DMA: stage u, operand op (0 A, 1 B), instruction i, ring buffer b.
  // SEG2: u is a stage of the rank segment, whose chunks at or past K2 come
  // back as zero through an out-of-range offset.
  auto dma = [&](int u, int b, int op, int i, auto seg2_c) {
    constexpr bool SEG2 = decltype(seg2_c)::value;
    const bool up = SW && op == 1 && i >= 2;
    const int ii = (SW && op == 1) ? (i & 1) : i;
    const char* base;
    uint32_t vo, is;
    if constexpr (!SEG2) {
      base = (op == 0 ? ga1 : (up ? gb1u : gb1)) + (int64_t)u * (BKS * 2);
      vo = op == 0 ? va1 : vb1;
      is = op == 0 ? isa1 : isb1;
    } else {
      const int tt = u - nk1;
      const int kk = tt * BKS + 8 * dc;  // the lane's first rank column
      if (op == 0) {
        base = ga2;
        vo = kk < k2 ? va2 + (uint32_t)(tt * BKS * 2) : w4::OOB;
        is = isa2;
      } else if (!SW) {
        base = gb2;
        vo = kk < k2 ? vb2 + (uint32_t)(tt * BKS * 2) : w4::OOB;
        is = isb2;
      } else if (!up) {
        base = gb2;
        vo = kk < k2s ? vb2 + (uint32_t)(tt * BKS * 2) : w4::OOB;
        is = isb2;
      } else {
        base = gb2u;
        vo = kk >= k2s && kk < k2 ? vb2u + (uint32_t)((kk - k2s) * 2) : w4::OOB;
        is = isb2u;
      }
    }
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, BIG, 0x00020000);
    char* dst = smem + b * STAGE + op * A_BYTES + (4 * wave + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, (int)(vo + (uint32_t)ii * is), 0, 0, 0);
  };

  // ---- fragments ----
  // lane reads row 32 blk + l32 of its wave's half, logical chunk 2 s + hh
  const int sw = (l32 >> 2) & 3;
  const uint32_t oa0 = (uint32_t)(wm * TM + l32) * 64 + (uint32_t)(((0 + hh) ^ sw) << 4);
  const uint32_t oa1 = (uint32_t)(wm * TM + l32) * 64 + (uint32_t)(((2 + hh) ^ sw) << 4);
  const uint32_t ob0 = (uint32_t)A_BYTES + (uint32_t)(wn * TN + l32) * 64 + (uint32_t)(((0 + hh) ^ sw) << 4);
  const uint32_t ob1 = (uint32_t)A_BYTES + (uint32_t)(wn * TN + l32) * 64 + (uint32_t)(((2 + hh) ^ sw) << 4);
  bf16x8 fa[2][FM], fb[2][FN];
  // read k of step s (k < 4: A block k, else B block k - 4) of buffer b into set f
  auto rd1 = [&](int b, int s, auto fsel, int k) {
    constexpr int f = decltype(fsel)::value;
    const char* sb = smem + b * STAGE;
    if (k < FM)
      fa[f][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + (s ? oa1 : oa0) + k * 32 * 64));
    else
      fb[f][k - FM] =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + (s ? ob1 : ob0) + (k - FM) * 32 * 64));
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
    // prologue: stages 0 .. LEAD-1 in flight; wait for stage 0 only
#pragma unroll
    for (int u = 0; u < LEAD; ++u) {
      if (u < nk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (u < nk1) {
            dma(u, u, 0, i, F_{});
            dma(u, u, 1, i, F_{});
          } else {
            dma(u, u, 0, i, T_{});
            dma(u, u, 1, i, T_{});
          }
        }
      }
    }
    static_assert(LEAD == 3, "prologue waits are written for a lead of 3");
    if (nk >= 3)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
    else if (nk == 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 8; ++k) rd1(0, 0, I0{}, k);

    // One stage.  ISSUE: 0 none, 1 stage t + LEAD of the main segment, 2 of
    // the rank segment.  VM: DMAs that may still fly at the mid-stage wait
    // (everything after stage t+1).  NEXT: stage t+1 exists.
    auto stage = [&](int t, auto issue_c, auto vm_c, auto next_c) {
      constexpr int ISSUE = decltype(issue_c)::value, VM = decltype(vm_c)::value;
      constexpr bool NEXT = decltype(next_c)::value;
      using S2 = std::integral_constant<bool, ISSUE == 2>;
      const int cur = t % NBUF, nxt = (t + 1) % NBUF, far = (t + LEAD) % NBUF;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I0{}, q);
        if (q < 8)
          rd1(cur, 1, I1{}, q);
        else if (ISSUE && (q & 1) == 0)
          dma(t + LEAD, far, 0, (q - 8) >> 1, S2{});
        fence();
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(VM));
      lds_barrier();
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        mf(I1{}, q);
        if (q < 8) {
          if (NEXT) rd1(nxt, 0, I0{}, q);
        } else if (ISSUE && (q & 1) == 0) {
          dma(t + LEAD, far, 1, (q - 8) >> 1, S2{});
        }
        fence();
      }
    };
    using N0 = std::integral_constant<int, 0>;
    using N1 = std::integral_constant<int, 1>;
    using N2 = std::integral_constant<int, 2>;
    int t = 0;
    for (; t + LEAD < nk1; ++t) stage(t, N1{}, std::integral_constant<int, 12>{}, T_{});
    for (; t + LEAD < nk; ++t) stage(t, N2{}, std::integral_constant<int, 12>{}, T_{});
    // the last stages issue nothing; with j stages after it, a stage lets the
    // DMAs of j - 1 of them fly
    if (nk - 1 - t == 2) stage(t++, N0{}, std::integral_constant<int, 8>{}, T_{});
    if (nk - 1 - t == 1) stage(t++, N0{}, std::integral_constant<int, 0>{}, T_{});
    stage(t, N0{}, std::integral_constant<int, 0>{}, F_{});
  }

  // (the RoPE epilogue reuses the ring for its cos/sin rows after a barrier)
  w4_epilogue<EPI>(p, acc, smem, m0, n0);
}

}  // namespace lora
