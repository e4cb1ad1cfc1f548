// gemm_w4_nf4.h - the whole-tile forward GEMM with an NF4 base weight
// expanded in its load stage: Y = alpha [X | sXA^T] [W | B]^T, W [d_out, d_in]
// given as 4-bit NormalFloat codes and one fp32 absmax per 64 consecutive
// elements of a row (QLoRA base of page "Unsloth教程：本地微调大模型速度提升数倍，
// 显存节省60%", section 显存优化策略; the dequantisation inside the GEMM of page
// "Unsloth自动化优化：无需手动调参的实现原理", section 5).
//
// Tile, waves, MFMA blocks, slot layout and fragment reads are those of
// gemm_w4_nt_kernel (256 x 256 tile, 4 waves of 128 x 128, 64-deep stages,
// rows of 128 bytes with chunk c at c ^ ((row >> 1) & 7)).  What differs is
// how W's tile reaches LDS.  A 64-deep stage of one W row is exactly one NF4
// block: 32 code bytes and one absmax.  Each thread owns one row of the
// B tile; its codes and absmax come into registers a stage ahead, and in the
// stage before their use the thread expands them: per code byte two lookups
// of the 16 fp32 code values, held one per lane (lane l has value l % 16) and
// read across lanes with ds_bpermute, two fp32 products with the absmax and
// one RNE pack to bf16 (the values of nf4_dequant, bit for bit), written as 8
// 16-byte pieces of the thread's LDS row into the B slot.  The rank segment's
// B tile (the adapter's B) is DMA'd as in the bf16 kernel.
//
// Why cross-lane reads and not a table in LDS: the compiler cannot tell an LDS
// read from the DMA writes in flight, and waited for every DMA before each
// table read (a whole-ring drain per stage); the permute reads no LDS memory.
// The expansion costs about 24 VALU instructions and 8 permutes per code
// dword, spread over the 48 MFMA slots of steps 0-2 (at most about 8 VALU
// instructions per MFMA, what one 32-cycle MFMA covers).
//
// LDS (128 KiB): A slots 0 and 1 (A(t) in slot t & 1, DMA'd), B slots 2 and 3
// (B(t) in slot 2 + (t & 1)).
//
// Stage t (four contraction steps of 16 MFMAs on A(t), B(t)):
//   steps 0-2: fragment reads of steps 1-3 (as the bf16 kernel); in the other
//              MFMA slots the expansion of B(t+1) from the thread's current
//              codes (into the slot of B(t-1), whose reads all came before the
//              barrier of stage t-1), or, for a rank-segment B(t+1), its DMA
//   wait for every load (A(t+1) and codes(t+2), both issued in stage t-1),
//   barrier
//   step 3:    reads of stage t+1's step-0 fragments; the next codes become
//              the current ones (register moves), the loads of codes(t+3)
//              into the next ones, and the DMA of A(t+2) into the slot of A(t)
// So codes are issued one stage ahead of the stage that expands them, which
// never waits on a load: the wait of the stage before covered them.  (Two
// register sets addressed by stage parity instead of the moves needed
// parity-dependent copies of the last stages, and the register allocator
// then spilled the accumulators.)
#pragma once

#include <type_traits>

#include "gemm_w4.h"
#include "gemm_w4_nt.h"

namespace lora {

namespace w4q {
constexpr int BK = 64;
constexpr int SLOT = w4::BM * 128;  // one operand tile of a stage (32 KiB)
constexpr int LDS = 4 * SLOT;       // 128 KiB
}  // namespace w4q

__global__ void __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_w4_nf4_kernel(const GemmArgs p) {
  using namespace w4;
  using w4nt::vmcnt_imm;
  using w4q::SLOT;
  constexpr int BKS = w4q::BK;
  __shared__ __attribute__((aligned(1024))) char smem[w4q::LDS];
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
  const int k2 = __builtin_amdgcn_readfirstlane((int)p.K2);

  // ---- A DMA (both segments) and the rank segment's B DMA, as in the bf16
  // NT kernel: instruction i (< 8) of wave w moves rows 64 w + 8 i + lane / 8,
  // the lane's logical chunk dce / dco for even / odd instructions ----
  const int dr = lane >> 3;
  const int dce = (lane & 7) ^ (lane >> 4), dco = (lane & 7) ^ ((lane >> 4) | 4);
  const int rowd = 64 * wave + dr;
  const char* ga1 = reinterpret_cast<const char*>(p.a1) + m0 * p.lda1 * 2;
  const char* ga2 = reinterpret_cast<const char*>(p.a2) + m0 * p.lda2 * 2;
  const char* gb2 = reinterpret_cast<const char*>(p.b2) + n0 * p.ldb2 * 2;
  const uint32_t ra1 = (uint32_t)(rowd * p.lda1 * 2), ra2 = (uint32_t)(rowd * p.lda2 * 2);
  const uint32_t rb2 = (uint32_t)(rowd * p.ldb2 * 2);
  const uint32_t va1[2] = {ra1 + (uint32_t)(dce * 16), ra1 + (uint32_t)(8 * p.lda1 * 2 + dco * 16)};
  const uint32_t isa1 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda1 * 2));
  const uint32_t isa2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.lda2 * 2));
  const uint32_t isb2 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * p.ldb2 * 2));
  const uint32_t oda2 = (uint32_t)(8 * p.lda2 * 2), odb2 = (uint32_t)(8 * p.ldb2 * 2);
  // op 0: A(u) (SEG2: u a stage of the rank segment, chunks at or past K2
  // read as zero); op 1: B(u) of the rank segment
  auto dma = [&](int u, int s, int op, int i, auto seg2_c) {
    constexpr bool SEG2 = decltype(seg2_c)::value;
    const int odd = i & 1, pair = i >> 1;
    const int dc = odd ? dco : dce;
    const char* base;
    uint32_t vo, is;
    if (op == 0 && !SEG2) {
      base = ga1 + (int64_t)u * (BKS * 2);
      vo = va1[odd];
      is = isa1;
    } else {
      const int tt = u - nk1;
      const int kk = tt * BKS + 8 * dc;
      const uint32_t kc = (uint32_t)(tt * BKS * 2 + dc * 16);
      if (op == 0) {
        base = ga2;
        vo = kk < k2 ? ra2 + (odd ? oda2 : 0u) + kc : w4::OOB;
        is = isa2;
      } else {
        base = gb2;
        vo = kk < k2 ? rb2 + (odd ? odb2 : 0u) + kc : w4::OOB;
        is = isb2;
      }
    }
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, BIG, 0x00020000);
    char* dst = smem + s * SLOT + (8 * wave + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, (int)(vo + (uint32_t)pair * is), 0, 0, 0);
  };

  // ---- NF4 codes: the thread's B-tile row.  Rows of 8 consecutive lanes
  // have 8 different (row >> 1) & 7, so each 16-byte LDS write of 8 lanes
  // lands in 8 different chunks ----
  const int rq = 64 * wave + 16 * (lane >> 4) + 2 * (lane & 7) + ((lane >> 3) & 1);
  const int sq = (rq >> 1) & 7;
  const __amdgpu_buffer_rsrc_t rcode = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.codes) + n0 * p.codes_ld, (short)0, BIG, 0x00020000);
  const __amdgpu_buffer_rsrc_t ram = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.absmax) + n0 * p.blocks_per_row, (short)0, BIG, 0x00020000);
  const uint32_t qo = (uint32_t)(rq * p.codes_ld), ao = (uint32_t)(rq * p.blocks_per_row * 4);
  // cq / am: the codes being expanded; nq / nam: the next stage's, in flight
  u32x4 cq[2], nq[2];
  float am, nam;
  auto load_codes = [&](int u, u32x4 (&q)[2], float& a) {
    q[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rcode, (int)(qo + 32u * u), 0, 0));
    q[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rcode, (int)(qo + 32u * u + 16u), 0, 0));
    a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ram, (int)(ao + 4u * u), 0, 0));
  };
  auto load_next = [&](int u) { load_codes(u, nq, nam); };
  // (the empty asm pins the moves here: left to itself the compiler renames
  // the sets and moves freshly loaded registers at the loop's end instead,
  // which waits for the loads just issued)
  auto take_next = [&] {
    cq[0] = nq[0];
    cq[1] = nq[1];
    am = nam;
    asm volatile("" : "+v"(cq[0]), "+v"(cq[1]), "+v"(am));
  };
  // Chunk c (elements 8c .. 8c+7 = code dword c) in three parts: lookups of
  // bytes 2h, 2h+1 (half h) into tv, products into pv, packs and the LDS
  // write into slot s.  Byte b gives elements (table[b >> 4], table[b & 15]):
  // the high nibble is the element first in memory.
  const int tabv = __builtin_bit_cast(int, tab16(p.nf4_table, lane & 15));
  float2 tv[8][4];
  auto lookup = [&](int c, int h) {
    const uint32_t w = cq[c >> 2][c & 3];
    // byte addresses (4 x nibble) of the high and low nibbles of every byte
    const uint32_t wh = (w >> 2) & 0x3c3c3c3cu, wl = (w << 2) & 0x3c3c3c3cu;
#pragma unroll
    for (int q = 2 * h; q < 2 * h + 2; ++q) {
      const int ah = (int)((wh >> (8 * q)) & 0xffu), al = (int)((wl >> (8 * q)) & 0xffu);
      tv[c][q] = make_float2(__builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(ah, tabv)),
                             __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(al, tabv)));
    }
  };
  auto product = [&](int c) {
#pragma unroll
    for (int q = 0; q < 4; ++q) tv[c][q] = make_float2(tv[c][q].x * am, tv[c][q].y * am);
  };
  auto store = [&](int c, int s) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(tv[c][q].x, tv[c][q].y);
    *reinterpret_cast<u32x4*>(smem + s * SLOT + rq * 128 + ((c ^ sq) << 4)) = o;
  };
  auto expand_all = [&](int s) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lookup(c, 0);
      lookup(c, 1);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      product(c);
      store(c, s);
    }
  };

  // ---- fragments (as the bf16 kernel) ----
  const uint32_t ra = (uint32_t)(wm * TM + l32) * 128;
  const uint32_t rb = (uint32_t)(wn * TN + l32) * 128;
  const int swz = (l32 >> 1) & 7;
  bf16x8 fa[2][FM], fb[2][FN];
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
  auto mf = [&](auto fsel, int q) {
    constexpr int f = decltype(fsel)::value;
    acc[q >> 2][q & 3] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][q >> 2], fb[f][q & 3], acc[q >> 2][q & 3], 0, 0, 0);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T_ = std::true_type;
  using F_ = std::false_type;

  // ---- prologue: B(0) expanded, A(0) landed; codes(1) current,
  // A(1) and codes(2) in flight ----
  load_codes(0, cq, am);
  if (nk1 > 1) load_next(1);
#pragma unroll
  for (int i = 0; i < 8; ++i) dma(0, 0, 0, i, F_{});
  expand_all(2);
  if (nk1 > 1) take_next();
  if (nk1 > 2) load_next(2);
  if (nk > 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (nk1 > 1)
        dma(1, 1, 0, i, F_{});
      else
        dma(1, 1, 0, i, T_{});
    }
  }
  // A(0) landed: at most codes(2) and A(1) may still fly
  if (nk > 1 && nk1 > 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(11));
  else if (nk > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
#pragma unroll
  for (int k = 0; k < 8; ++k) rd1(0, 2, 0, I0{}, k);

  // One stage.  DQ: B(t+1) expanded from the current codes (codes(t+1)),
  // else (RB) DMA'd from the rank segment when t+1 < nk.  CP: after the
  // barrier, codes(t+2) become current (1), and codes(t+3) are loaded (2).
  // AD: A(t+2) DMA'd from the first (1) or the rank (2) segment, or not (0).
  // NEXT: stage t+1 exists.  Every choice is made at compile time: uniform
  // branches between the MFMAs of a stage made the register allocator spill
  // the accumulators.
  auto stage = [&](int t, auto dq_c, auto rb_c, auto cp_c, auto ad_c, auto next_c) {
    constexpr bool DQ = decltype(dq_c)::value, RB = decltype(rb_c)::value;
    constexpr int CP = decltype(cp_c)::value, AD = decltype(ad_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    static_assert(!(DQ && RB) && (DQ || CP == 0), "one source for B(t+1); codes move only with expansions");
    const int sa = t & 1, sb = 2 + (t & 1);
    const int na = (t + 1) & 1, nb = 2 + ((t + 1) & 1);
    // MFMA slots g = 0 .. 47 (steps 0-2): chunk c's lookups at g = 6c and
    // 6c + 1, its products at 6c + 3, its packs and write at 6c + 4 (a
    // rank-segment B(t+1): its DMA instructions at g = 8 .. 15)
    auto extra = [&](int g) {
      if constexpr (DQ) {
        const int c = g / 6, ph = g % 6;
        if (ph == 0 || ph == 1) lookup(c, ph);
        if (ph == 3) product(c);
        if (ph == 4) store(c, nb);
      } else if constexpr (RB) {
        if (g >= 8 && g < 16) dma(t + 1, nb, 1, g - 8, T_{});
      }
    };
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mf(I0{}, q);
      if (q < 8) rd1(sa, sb, 1, I1{}, q);
      extra(q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mf(I1{}, q);
      if (q < 8) rd1(sa, sb, 2, I0{}, q);
      extra(16 + q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mf(I0{}, q);
      if (q < 8) rd1(sa, sb, 3, I1{}, q);
      extra(32 + q);
      fence();
    }
    // A(t+1) and codes(t+2) (a rank-segment B(t+1) too) have landed, and
    // every wave is done with stage t's slots
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mf(I1{}, q);
      if (q < 8) {
        if (NEXT) rd1(na, nb, 0, I0{}, q);
        if (CP >= 1 && q == 6) take_next();
        if (CP == 2 && q == 7) load_next(t + 3);
      } else if (AD == 1) {
        dma(t + 2, sa, 0, q - 8, F_{});
      } else if (AD == 2) {
        dma(t + 2, sa, 0, q - 8, T_{});
      }
      fence();
    }
  };
  using A0 = std::integral_constant<int, 0>;
  using A1 = std::integral_constant<int, 1>;
  using A2 = std::integral_constant<int, 2>;
  int t = 0;
  // W's stages while codes(t+3) is still a stage of W, then the one whose
  // codes(t+2) is W's last, then the one whose A(t+2) is the rank segment's
  // first
  for (; t + 3 < nk1; ++t) stage(t, T_{}, F_{}, A2{}, A1{}, T_{});
  if (t + 2 < nk1) stage(t++, T_{}, F_{}, A1{}, A1{}, T_{});
  if (t + 1 < nk1) stage(t++, T_{}, F_{}, A0{}, A2{}, T_{});
  // the rank segment (B(t+1) DMA'd), then the last stage
  for (; t + 2 < nk; ++t) stage(t, F_{}, T_{}, A0{}, A2{}, T_{});
  if (t + 1 < nk) stage(t++, F_{}, T_{}, A0{}, A0{}, T_{});
  stage(t, F_{}, F_{}, A0{}, A0{}, F_{});

  w4_epilogue<EPI_STORE>(p, acc, smem, m0, n0, p.c, p.ldc);
}

}  // namespace lora
