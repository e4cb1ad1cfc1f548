// gemm_w4.h - the whole-tile bf16 GEMMs of the fused LoRA linear layer on
// gfx950: 256 x 256 tiles, 4 waves of 128 x 128, one wave per SIMD,
// v_mfma_f32_32x32x16_bf16 with the accumulators in the accumulation
// registers.
//
// Same contraction as gemm.h (two segments into one fp32 accumulator: the
// forward [X | sXA^T] [W | B]^T and the input gradient [G | sGB] [W ; A] of
// page "UnSloth加速微调体验…", section 算子融合), for the shapes that
// dominate the layer: every tile whole in m and n and the first segment a
// whole number of 64-wide stages; the rank-r segment may be ragged.
//
// This file holds what both orientations share (the tile constants and the
// epilogues) and the NN kernel, whose second operand is stored contraction-
// major (the input gradient through W when no W^T is at hand).  The NT
// kernel, which every large forward GEMM and the input gradient through W^T
// run, is in gemm_w4_nt.h.
//
// Why this shape.  Measured with the SQ counters on MI355X, the GEMM runs
// power-limited (about 1.8 GHz) and what separates a fast kernel from a slow
// one is the share of cycles the MFMA pipe is busy; LDS traffic is the main
// thing that steals those cycles.  A 128 x 128 wave tile reads each LDS row
// twice per stage (a 64 x 128 one three times on average), and with one wave
// per SIMD each wave owns 512 registers: 256 accumulators, two sets of
// fragments and the register staging of the next global tile, so nothing
// spills and no loop-invariant address is recomputed.
//
// 32x32x16 MFMA: A lane l holds row l % 32, contraction 8 (l / 32) .. +7; B
// lane l holds column l % 32, the same contraction range; the 16 fp32 results
// of lane l are rows 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
#pragma once

#include <type_traits>

#include "gemm.h"

namespace lora {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace w4 {
constexpr int BM = 256, BN = 256;
constexpr int NT = 256;
constexpr int TM = 128, TN = 128;          // wave tile, 2 x 2 waves
constexpr int FM = TM / 32, FN = TN / 32;  // 4 x 4 MFMA blocks
constexpr int BK = 64;                     // NN stage depth
constexpr int A_STAGE = BM * 128, B_STAGE = BN * 128;
constexpr int B_BASE = 2 * A_STAGE;
constexpr int LDS = 2 * (A_STAGE + B_STAGE);
constexpr int BIG = 0x40000000;        // resource size with nothing masked
constexpr uint32_t OOB = 0x40000000u;  // lane offset that reads zero
}  // namespace w4

// ---------------------------------------------------------------------------
// Epilogues of a 256 x 256 tile from the accumulators of the calling wave:
//   acc[i][j][v] = C[row, col], row = m0 + wm*TM + 32 i + 8 (v / 4) + 4 hh + v % 4,
//                               col = n0 + wn*TN + 32 j + l32
// (wm, wn the wave's position, l32 / hh the lane's).  The lane indices are
// derived afresh from threadIdx: values kept from before the main loop would
// be spilled, and each reload's wait between the stores also waits for every
// store issued before it.  smem (at least 2 x 256 x 64 floats) must be free:
// the RoPE epilogue stages its cos/sin rows there.
//   EPI_STORE:  C = alpha acc, bf16.
//   EPI_ROPE:   a wave's 128 columns are one head; columns c and c + 64 are
//               rotated together by the angle of the row's position (page
//               "UnSloth加速微调体验…", section RoPE缓存集成).
//   EPI_SWIGLU: MFMA blocks j = 0, 2 hold the gate and j = 1, 3 the up
//               projection of output columns n0 / 2 + 64 wn + 32 (j / 2) + l32;
//               C = silu(g) u, and g / u are also stored to cg / cu when
//               set.
template <int EPI>
__device__ __forceinline__ void w4_epilogue(const GemmArgs& p, f32x16 (&acc)[w4::FM][w4::FN], char* smem,
                                            int64_t m0, int64_t n0, void* c_out, int64_t ldc) {
  using namespace w4;
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  int te = threadIdx.x;
  asm volatile("" : "+v"(te));
  const int l32 = te & 31, hh = (te >> 5) & 1;
  const int wm = __builtin_amdgcn_readfirstlane(te >> 7), wn = __builtin_amdgcn_readfirstlane((te >> 6) & 1);
  const int64_t rbase = m0 + wm * TM + 4 * hh;
  const int64_t cbase = n0 + wn * TN + l32;
  uint16_t* out = reinterpret_cast<uint16_t*>(c_out);
  if constexpr (EPI == EPI_ROPE) {
    // The tile's 256 rows of the cos/sin cache (64 frequencies each) go to LDS
    // first: the tile's positions (one per thread) through LDS, then each
    // thread's 32 16-byte cache loads all in flight together.  (A load per
    // position read and branch had cost the launch 20 us more at the
    // Llama-3-8B attention shapes.)
    // Row q's 64 values sit rotated by 32 when (q >> 2) & 1, so the reads
    // below (rows q and q + 4, 32 consecutive frequencies each) hit distinct
    // banks.
    __syncthreads();
    float* cs_l = reinterpret_cast<float*>(smem);
    float* sn_l = cs_l + BM * 64;
    int32_t* pos_l = reinterpret_cast<int32_t*>(sn_l + BM * 64);
    static_assert(NT == BM, "one position per thread");
    pos_l[te] = p.pos[m0 + te];
    __syncthreads();
    {
      // thread t takes the 16-byte chunks (q, ch) = ((t + 256 k) / 16,
      // (t + 256 k) % 16), k < 16, of both the cos and the sin row of tile row
      // q: the 16 positions first (one wait), then 32 buffer loads with no
      // branch, cos and sin through two wave-uniform resources sharing one
      // 32-bit offset; a position outside the cache gets an offset past the
      // resource, which reads zeros
      // max_pos < 2^23 (validated on the host): every row ends below 2^31 and
      // 2^31 lies past the resource for any cache size
      const int nrec = (int)(p.max_pos * 256);
      constexpr uint32_t PAST = 0x80000000u;
      const __amdgpu_buffer_rsrc_t rc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.cosc), (short)0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.sinc), (short)0, nrec, 0x00020000);
      const int ch = te & 15;
      uint32_t off[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int32_t ps = pos_l[(te + NT * k) >> 4];
        off[k] = rope_pos_ok(ps, p.max_pos) ? (uint32_t)ps * 256u + 16u * ch : PAST;
      }
      u32x4 bc[16], bs[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        bc[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (int)off[k], 0, 0));
        bs[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[k], 0, 0));
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int q = (te + NT * k) >> 4;
        const int o = q * 64 + ((4 * ch + 32 * ((q >> 2) & 1)) & 63);
        *reinterpret_cast<u32x4*>(cs_l + o) = bc[k];
        *reinterpret_cast<u32x4*>(sn_l + o) = bs[k];
      }
    }
    __syncthreads();
    // column 32 j + l32 (j < 2) pairs with column 32 (j + 2) + l32 = +64, both
    // in this lane
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        // 4 rows at a time: 16 reads in flight, then their 16 stores
        float cs[4][2], sn[4][2];
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int q = wm * TM + 32 * i + 8 * vb + vv + 4 * hh;
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const int li = q * 64 + ((32 * j + l32 + 32 * ((q >> 2) & 1)) & 63);
            cs[vv][j] = cs_l[li];
            sn[vv][j] = sn_l[li];
          }
        }
        fence();
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int v = 4 * vb + vv;
          const int64_t row = m0 + wm * TM + 32 * i + 8 * vb + vv + 4 * hh;
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const int64_t col = cbase + 32 * j;
            const float z1 = acc[i][j][v] * p.alpha, z2 = acc[i][j + FN / 2][v] * p.alpha;
            out[row * ldc + col] = f2bf(z1 * cs[vv][j] - z2 * sn[vv][j]);
            out[row * ldc + col + 64] = f2bf(z2 * cs[vv][j] + z1 * sn[vv][j]);
          }
        }
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const int64_t hbase = n0 / 2 + 64 * wn + l32;
    uint16_t* og = reinterpret_cast<uint16_t*>(p.cg);
    uint16_t* ou = reinterpret_cast<uint16_t*>(p.cu);
    // GU: 0 neither G nor U stored, 1 both, 2 either one (tested per store)
    auto emit = [&](auto gu_c) {
      constexpr int GU = decltype(gu_c)::value;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const float g = acc[i][2 * jj][v], u = acc[i][2 * jj + 1][v];
            const int64_t o = row * ldc + hbase + 32 * jj;
            // silu(g) u with the hardware reciprocal (one instruction; the
            // division's IEEE sequence is ten, per element of the epilogue)
            out[o] = f2bf(g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u);
            if constexpr (GU == 1) {
              og[o] = f2bf(g);
              ou[o] = f2bf(u);
            } else if constexpr (GU == 2) {
              if (og) og[o] = f2bf(g);
              if (ou) ou[o] = f2bf(u);
            }
          }
        }
    };
    if (og && ou)
      emit(std::integral_constant<int, 1>{});
    else if (!og && !ou)
      emit(std::integral_constant<int, 0>{});
    else
      emit(std::integral_constant<int, 2>{});
  } else {
    static_assert(EPI == EPI_STORE, "store, RoPE or SwiGLU epilogue");
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
#pragma unroll
        for (int j = 0; j < FN; ++j) out[row * ldc + cbase + 32 * j] = f2bf(acc[i][j][v] * p.alpha);
      }
  }
}

// ---------------------------------------------------------------------------
// NN kernel: C = alpha (A1 B1 + A2 B2), A row-major [m][k], B contraction-
// major [k][n] (W itself for the input gradient G W; A of the adapter for
// the rank segment), 256 x 256 x 64 stages, register-staged global tiles.
//
// Per stage t (LDS buffer t & 1) each wave runs four contraction steps of 16
// MFMAs, each MFMA followed by one memory operation:
//   step 0: reads of step 1's fragments, then LDS writes of stage t+1's A
//           tile (from registers, into the other buffer)
//   step 1: reads of step 2's fragments, then stage t+1's B tile
//   step 2: reads of step 3's fragments, then global loads of a later A tile
//   barrier (stage t+1 is complete, nobody reads buffer t & 1 any more)
//   step 3: reads of stage t+1's step-0 fragments, then the later B tile
// so the LDS and the load path see an even stream and the LDS latency at
// stage boundaries is hidden as well.
//
// LDS: [A 0][A 1][B 0][B 1].  A: 256 rows of 128 bytes each, chunk c of row r
// at chunk c ^ ((r >> 1) & 7).  B: [64 contraction rows][256 columns],
// 512-byte rows, the 16-byte chunk c of row k stored at chunk c ^ nn_swz(k)
// (nn_swz(k) = 2 f(k), f(k) = (k & 3) | ((k >> 1) & 4)).  Both keep the tile
// writes and the fragment reads free of bank conflicts (measured with the LDS
// bank-conflict counter).
template <int PF>
__global__ void __launch_bounds__(w4::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_w4_nn_kernel(const GemmArgs p) {
  using namespace w4;
  static_assert(PF == 1 || PF == 2, "one or two staged tiles");
  __shared__ __attribute__((aligned(16))) char smem[LDS];
  // keep the MFMA accumulators in the accumulation registers
  asm volatile("" ::: "a0");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int lt = tid;

  const int bid = blockIdx.x;
  const int64_t m0 = (int64_t)(bid % p.tiles_m) * BM;
  const int64_t n0 = (int64_t)(bid / p.tiles_m) * BN;
  const int nk1 = (int)(p.K1 / BK);
  const int nk = nk1 + (int)((p.K2 + BK - 1) / BK);

  // ---- loaders ----
  // A: lane lt moves chunk lt & 7 of rows (lt >> 3) + 32 i, i < 8.  B: lane
  // lt moves chunk lt & 31 (8 columns) of contraction rows (lt >> 5) + 8 i,
  // i < 8: each load instruction covers two whole 512-byte rows.  Every load
  // is a raw buffer load (wave-uniform resource + one lane offset); an offset
  // at or beyond the resource's size reads zero, which masks the ragged
  // rank-r segment.
  const int kc = (lt & 7) * 8;
  const char* ga1 = reinterpret_cast<const char*>(p.a1) + m0 * p.lda1 * 2;
  const char* ga2 = reinterpret_cast<const char*>(p.a2) + m0 * p.lda2 * 2;
  const uint32_t va1 = (uint32_t)((lt >> 3) * p.lda1 * 2 + (lt & 7) * 16);
  const uint32_t va2 = (uint32_t)((lt >> 3) * p.lda2 * 2 + (lt & 7) * 16);
  const char* gb1 = reinterpret_cast<const char*>(p.b1) + n0 * 2;
  const char* gb2 = reinterpret_cast<const char*>(p.b2) + n0 * 2;
  const uint32_t vb1 = (uint32_t)((lt >> 5) * p.ldb1 * 2 + (lt & 31) * 16);
  const uint32_t vb2 = (uint32_t)((lt >> 5) * p.ldb2 * 2 + (lt & 31) * 16);
  // segment 2 of B: rows at or beyond K2 lie past the resource's end
  const int nrecb2 = (int)(p.K2 * p.ldb2 * 2 - n0 * 2);
  // per-segment strides, pinned in scalar registers (a select between two
  // kernel arguments is otherwise turned into a load from a selected
  // address inside the loop, whose wait drains every LDS operation)
  const uint32_t isa1 = __builtin_amdgcn_readfirstlane((uint32_t)(32 * p.lda1 * 2));
  const uint32_t isa2 = __builtin_amdgcn_readfirstlane((uint32_t)(32 * p.lda2 * 2));
  const uint32_t isb1 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * p.ldb1 * 2));
  const uint32_t isb2 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * p.ldb2 * 2));
  const int64_t kstb1 = (int64_t)BK * p.ldb1 * 2;
  const uint32_t kstb2 = __builtin_amdgcn_readfirstlane((uint32_t)(BK * p.ldb2 * 2));
  const int k2 = __builtin_amdgcn_readfirstlane((int)p.K2);

  u32x4 sa[PF][8], sb[PF][8];

  // Global loads of stage u (u < nk): a per-stage descriptor (uniform
  // resource, lane offset, stride between a lane's 8 chunks), then one
  // 16-byte load per chunk into staging buffer b.
  struct LoadDesc {
    __amdgpu_buffer_rsrc_t r;
    uint32_t vo, is;
  };
  auto desc_a = [&](int u) {
    const bool seg1 = u < nk1;
    const int tt = u - nk1;
    const char* base = seg1 ? ga1 + (int64_t)u * (BK * 2) : ga2;
    LoadDesc d;
    d.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, BIG, 0x00020000);
    d.vo = seg1 ? va1 : (tt * BK + kc < k2 ? va2 + (uint32_t)(tt * BK * 2) : OOB);
    d.is = seg1 ? isa1 : isa2;
    return d;
  };
  auto desc_b = [&](int u) {
    const bool seg1 = u < nk1;
    const int tt = u - nk1;
    LoadDesc d;
    const char* base = seg1 ? gb1 + (int64_t)u * kstb1 : gb2;
    d.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, seg1 ? BIG : nrecb2, 0x00020000);
    d.vo = seg1 ? vb1 : vb2 + (uint32_t)tt * kstb2;
    d.is = seg1 ? isb1 : isb2;
    return d;
  };
  auto ld = [&](const LoadDesc& d, int i) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(d.r, (int)(d.vo + i * d.is), 0, 0));
  };
  auto load_a = [&](int u, auto bsel) {
    constexpr int b = decltype(bsel)::value;
    const LoadDesc d = desc_a(u);
#pragma unroll
    for (int i = 0; i < 8; ++i) sa[b][i] = ld(d, i);
  };
  auto load_b = [&](int u, auto bsel) {
    constexpr int b = decltype(bsel)::value;
    const LoadDesc d = desc_b(u);
#pragma unroll
    for (int i = 0; i < 8; ++i) sb[b][i] = ld(d, i);
  };

  // ---- registers -> LDS buffer st ----
  // rows (lt >> 3) + 32 i all have (row >> 1) & 7 = (lt >> 4) & 7
  const uint32_t wr_off = (uint32_t)(lt >> 3) * 128 + (uint32_t)(((lt & 7) ^ ((lt >> 4) & 7)) << 4);
  // B row (lt >> 5) + 8 i has nn_swz = 2 ((lt >> 5) & 3) ^ 8 (i & 1)
  const uint32_t nn_w0 = (uint32_t)B_BASE + (uint32_t)(lt >> 5) * 512 +
                         (uint32_t)(((lt & 31) ^ (2 * ((lt >> 5) & 3))) << 4);
  const uint32_t nn_w1 = (uint32_t)B_BASE + (uint32_t)(lt >> 5) * 512 +
                         (uint32_t)(((lt & 31) ^ (2 * ((lt >> 5) & 3)) ^ 8) << 4);
  // one 16-byte LDS write of chunk i of the staged A / B tile into buffer st
  auto st_a = [&](int st, auto bsel, int i) {
    constexpr int b = decltype(bsel)::value;
    *reinterpret_cast<u32x4*>(smem + wr_off + st * A_STAGE + i * 32 * 128) = sa[b][i];
  };
  auto st_b = [&](int st, auto bsel, int i) {
    constexpr int b = decltype(bsel)::value;
    // chunk as loaded: contraction row (lt >> 5) + 8 i
    *reinterpret_cast<u32x4*>(smem + (i & 1 ? nn_w1 : nn_w0) + st * B_STAGE + i * 8 * 512) = sb[b][i];
  };
  auto store_a = [&](int st, auto bsel) {
#pragma unroll
    for (int i = 0; i < 8; ++i) st_a(st, bsel, i);
  };
  auto store_b = [&](int st, auto bsel) {
#pragma unroll
    for (int i = 0; i < 8; ++i) st_b(st, bsel, i);
  };

  // ---- fragments ----
  // A rows wm*TM + 32 i + l32 all have (row >> 1) & 7 = (l32 >> 1) & 7.
  const uint32_t ra = (uint32_t)(wm * TM + l32) * 128;
  const int swz = (l32 >> 1) & 7;
  bf16x8 fa[2][FM], fb[2][FN];
  // B fragments from ds_read_b64_tr_b16: within each 16-lane group, lane i
  // receives element (4 q + i / 4, i % 4) of the group's 4 x 4 loads (q < 4),
  // so pointing lane i at contraction row k0 + i / 4 and columns
  // n0 + 4 (i % 4) .. +3 hands it rows k0 .. k0 + 3 of column n0 + i.  Lane l
  // of the 32x32x16 fragment needs column 32 j + l % 32 and rows 8 (l / 32) ..
  // +7 of step s: group gq = l >> 4 takes columns n0 = 32 j + 16 (gq & 1) and
  // rows 16 s + 8 (gq >> 1) + 4 h, h < 2.  The row's swizzle is the same for
  // every s, j, h: f = ((l & 15) >> 2) | 4 (gq >> 1).
  uint32_t nn_r[FN];
  {
    const int gq = lane >> 4, i16 = lane & 15;
    const int f = (i16 >> 2) | ((gq >> 1) << 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int chunk = (wn * TN + 32 * j + 16 * (gq & 1) + 4 * (i16 & 3)) >> 3;
      nn_r[j] = (uint32_t)B_BASE + (uint32_t)(8 * (gq >> 1) + (i16 >> 2)) * 512 +
                (uint32_t)((chunk ^ (2 * f)) << 4) + (uint32_t)((i16 & 1) << 3);
    }
  }
  auto rd_nn = [&](int st, int s, int j) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    i16x4 h[2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
      h[hq] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(
          (__attribute__((address_space(3))) char*)smem + nn_r[j] + st * B_STAGE + (16 * s + 4 * hq) * 512));
    u32x4 v;
    v[0] = (uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16);
    v[1] = (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16);
    v[2] = (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16);
    v[3] = (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16);
    return __builtin_bit_cast(bf16x8, v);
  };
  auto rd = [&](int st, int s, auto fsel) {
    constexpr int f = decltype(fsel)::value;
    const uint32_t c = (uint32_t)(((2 * s + hh) ^ swz) << 4);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[f][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + ra + c + st * A_STAGE + i * 32 * 128));
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[f][j] = rd_nn(st, s, j);
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
    acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][q >> 2], fb[f][q & 3], acc[q >> 2][q & 3], 0, 0, 0);
  };
  // issue-order fence: nothing is scheduled across it
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // one fragment read (k < 4: A block k, else B block k - 4) of step s
  auto rd1 = [&](int st, int s, auto fsel, int k) {
    constexpr int f = decltype(fsel)::value;
    const uint32_t c = (uint32_t)(((2 * s + hh) ^ swz) << 4);
    if (k < FM)
      fa[f][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + ra + c + st * A_STAGE + k * 32 * 128));
    else
      fb[f][k - FM] = rd_nn(st, s, k - FM);
  };

  // one stage t (LDS buffer ST = t & 1); stage t+1 is staged in registers
  // sa/sb[(t+1) % PF]; loads issued here are for stage t+1+PF (clamped to the
  // last stage: a repeated load past the end is harmless)
  auto stage = [&](int t, auto stsel) {
    constexpr int ST = decltype(stsel)::value;
    constexpr int U = ST ^ 1;
    using SB = std::integral_constant<int, (ST + 1) % PF>;
    const int nxt = t + 1 + PF < nk ? t + 1 + PF : nk - 1;
    // Issue order, fixed by fences: every MFMA is followed by one memory
    // operation, so the LDS and the load path see an even stream:
    //   step 0: 8 x (MFMA, fragment read for step 1), 8 x (MFMA, A-tile write)
    //   step 1: 8 x (MFMA, read for step 2),          8 x (MFMA, B-tile write)
    //   step 2: 8 x (MFMA, read for step 3),          8 x (MFMA, A-tile load)
    //   barrier
    //   step 3: 8 x (MFMA, read of stage t+1 step 0), 8 x (MFMA, B-tile load)
    // (a step's first MFMA only waits for reads issued before the previous
    // step's writes: LDS operations complete in order)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I0{}, q);
      rd1(ST, 1, I1{}, q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I0{}, 8 + q);
      st_a(U, SB{}, q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I1{}, q);
      rd1(ST, 2, I0{}, q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I1{}, 8 + q);
      st_b(U, SB{}, q);
      fence();
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I0{}, q);
      rd1(ST, 3, I1{}, q);
      fence();
    }
    {
      const LoadDesc d = desc_a(nxt);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mf(I0{}, 8 + q);
        sa[SB::value][q] = ld(d, q);
        fence();
      }
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mf(I1{}, q);
      rd1(U, 0, I0{}, q);
      fence();
    }
    {
      const LoadDesc d = desc_b(nxt);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        mf(I1{}, 8 + q);
        sb[SB::value][q] = ld(d, q);
        fence();
      }
    }
  };

  // ---------------- main loop ----------------
  if (nk > 0) {
    load_a(0, I0{});
    load_b(0, I0{});
    store_a(0, I0{});
    store_b(0, I0{});
    if (PF == 1) {
      load_a(nk > 1 ? 1 : 0, I0{});
      load_b(nk > 1 ? 1 : 0, I0{});
    } else {
      load_a(nk > 1 ? 1 : 0, std::integral_constant<int, 1 % PF>{});
      load_b(nk > 1 ? 1 : 0, std::integral_constant<int, 1 % PF>{});
      load_a(nk > 2 ? 2 : nk - 1, I0{});
      load_b(nk > 2 ? 2 : nk - 1, I0{});
    }
    lds_barrier();
    rd(0, 0, I0{});
    int t = 0;
    for (; t + 1 < nk; t += 2) {
      stage(t, I0{});
      stage(t + 1, I1{});
    }
    if (t < nk) stage(t, I0{});
  }

  w4_epilogue<EPI_STORE>(p, acc, smem, m0, n0, p.c, p.ldc);
}

}  // namespace lora
