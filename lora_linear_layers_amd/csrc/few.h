// few.h - the fused LoRA layer for few tokens (M <= 128, bf16 activations):
// the forward in two launches (NF4 W, or bf16 W where the dispatch takes it),
// the backward in three or two.
//
//     forward   Y  = X W^T + bf16(s X A^T) B^T           (page "UnSloth加速微调
//     backward  dX = G W + bf16(s G B) A,                  体验…", sections 算子融合
//               dB = G^T bf16(s X A^T),                    and 反向传播优化)
//               dA = bf16(s G B)^T X,   G = R(-angle) dY with RoPE (section
//                                                           RoPE缓存集成), else dY
//
// With few tokens every operand except W is a few hundred KB: the layer is a
// stream of W (bf16, or NF4 codes and absmax, page "Unsloth教程…", section
// 显存优化策略, QLoRA paragraph) and launches cost as much as the stream.
//
//   launch 1 (few_panel_kernel): fp32 partial sums of the rank-r panels over
//     chunks of their contraction, P = X A^T (both directions) and, in the
//     backward, Q = G B; with RoPE it forms G from dY on load, rotating each
//     head's pairs (i, i + 64) by the negated angle, and stores G for launch
//     2.  It also clears the W stream's arrival counters.  The backward's W
//     stream sums the panels itself, P_s = bf16(s P) and Q_s = bf16(s Q),
//     while its first stages fly when the partials are few enough (fold);
//     else a launch between sums them once (few_reduce_kernel).
//   the W stream (few_fwd_nf4_kernel, few_fwd_bf16_kernel, few_bwd_kernel):
//     column tiles of 128 outputs, each a sequence of contraction stages; the
//     tiles' stages in sequence are cut into 256 equal contiguous ranges,
//     one block (one CU) each, so every CU streams the same share of W in
//     one round.  W stages land in a ring of LDS slots by DMA (buffer_load
//     ... lds), the stage's resource based at its tile so rows past the end
//     read zero.  A block
//     leaves one fp32 partial per tile it touches (at most two); the LAST
//     block of a tile to arrive (an atomic counter; partials written and
//     read with device-scope loads and stores) sums the tile's partials in
//     block order, so the result does not depend on arrival order, adds the
//     rank term (P_s B^T, or Q_s A) and applies RoPE or stores.  The
//     backward's blocks also produce dB rows (every G row of a stage meets all
//     M tokens inside one block, so dB needs no partials) and dA columns.
//
// MFMA v_mfma_f32_16x16x32_bf16.  A lane l holds row l % 16, contraction
// 8 (l / 16) .. +7; B lane l holds column l % 16, the same contraction; the 4
// results of lane l are rows 4 (l / 16) + v, column l % 16.
//
// LDS tiles.  "NT" tiles (rows of 64 contraction elements, 128 bytes): chunk
// c of row r at chunk c ^ (r & 7); a fragment read (16 rows, one chunk) is
// conflict-free.  "NN" tiles (contraction rows of 128 columns, 256 bytes),
// read with ds_read_b64_tr_b16 (in each 16-lane group, lane i points at row
// k0 + i / 4, columns n0 + 4 (i % 4) .. +3 and receives column n0 + i, rows
// k0 .. k0 + 3): the 32-byte segment s of row r sits at segment
// (s & ~3) | ((s ^ r) & 3), so the four rows of a group read four different
// 32-byte bank windows.
#pragma once

#include <type_traits>

#include "few_args.h"
#include "gemm.h"

namespace lora {

__device__ __forceinline__ __amdgpu_buffer_rsrc_t few_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
}

__device__ __forceinline__ u32x4 few_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// An ordering point for the compiler only (no instruction, no wait): memory
// operations written before it are issued before those written after it.  A W
// stream puts one between the loads it issues ahead of its DMAs and the DMAs:
// the compiler would otherwise sink such a load into the branch that uses it,
// past the DMAs, and a load issued after them completes only after all of them.
__device__ __forceinline__ void few_issue_order() { asm volatile("" ::: "memory"); }

// One DMA instruction (SIZE bytes per lane) into LDS at lds_base + SIZE lane.
// voff: the lane's byte offset (a loop-invariant register: a register that a
// DMA still in flight reads must not be rewritten, so one that changed per
// stage would make the compiler wait for every DMA before reusing it);
// soff: the stage's scalar offset.  Out-of-range lanes carry voff >= 2^31,
// past every resource (the scalar offset is never large enough to wrap).
template <int SIZE = 16>
__device__ __forceinline__ void few_dma(__amdgpu_buffer_rsrc_t r, char* lds_base, uint32_t voff, int soff) {
  static_assert(SIZE == 16 || SIZE == 4, "16 or 4 bytes per lane");
  auto* dst = (__attribute__((address_space(3))) void*)lds_base;
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, (int)voff, soff, 0, 0);
}

// NT tile: byte offset of 16-byte chunk c of row r (rows of 128 bytes)
__device__ __forceinline__ int nt_off(int r, int c) { return (r << 7) + ((c ^ (r & 7)) << 4); }
// NN tile with rows of RB bytes (128 or 256): byte offset of 16-byte chunk c
// of row r
template <int RB = 256>
__device__ __forceinline__ int nn_off(int r, int c) {
  const int sg = c >> 1;
  return r * RB + ((((sg & ~3) | ((sg ^ r) & 3)) << 1 | (c & 1)) << 4);
}

// B fragment of a 16x16x32 MFMA from an NN tile: columns n0 .. n0 + 15, the
// contraction rows k0 .. k0 + 31 (k0 a multiple of 32).  Lane group gq =
// l / 16 takes rows k0 + 8 gq .. +7 in two transposing reads of 4 rows.
template <int RB = 256>
__device__ __forceinline__ bf16x8 nn_frag(const char* tile, int k0, int n0, int lane) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const int gq = lane >> 4, i = lane & 15;
  i16x4 h[2];
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int row = k0 + 8 * gq + 4 * hq + (i >> 2);
    const int col = n0 + 4 * (i & 3);  // 4 columns = 8 bytes inside 16-byte chunk col / 8
    const int off = nn_off<RB>(row, col >> 3) + ((col & 7) << 1);
    h[hq] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)tile + off));
  }
  u32x4 v;
  v[0] = (uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16);
  v[1] = (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16);
  v[2] = (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16);
  v[3] = (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16);
  return __builtin_bit_cast(bf16x8, v);
}

// Fragment read transposed from an NT tile (rows = contraction, 64 columns):
// lane l gets column n0 + l % 16, contraction rows k0 + 8 (l / 16) .. +7 (the
// transposing read of nn_frag on the NT chunk layout)
__device__ __forceinline__ bf16x8 nt_tr_frag(const char* tile, int k0, int n0, int lane) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const int gq = lane >> 4, i = lane & 15;
  i16x4 h[2];
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int row = k0 + 8 * gq + 4 * hq + (i >> 2);
    const int col = n0 + 4 * (i & 3);
    const int off = nt_off(row, col >> 3) + ((col & 7) << 1);
    h[hq] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)tile + off));
  }
  u32x4 v;
  v[0] = (uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16);
  v[1] = (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16);
  v[2] = (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16);
  v[3] = (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16);
  return __builtin_bit_cast(bf16x8, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// The LDS addresses of the two transposing reads of nn_frag / nt_tr_frag
template <int RB = 256>
__device__ __forceinline__ u32x2 nn_frag_addr(const char* tile, int k0, int n0, int lane) {
  const int gq = lane >> 4, i = lane & 15;
  u32x2 a;
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int row = k0 + 8 * gq + 4 * hq + (i >> 2);
    const int col = n0 + 4 * (i & 3);
    a[hq] = lds_addr(tile + nn_off<RB>(row, col >> 3) + ((col & 7) << 1));
  }
  return a;
}
__device__ __forceinline__ u32x2 nt_tr_frag_addr(const char* tile, int k0, int n0, int lane) {
  const int gq = lane >> 4, i = lane & 15;
  u32x2 a;
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const int row = k0 + 8 * gq + 4 * hq + (i >> 2);
    const int col = n0 + 4 * (i & 3);
    a[hq] = lds_addr(tile + nt_off(row, col >> 3) + ((col & 7) << 1));
  }
  return a;
}


// A or B fragment from an NT tile: rows r0 .. r0 + 15, contraction 32 s .. +31
__device__ __forceinline__ bf16x8 nt_frag(const char* tile, int r0, int s, int lane) {
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(tile + nt_off(r0 + (lane & 15), 4 * s + (lane >> 4))));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint32_t h) { return __builtin_bit_cast(float, h << 16); }

// cos / sin of the row's position at frequencies f .. f + 3 (zeros for a
// position outside the cache: row 0 is read and the values dropped, so that
// no branch holds the loads back)
__device__ __forceinline__ void few_cs4(const FewArgs& p, int t, int f, f32x4& c, f32x4& s) {
  const int32_t q = p.pos[t];
  const bool ok = rope_pos_ok(q, p.max_pos);
  const int64_t o = (int64_t)(ok ? q : 0) * 64 + f;
  const f32x4 cv = *reinterpret_cast<const f32x4*>(p.cosc + o), sv = *reinterpret_cast<const f32x4*>(p.sinc + o);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  c = ok ? cv : z;
  s = ok ? sv : z;
}

// ---------------------------------------------------------------------------
// launch 1: panel partials.  Blocks [0, Sp pg): P, chunk b % Sp of d_in and
// (pg > 1, the forward, MB = 1) rows 16 (b / Sp) .. + 15; blocks
// [Sp pg, Sp pg + Sq): Q chunk of d_out.  A block's 4 waves take the chunk's
// 32-wide steps in turn (Q: a wave takes a whole head, so that with RoPE its
// pairs (i, i+64) meet in one lane), then the waves' sums meet in LDS.
// ---------------------------------------------------------------------------
template <int MB>
__global__ void __launch_bounds__(few::NT) few_panel_kernel(const FewArgs p) {
  using namespace few;
  constexpr int RB = MAXR / 16;
  constexpr int MP = MB * 16;
  // LDS: Q's per-wave B tiles (128 rows of B, an NN tile of 64 rank columns,
  // 16 KB each), then with RoPE the cos | sin rows of the tokens' positions
  // (128 floats a row, padded to CSW); afterwards, over both, the waves'
  // partial sums [4][MP][RW] fp32 (rows padded so that the 4 row groups of a
  // fragment's store fall in different banks)
  constexpr int BT = 128 * 128, CSW = 132, RW = MAXR + 4;
  constexpr int TOP = 4 * BT + MP * CSW * 4, RED = 4 * MP * RW * 4;
  __shared__ __attribute__((aligned(16))) char smem[RED > TOP ? RED : TOP];
  float(*red)[MP][RW] = reinterpret_cast<float(*)[MP][RW]>(smem);
  float* cst = reinterpret_cast<float*>(smem + 4 * BT);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int rb_n = (p.r8 + 15) >> 4;  // 16-column rank blocks that exist

  if (blockIdx.x == 0)
    for (int i = tid; i < p.n_tiles; i += NT) p.cnt[i] = 0;

  f32x4 acc[MB][RB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[mb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int np = p.Sp * p.pg;  // P blocks
  const bool isq = (int)blockIdx.x >= np;
  const int chunk = isq ? (int)blockIdx.x - np : (int)blockIdx.x % p.Sp;
  const int row0 = isq ? 0 : MP * ((int)blockIdx.x / p.Sp);  // the block's first token row
  if (!isq) {
    // P chunk: [X rows] x [A rows]^T over k in [k0, k1)
    const int k0 = chunk * p.Kp;
    const int k1 = min(p.d_in, k0 + p.Kp);
    const __amdgpu_buffer_rsrc_t rx = few_rsrc(p.X, (int64_t)p.M * p.d_in * 2);
    const __amdgpu_buffer_rsrc_t ra = few_rsrc(p.A, (int64_t)p.r8 * p.d_in * 2);
    // UP of the wave's 32-wide steps at a time (a chunk of up to 512 is 4 a
    // wave): all their loads in flight before the first product (steps past
    // k1 load zeros and are skipped)
    constexpr int UP = MB <= 4 ? 4 : 2;
    for (int kb = k0 + 32 * wave; kb < k1; kb += 128 * UP) {
      bf16x8 xf[UP][MB], af[UP][RB];
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        const int k = kb + 128 * u;
        const int kk = k + 8 * g;  // the lane's first element (k1 - k0 is a multiple of 32)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = row0 + 16 * mb + l16;
          xf[u][mb] = __builtin_bit_cast(
              bf16x8, few_ld16(rx, row < p.M && k < k1 ? (uint32_t)((row * p.d_in + kk) * 2) : OOB));
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int row = 16 * rb + l16;
          af[u][rb] = __builtin_bit_cast(
              bf16x8, few_ld16(ra, row < p.r8 && k < k1 ? (uint32_t)((row * p.d_in + kk) * 2) : OOB));
        }
      }
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        if (kb + 128 * u >= k1) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (rb < rb_n) acc[mb][rb] = mfma16(xf[u][mb], af[u][rb], acc[mb][rb]);
      }
    }
  } else {
    // Q chunk: [G rows] x B over i in [i0, i1), a head (128 rows of B) per
    // wave at a time; B's rows go to the wave's NN tile (rows of 64 rank
    // columns, zero past r8), read back with the transposing LDS read
    const int i0 = chunk * p.Kq;
    const int i1 = min(p.d_out, i0 + p.Kq);
    const __amdgpu_buffer_rsrc_t ry = few_rsrc(p.dY, (int64_t)p.M * p.d_out * 2);
    const __amdgpu_buffer_rsrc_t rbr = few_rsrc(p.B, (int64_t)p.d_out * p.r8 * 2);
    char* bt = smem + wave * BT;
    // a head's loads: dY fragments (4 steps of 32 rows of the head; with RoPE
    // the lane's elements of steps 0 / 1 pair with those of steps 2 / 3) and
    // B rows h .. h + 127 (fewer at the end: zeros), 8 rank columns per
    // 16-byte chunk: lane -> row h + lane + 64 j, chunks 0 .. 7
    bf16x8 gf[4][MB];
    u32x4 bv[2][8];
    auto load_g = [&](int h) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = 16 * mb + l16;
          const int ii = h + 32 * st + 8 * g;
          gf[st][mb] = __builtin_bit_cast(
              bf16x8, few_ld16(ry, row < p.M && ii < i1 ? (uint32_t)((row * p.d_out + ii) * 2) : OOB));
        }
    };
    auto load_b = [&](int h) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = lane + 64 * j;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          const bool ok = h + row < i1 && 8 * cc < p.r8;
          bv[j][cc] = few_ld16(rbr, ok ? (uint32_t)(((h + row) * p.r8 + 8 * cc) * 2) : OOB);
        }
      }
    };
    // With RoPE, the cos | sin rows of each token's position (zeros for a
    // position outside the cache) go to LDS in 16-byte pieces, item e ->
    // token e / 16, piece e % 16 of cos and of sin.  The positions are loaded
    // first and the first head's loads after them (128 tokens: B only, for
    // registers), so that the wait for the positions does not wait for those
    // (loads complete in issue order) and they fly while the rows land.  The
    // loads take no branch (rows past M read token 0's position, an invalid
    // position reads row 0 and is zeroed), so that all of them are in flight
    // at once.
    constexpr int IT = MP * 16 / NT;
    constexpr bool PRE_G = MB <= 4;
    int32_t pq[IT];
    if (p.rope) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int t = (tid + NT * i) >> 4;
        pq[i] = p.pos[t < p.M ? t : 0];
      }
    }
    // (a wave without a head loads zeros: its offsets lie past the resources)
    const int hw = i0 + 128 * wave;
    load_b(hw);
    if (PRE_G) load_g(hw);
    if (p.rope) {
      f32x4 cv[IT], sv[IT];
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int pc = (tid + NT * i) & 15;
        const int64_t off = (int64_t)(rope_pos_ok(pq[i], p.max_pos) ? pq[i] : 0) * 64 + 4 * pc;
        cv[i] = *reinterpret_cast<const f32x4*>(p.cosc + off);
        sv[i] = *reinterpret_cast<const f32x4*>(p.sinc + off);
      }
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        const int e = tid + NT * i, t = e >> 4, pc = e & 15;
        const bool ok = rope_pos_ok(pq[i], p.max_pos);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(cst + t * CSW + 4 * pc) = ok ? cv[i] : z;
        *reinterpret_cast<f32x4*>(cst + t * CSW + 64 + 4 * pc) = ok ? sv[i] : z;
      }
      __syncthreads();
    }
    for (int h = hw; h < i1; h += 512) {
      if (h != hw) load_b(h);
      if (h != hw || !PRE_G) load_g(h);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) *reinterpret_cast<u32x4*>(bt + nn_off<128>(lane + 64 * j, cc)) = bv[j][cc];
      // the wave reads back only what it wrote (its LDS operations complete in order)
      if (p.rope) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int row = 16 * mb + l16;
          if (row >= p.M) continue;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int f = 32 * st + 8 * g;  // frequency of the lane's first pair
            const float* cr = cst + row * CSW + f;
            const f32x4 c0 = *reinterpret_cast<const f32x4*>(cr), c1 = *reinterpret_cast<const f32x4*>(cr + 4);
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(cr + 64), s1 = *reinterpret_cast<const f32x4*>(cr + 68);
            const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
            const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
            const u32x4 y1 = __builtin_bit_cast(u32x4, gf[st][mb]);
            const u32x4 y2 = __builtin_bit_cast(u32x4, gf[st + 2][mb]);
            u32x4 g1, g2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a0 = bf2f(y1[e] & 0xffff), a1 = bf2f(y1[e] >> 16);
              const float b0 = bf2f(y2[e] & 0xffff), b1 = bf2f(y2[e] >> 16);
              const float c_0 = cs[2 * e], c_1 = cs[2 * e + 1], s_0 = sn[2 * e], s_1 = sn[2 * e + 1];
              g1[e] = pack_bf16x2(a0 * c_0 + b0 * s_0, a1 * c_1 + b1 * s_1);
              g2[e] = pack_bf16x2(b0 * c_0 - a0 * s_0, b1 * c_1 - a1 * s_1);
            }
            gf[st][mb] = __builtin_bit_cast(bf16x8, g1);
            gf[st + 2][mb] = __builtin_bit_cast(bf16x8, g2);
            const int ii = h + 32 * st + 8 * g;
            *reinterpret_cast<u32x4*>(p.G + (int64_t)row * p.d_out + ii) = g1;
            *reinterpret_cast<u32x4*>(p.G + (int64_t)row * p.d_out + ii + 64) = g2;
          }
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 bf[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) bf[rb] = nn_frag<128>(bt, 32 * st, 16 * rb, lane);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (rb < rb_n) acc[mb][rb] = mfma16(gf[st][mb], bf[rb], acc[mb][rb]);
      }
    }
  }
  // the waves' sums meet in LDS (over the B tiles and RoPE rows: every wave
  // is done with them)
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][16 * mb + 4 * g + v][16 * rb + l16] = acc[mb][rb][v];
  __syncthreads();
  // a thread stores 4 rank columns of a token row: 16 threads a row
  float* out = (isq ? p.Qp : p.Pp) + (int64_t)chunk * p.Mp * p.r8 + (int64_t)row0 * p.r8;
  const int q = 4 * (tid & 15);
  if (q < p.r8)
    for (int t = tid >> 4; t < MP; t += NT / 16) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(&red[0][t][q]), s1 = *reinterpret_cast<const f32x4*>(&red[1][t][q]);
      const f32x4 s2 = *reinterpret_cast<const f32x4*>(&red[2][t][q]), s3 = *reinterpret_cast<const f32x4*>(&red[3][t][q]);
      *reinterpret_cast<f32x4*>(out + t * p.r8 + q) = ((s0 + s1) + s2) + s3;
    }
}

// ---------------------------------------------------------------------------
// launch 2 pieces shared by both directions
// ---------------------------------------------------------------------------
// The NF4 byte -> bf16 pair table, 16 copies: entry b of copy k at float2 index
// 16 b + k.  Lane l reads copy l % 16, so the 16 lanes of a 128-byte LDS
// cycle hit 16 different bank pairs whatever their code bytes (one shared
// copy measured about 2x more bank-conflict cycles than LDS cycles).
constexpr int NF4_TAB_BYTES = 256 * 16 * 8;

// A thread writes entries tid + NTH i: byte b = tid / 16 + (NTH / 16) i, so
// its low nibble's value is the same in all of them and the high nibble is
// i (NTH = 256) or 2 i + tid / 256 (NTH = 512).
template <int NTH>
__device__ __forceinline__ void few_fill_tab(f32x2* tab, const float (&table)[16]) {
  static_assert(NTH == 256 || NTH == 512, "the table entries of a thread");
  auto u = [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x))); };
  const int tid = threadIdx.x;
  const float lo = tab16(table, (tid >> 4) & 15);
#pragma unroll
  for (int i = 0; i < 4096 / NTH; ++i) {
    const float hi = NTH == 256 ? u(table[i]) : ((tid >> 8) ? u(table[2 * i + 1]) : u(table[2 * i]));
    tab[tid + NTH * i] = f32x2{hi, lo};
  }
}

// two bf16 of code byte b: bf16(f32(table[c] * absmax)) for the high and low
// nibble (the same products as nf4_byte_to_bf16x2); tabl = tab + lane % 16
__device__ __forceinline__ uint32_t few_nf4_pair(const f32x2* tabl, uint32_t b, float am) {
  const f32x2 t = tabl[b << 4];
  return pack_bf16x2(t.x * am, t.y * am);
}

// Stage ring geometry: the W slot (bf16 rows, or NF4 codes and absmax) and the
// activation slot (MP rows of 64 elements, NT layout) of one stage, and how
// many stages fit next to the fixed LDS (NF4: two bf16 W tiles and the byte
// -> pair table).
template <int MB, bool NF4, int WROWS, int WBYTES_BF16, int EXTRA = 0>
struct FewRing {
  static constexpr int MP = MB <= 2 ? 32 : (MB <= 4 ? 64 : 128);  // activation rows in LDS (8 per DMA, 4 waves)
  static constexpr int XI = MP / 32;                               // activation DMAs per wave per stage
  static constexpr int CODES = WROWS * 32;                         // NF4 codes of a stage (64 elements per row)
  static constexpr int AM = 1024;                                   // absmax: 4 waves x 64 lanes x 4 bytes
  static constexpr int WSLOT = NF4 ? CODES + AM : WBYTES_BF16;
  static constexpr int XSLOT = MP * 128;
  static constexpr int STAGE = WSLOT + XSLOT;
  static constexpr int FIXED = (NF4 ? 2 * WBYTES_BF16 + NF4_TAB_BYTES : 0) + EXTRA;
  static constexpr int BUDGET = 160 * 1024 - 256 - FIXED;
  static constexpr int NS0 = BUDGET / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;
  // (+16: the finishing handshake's flag, in the same LDS array: a second
  // __shared__ variable gives the LDS accesses alias-scope metadata, after
  // which the compiler waits for every DMA in flight before each LDS read)
  static constexpr int LDS = FIXED + NS * STAGE + 16;
  static_assert(NS >= 3, "at least three stages");
};

// Partials exchanged between the blocks of one launch are written with
// device-scope (agent) relaxed atomic stores and read back with loads of the
// same cache policy (few_sum4_dev): on gfx950 these are plain stores and
// loads marked sc1, which go through the XCD's L2 to the device's coherence
// point.  A device-scope fence would instead write back and invalidate the
// whole L2 of the XCD (measured on MI355X: about 1.2 us per fence, serialised
// per XCD, which on a 4096 x 4096 weight stream cost 4x its time).
__device__ __forceinline__ void few_st_dev(float* q, float v) {
  __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The work split of launch 2: the tiles' stages in sequence (a tile's in
// contraction order, tiles in order), block b of nblk taking the contiguous
// range [b T / nblk, (b + 1) T / nblk).  With n_tiles <= nblk a range holds at most
// nkt stages, so it covers one tile or the end of one and the start of the
// next.  nk: the range's stages; a0: its first tile; s0: the first stage's
// index in that tile; te: the local index of tile a0's last stage in the range
// (nk - 1 when the range stays in a0).
struct FewSpan {
  int nk, a0, s0, te;
};
__device__ __forceinline__ FewSpan few_span(const FewArgs& p, int b) {
  const int g0 = (int)((int64_t)b * p.T / p.nblk), g1 = (int)((int64_t)(b + 1) * p.T / p.nblk);
  FewSpan s;
  s.nk = g1 - g0;
  s.a0 = g0 / p.nkt;
  s.s0 = g0 - s.a0 * p.nkt;
  s.te = min(s.nk, p.nkt - s.s0) - 1;
  return s;
}
// the block whose range holds stage x: the largest b with b T / nblk <= x
__device__ __forceinline__ int few_blk_of(const FewArgs& p, int x) {
  return (int)(((int64_t)(x + 1) * p.nblk - 1) / p.T);
}

// The finishing handshake, after every partial store of the block: each
// thread waits until its stores have been performed at the coherence point
// (vmcnt), the block meets, then one device-scope atomic per tile the block
// covers (n of them, the tiles' counters at cnt); flag[i] is set in the block
// that arrives last at tile i, whose device-scope loads (issued only after
// that atomic has returned) then see every other block's partial.  total(i):
// the blocks of tile i.
template <class F>
__device__ __forceinline__ void few_arrive(int* cnt, int n, F total, int* flag) {
  __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(0));
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = 0; i < n; ++i)
      flag[i] = __hip_atomic_fetch_add(cnt + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total(i) - 1;
  __syncthreads();
}

// f(integral_constant<int, j>) for j = 0 .. U-1, in order
template <int U, class F, int... js>
__device__ __forceinline__ void few_unroll_(F&& f, std::integer_sequence<int, js...>) {
  (f(std::integral_constant<int, js>{}), ...);
}
template <int U, class F>
__device__ __forceinline__ void few_unroll(F&& f) {
  few_unroll_<U>(f, std::make_integer_sequence<int, U>{});
}

// wait until at most n stages of this wave's DMAs (per stage PER instructions)
// are outstanding, n in 0 .. 7
template <int PER>
__device__ __forceinline__ void few_wait_stages(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 1 > 63 ? 63 : PER * 1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 2 > 63 ? 63 : PER * 2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 3 > 63 ? 63 : PER * 3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 4 > 63 ? 63 : PER * 4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 5 > 63 ? 63 : PER * 5)); break;
    default: __builtin_amdgcn_s_waitcnt(few::vmcnt_imm(PER * 6 > 63 ? 63 : PER * 6)); break;
  }
}

// Fixed-order sums of fp32 partial slabs, float4 at a time: out[i] =
// sum over z < S of src[z * zstride + off[i]] for the NI offsets a thread owns
// (off < 0: skipped, out zero), the loads of U slabs of every item in flight
// before any add.
template <int NI, int U = 8>
__device__ __forceinline__ void few_sum4(const float* src, int S, int64_t zstride, const int64_t (&off)[NI],
                                         float4 (&out)[NI]) {
#pragma unroll
  for (int i = 0; i < NI; ++i) out[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z0 = 0; z0 < S; z0 += U) {
    float4 v[NI][U];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[i][u] = (off[i] >= 0 && z0 + u < S)
                      ? *reinterpret_cast<const float4*>(src + (int64_t)(z0 + u) * zstride + off[i])
                      : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        out[i].x += v[i][u].x;
        out[i].y += v[i][u].y;
        out[i].z += v[i][u].z;
        out[i].w += v[i][u].w;
      }
  }
}

// The forward's rank panel P_s = bf16(s P), P the sum of launch 1's Sp slabs
// in slab order, into an NT tile of Mp rows and 64 columns (zeros past M and
// r8).  Item it: token it / 16, columns 4 (it % 16) .. + 3, IPT items a
// thread.  load() issues every slab load of the thread's items, to go ahead
// of the stream's DMAs (a load issued after them completes only after all of
// them); store() sums once they have landed.  The plan keeps Sp <= SMAX.
template <int MB, int NTH>
struct FewPanelPre {
  static constexpr int ITEMS = MB * 16 * 16;
  static constexpr int IPT = (ITEMS + NTH - 1) / NTH;
  static constexpr int SMAX = 16 / IPT;
  f32x4 v[IPT][SMAX];
  __device__ __forceinline__ void load(const FewArgs& p) {
    const __amdgpu_buffer_rsrc_t r = few_rsrc(p.Pp, (int64_t)p.Sp * p.Mp * p.r8 * 4);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = threadIdx.x + NTH * i, t = it >> 4, q = 4 * (it & 15);
      const bool ok = it < ITEMS && t < p.M && q < p.r8;
#pragma unroll
      for (int z = 0; z < SMAX; ++z)
        v[i][z] = __builtin_bit_cast(
            f32x4, few_ld16(r, ok && z < p.Sp ? (uint32_t)(((z * p.Mp + t) * p.r8 + q) * 4) : few::OOB));
    }
  }
  __device__ __forceinline__ void store(const FewArgs& p, char* tile) const {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = threadIdx.x + NTH * i, t = it >> 4, q = 4 * (it & 15);
      if (it >= ITEMS) continue;
      f32x4 a = v[i][0];
#pragma unroll
      for (int z = 1; z < SMAX; ++z)
        if (z < p.Sp) a += v[i][z];
      *reinterpret_cast<u32x2*>(tile + nt_off(t, q >> 3) + 2 * (q & 7)) =
          u32x2{pack_bf16x2(p.s * a[0], p.s * a[1]), pack_bf16x2(p.s * a[2], p.s * a[3])};
    }
  }
};

// few_sum4 over partials written by other blocks of the same launch:
// device-scope loads, 8 slabs of every item in flight.
template <int NI>
__device__ __forceinline__ void few_sum4_dev(const float* src, int S, int64_t zstride, const int64_t (&off)[NI],
                                             float4 (&out)[NI]) {
  // 16-byte buffer loads with the same cache policy as a device-scope
  // relaxed atomic load (sc1: served at the coherence point, not from a
  // possibly stale line of this XCD's L2); out-of-range items and slabs read
  // zero through an offset past the resource
  const __amdgpu_buffer_rsrc_t r = few_rsrc(src, (int64_t)S * zstride * 4);
#pragma unroll
  for (int i = 0; i < NI; ++i) out[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z0 = 0; z0 < S; z0 += 8) {
    f32x4 v[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t o =
            (off[i] >= 0 && z0 + u < S) ? (uint32_t)(((int64_t)(z0 + u) * zstride + off[i]) * 4) : few::OOB;
        v[i][u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 16);
      }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        out[i].x += v[i][u][0];
        out[i].y += v[i][u][1];
        out[i].z += v[i][u][2];
        out[i].w += v[i][u][3];
      }
  }
}

// The finishing block's output pass: y = the sum over the tile's partials (the
// rank term is in the partial of the tile's first block), then bf16 stores of
// four columns per item, or, with RoPE (BNT = 128, one head), the rotation of
// the pairs (f, f + 64) of each row.
// part: the tile's first partial slab ([Mp][BNT] each, S of them, summed in
// slab order).
template <int BNT, int NTH = few::NT>
__device__ __forceinline__ void few_finish(const FewArgs& p, const float* part, int S, int n0, int N, uint16_t* out,
                                           bool rope) {
  // NI items (16 bytes of 4 columns) of every slab in flight per thread (8
  // measured slower: the kernel's register allocation grows to all 256 and
  // its stream slows down)
  constexpr int NI = 4;
  const int64_t zs = (int64_t)p.Mp * BNT;
  if (!rope) {
    const int items = p.M * (BNT / 4);
    for (int i0 = threadIdx.x; i0 < items; i0 += NI * NTH) {
      int64_t off[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int it = i0 + i * NTH, t = it / (BNT / 4), c = 4 * (it % (BNT / 4));
        off[i] = (it < items && n0 + c < N) ? (int64_t)t * BNT + c : -1;
      }
      float4 a[NI];
      few_sum4_dev<NI>(part, S, zs, off, a);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (off[i] < 0) continue;
        const int it = i0 + i * NTH, t = it / (BNT / 4), c = 4 * (it % (BNT / 4));
        *reinterpret_cast<uint2*>(out + (int64_t)t * N + n0 + c) =
            make_uint2(pack_bf16x2(a[i].x, a[i].y), pack_bf16x2(a[i].z, a[i].w));
      }
    }
    return;
  }
  // RoPE: item = (row t, frequencies f .. f + 3); both halves summed.  The
  // positions and their cos / sin are loaded ahead of the partials.
  constexpr int IP = NI / 2;
  const int items = p.M * 16;
  for (int i0 = threadIdx.x; i0 < items; i0 += IP * NTH) {
    f32x4 cv[IP], sv[IP];
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int it = min(i0 + i * NTH, items - 1);
      few_cs4(p, it >> 4, 4 * (it & 15), cv[i], sv[i]);
    }
    int64_t off[NI];
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int it = i0 + i * NTH, t = it >> 4, f = 4 * (it & 15);
      off[2 * i] = it < items ? (int64_t)t * BNT + f : -1;
      off[2 * i + 1] = it < items ? (int64_t)t * BNT + f + 64 : -1;
    }
    float4 a[NI];
    few_sum4_dev<NI>(part, S, zs, off, a);
#pragma unroll
    for (int i = 0; i < IP; ++i) {
      const int it = i0 + i * NTH, t = it >> 4, f = 4 * (it & 15);
      if (it >= items) continue;
      const f32x4 cc = cv[i], ss = sv[i];
      const float z1[4] = {a[2 * i].x, a[2 * i].y, a[2 * i].z, a[2 * i].w};
      const float z2[4] = {a[2 * i + 1].x, a[2 * i + 1].y, a[2 * i + 1].z, a[2 * i + 1].w};
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y1[e] = z1[e] * cc[e] - z2[e] * ss[e];
        y2[e] = z2[e] * cc[e] + z1[e] * ss[e];
      }
      uint16_t* o = out + (int64_t)t * N + n0 + f;
      *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]));
      *reinterpret_cast<uint2*>(o + 64) = make_uint2(pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]));
    }
  }
}

// ---------------------------------------------------------------------------
// backward, between the launches: P_s = bf16(s X A^T) and Q_s = bf16(s G B)
// from the panel partials (block 0: P, block 1: Q), [Mp, r8] bf16 each
// ---------------------------------------------------------------------------
// Blocks [0, nb): P; [nb, 2 nb): Q; one float4 of the panel per thread, the
// loads of up to 32 slabs in flight at once.
__global__ void __launch_bounds__(few::NT) few_reduce_kernel(const FewArgs p) {
  const int nb = gridDim.x / 2;
  const bool q = (int)blockIdx.x >= nb;
  const float* part = q ? p.Qp : p.Pp;
  const int S = q ? p.Sq : p.Sp;
  uint16_t* out = q ? p.Qs : p.Ps;
  const int items = p.Mp * p.r8 / 4;
  const int it = (blockIdx.x - (q ? nb : 0)) * few::NT + threadIdx.x;
  int64_t off[1] = {it < items ? 4 * (int64_t)it : -1};
  float4 a[1];
  few_sum4<1, 32>(part, S, (int64_t)p.Mp * p.r8, off, a);
  if (off[0] >= 0)
    *reinterpret_cast<uint2*>(out + off[0]) =
        make_uint2(pack_bf16x2(p.s * a[0].x, p.s * a[0].y), pack_bf16x2(p.s * a[0].z, p.s * a[0].w));
}

// ---------------------------------------------------------------------------
// launch 2, forward with an NF4 W.  Stages of 128 contraction steps (64 code
// bytes and two absmax per W row); codes, absmax and the activations land in
// LDS by DMA, and each lane expands the code bytes of its own MFMA B fragments
// through the byte -> pair table: no expanded bf16 tile, one barrier a stage.
// The expansion is VALU work of the order of the stream time, so the block
// has 8 waves (two per SIMD, one overlapping the other's waits), 16 columns
// each.  A tile: 128 output columns; its stages: the 128-wide steps of d_in;
// block b streams its range of the stage sequence (few_span), so every CU the
// same share of W; one partial per (block, tile) and the last block to arrive
// at a tile sums them (few_finish).
// ---------------------------------------------------------------------------
template <int MB>
struct FewNf4Ring {
  static constexpr int MP = MB <= 2 ? 32 : (MB <= 4 ? 64 : 128);  // activation rows in LDS
  static constexpr int XI = MP / 32;       // activation DMAs per wave per stage (two 64-wide NT sub-tiles)
  static constexpr int CODES = 128 * 64;   // 8 blocks of 16 rows x 64 bytes
  static constexpr int AM = 8 * 256;       // 8 blocks of 16 rows x 2 absmax (and 128 unused bytes)
  static constexpr int XSLOT = 2 * MP * 128;
  static constexpr int STAGE = CODES + AM + XSLOT;
  static constexpr int FIXED = NF4_TAB_BYTES;
  static constexpr int NS0 = (160 * 1024 - 256 - 16 - FIXED) / STAGE;
  static constexpr int NS = NS0 > 8 ? 8 : NS0;
  static constexpr int LDS = FIXED + NS * STAGE + 16;  // (+16: the handshake flags)
  static_assert(NS >= 3, "at least three stages");
};

template <int MB>
__global__ void __launch_bounds__(few::NT4) __attribute__((amdgpu_waves_per_eu(2, 2)))
few_fwd_nf4_kernel(const FewArgs p) {
  using namespace few;
  using R = FewNf4Ring<MB>;
  constexpr int NS = R::NS, BNF = 128, BKS = 128;
  constexpr int PER = 2 + R::XI;  // DMAs per wave per stage: codes, absmax, activations
  static_assert(R::LDS >= R::MP * BNF * 4, "the finish reuses the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[R::LDS];
  f32x2* tab2 = reinterpret_cast<f32x2*>(smem);  // at LDS address 0
  char* ring = smem + R::FIXED;
  auto cslot = [&](int s) { return ring + s * R::STAGE; };
  auto aslot = [&](int s) { return ring + s * R::STAGE + R::CODES; };
  auto xslot = [&](int s) { return ring + s * R::STAGE + R::CODES + R::AM; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const FewSpan sp = few_span(p, blockIdx.x);
  const int nk = sp.nk;
  const bool two = sp.te < nk - 1;
  // the lane's copy of the pair table: byte b's entry at 128 b + 8 (lane % 16)
  const uint32_t rep = 8 * l16;

  const __amdgpu_buffer_rsrc_t rx = few_rsrc(p.X, (int64_t)p.M * p.d_in * 2);
  // codes and absmax of the block's two tiles, each resource based at the
  // tile's first row: rows past d_out lie past its end and read zero
  const int64_t cb = p.d_in / 2, ab = p.d_in / 64;
  const int64_t r0 = (int64_t)sp.a0 * BNF, r1 = (int64_t)min(sp.a0 + 1, p.n_tiles - 1) * BNF;
  const __amdgpu_buffer_rsrc_t rc0 = few_rsrc(p.codes + r0 * cb, (p.d_out - r0) * cb);
  const __amdgpu_buffer_rsrc_t rc1 = few_rsrc(p.codes + r1 * cb, (p.d_out - r1) * cb);
  const __amdgpu_buffer_rsrc_t ra0 = few_rsrc(p.absmax + r0 * ab, (p.d_out - r0) * ab * 4);
  const __amdgpu_buffer_rsrc_t ra1 = few_rsrc(p.absmax + r1 * ab, (p.d_out - r1) * ab * 4);
  // Lane offsets at the tile's stage 0 (stage st adds a scalar offset).
  // Codes: wave w's block holds rows 16 w .. + 15; lane L fetches the quarter
  // L / 16 (32 elements) of row 16 w + L % 16 and lands at byte 256 (L / 16) +
  // 16 (L % 16) of the block, so that a fragment read (16 rows, one dword each
  // of one quarter) touches 64 different banks.
  const uint32_t vc = (uint32_t)((16 * wave + l16) * cb + 16 * g);
  // absmax: lane L < 32 of wave w takes row 16 w + L % 16, block L / 16
  const uint32_t vam = lane < 32 ? (uint32_t)(((16 * wave + l16) * ab + (lane >> 4)) * 4) : OOB;
  // activations: instruction k = wave + 8 i moves rows 8 (k % (MP / 8)) .. + 7
  // of sub-tile k / (MP / 8) (NT rows of 64 elements)
  const int drow = lane >> 3, dpc = lane & 7;
  uint32_t vx[R::XI];
#pragma unroll
  for (int i = 0; i < R::XI; ++i) {
    const int k = wave + NW4 * i, sub = k / (R::MP / 8);
    const int row = 8 * (k % (R::MP / 8)) + drow;
    vx[i] = row < p.M ? (uint32_t)((row * p.d_in + 64 * sub + 8 * (dpc ^ (row & 7))) * 2) : OOB;
  }
  auto issue = [&](int t, int slot) {
    const bool second = t > sp.te;
    const int st = second ? t - sp.te - 1 : sp.s0 + t;
    few_dma(second ? rc1 : rc0, cslot(slot) + wave * 1024, vc, st * (BKS / 2));
    few_dma<4>(second ? ra1 : ra0, aslot(slot) + wave * 256, vam, st * 8);
#pragma unroll
    for (int i = 0; i < R::XI; ++i) {
      const int k = wave + NW4 * i;
      few_dma(rx, xslot(slot) + (k / (R::MP / 8)) * (R::MP * 128) + (k % (R::MP / 8)) * 1024, vx[i], st * (BKS * 2));
    }
  };

  // acc0: tile a0's sum once the range has moved on; accr: tile a0 + 1's
  // starting value (its rank term)
  f32x4 acc[MB], acc0[MB], accr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = acc0[mb] = accr[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The wave's columns 16 wave + l16 are the W rows of code block wave;
  // fragment ss covers contraction 32 ss + 8 g .. + 7 of the stage: dword g of
  // quarter ss, scaled by the row's absmax ss / 2.  Byte q of a code dword
  // selects the pair-table entry at ((w >> (8 q - 7)) & 0x7f80) | rep.
  auto compute = [&](int slot) {
    const char* cs = cslot(slot) + wave * 1024 + 16 * l16 + 4 * g;
    const char* as = aslot(slot) + wave * 256 + 4 * l16;
    const char* xs = xslot(slot);
    uint32_t cw[4];
    float am[2];
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) cw[ss] = *reinterpret_cast<const uint32_t*>(cs + 256 * ss);
#pragma unroll
    for (int h = 0; h < 2; ++h) am[h] = *reinterpret_cast<const float*>(as + 64 * h);
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t off = ((q == 0 ? cw[ss] << 7 : cw[ss] >> (8 * q - 7)) & 0x7f80u) | rep;
        const f32x2 tv = *reinterpret_cast<const f32x2*>(smem + off);
        o[q] = pack_bf16x2(tv.x * am[ss >> 1], tv.y * am[ss >> 1]);
      }
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, o);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = mfma16(nt_frag(xs + (ss >> 1) * (R::MP * 128), 16 * mb, ss & 1, lane), bfr, acc[mb]);
    }
  };
  auto tile_done = [&](int t) {
    if (t == sp.te && two) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc0[mb] = acc[mb];
        acc[mb] = accr[mb];
      }
    }
  };

  // The rank term P_s B^T of a tile goes into the partial of the block that
  // streams the tile's first stage (tile a0 when s0 = 0, tile a0 + 1 when the
  // range reaches it).  Its B fragments (rows = the wave's 16 columns, r8
  // contiguous) and the panel partials are loaded ahead of the DMAs, with no
  // branch (offsets past a resource read zero: a load in a branch makes the
  // compiler wait for every load in flight, DMAs included, before its first
  // use); P_s goes to LDS no stage uses yet (the last ring slot) while the
  // first stages fly.
  const bool rk0 = sp.s0 == 0;
  const __amdgpu_buffer_rsrc_t rbr = few_rsrc(p.B, (int64_t)p.d_out * p.r8 * 2);
  FewPanelPre<MB, NT4> pre;
  pre.load(p);
  bf16x8 bq[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep) {
      const int q = 32 * sstep + 8 * g, col = (sp.a0 + u) * BNF + 16 * wave + l16;
      const bool ok = (u ? two : rk0) && col < p.d_out && q < p.r8;
      bq[u][sstep] = __builtin_bit_cast(bf16x8, few_ld16(rbr, ok ? (uint32_t)((col * p.r8 + q) * 2) : OOB));
    }

  // stages 0 .. NS - 2 in flight, with no branch (a range of fewer stages
  // loads its last stage again into slots it does not use; the loop's waits
  // count them, and its last wait, for none in flight, sees them land)
  few_issue_order();
  few_unroll<NS - 1>([&](auto sc) { issue(min((int)decltype(sc)::value, nk - 1), decltype(sc)::value); });
  if (rk0 || two) {
    char* ps = cslot(NS - 1);
    pre.store(p, ps);
    lds_barrier();  // (LDS only: a __syncthreads would also wait for every DMA in flight)
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = nt_frag(ps, 16 * mb, sstep, lane);
        if (rk0) acc[mb] = mfma16(af, bq[0][sstep], acc[mb]);
        if (two) accr[mb] = mfma16(af, bq[1][sstep], accr[mb]);
      }
    // (the slot's first DMA, at stage 0, follows the loop's first barrier)
  }
  // the pair table, read after the loop's first barrier (filled once the
  // loads and DMAs are out)
  few_fill_tab<NT4>(tab2, p.nf4_table);
  constexpr int U = (NS % 2) ? 2 * NS : NS;
  for (int t0 = 0; t0 < nk; t0 += U) {
    few_unroll<U>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int t = t0 + j;
      if (t >= nk) return;
      few_wait_stages<PER>(min(NS - 2, nk - 1 - t));
      lds_barrier();
      if (t + NS - 1 < nk) issue(t + NS - 1, (j + NS - 1) % NS);
      compute(j % NS);
      tile_done(t);
    });
  }

  // ---- one partial per covered tile, then the last block of a tile finishes ----
  const int b = blockIdx.x, na = two ? 2 : 1;
  auto store_part = [&](const f32x4 (&v)[MB], int a) {
    float* cp = p.Cp + (int64_t)(b + a) * p.Mp * BNF;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int row = 16 * mb + 4 * g + vv;
        if (row < p.M) few_st_dev(cp + row * BNF + 16 * wave + l16, v[mb][vv]);
      }
  };
  if (two) store_part(acc0, sp.a0);
  store_part(acc, sp.a0 + na - 1);
  int* flag = reinterpret_cast<int*>(smem + R::LDS - 16);
  few_arrive(p.cnt + sp.a0, na,
             [&](int i) {
               const int a = sp.a0 + i;
               return few_blk_of(p, (a + 1) * p.nkt - 1) - few_blk_of(p, a * p.nkt) + 1;
             },
             flag);
  const int fin0 = flag[0], fin1 = na > 1 ? flag[1] : 0;
  for (int i = 0; i < na; ++i) {
    if (!(i ? fin1 : fin0)) continue;
    // (the rank term is in the partial of the tile's first block)
    const int a = sp.a0 + i;
    const int lo = few_blk_of(p, a * p.nkt), hi = few_blk_of(p, (a + 1) * p.nkt - 1);
    few_finish<BNF, NT4>(p, p.Cp + (int64_t)(lo + a) * p.Mp * BNF, hi - lo + 1, a * BNF, p.d_out, p.Y,
                         p.rope != 0);
  }
}

// ---------------------------------------------------------------------------
// launch 2, forward with a bf16 W: the same tiles, ranges, partials, rank term
// and finish as the NF4 form, with 64-deep stages of W (128 rows of 128 bytes,
// NT layout) and of the activations landing by DMA; 4 waves of 32 columns.
// ---------------------------------------------------------------------------
template <int MB>
__global__ void __launch_bounds__(few::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
few_fwd_bf16_kernel(const FewArgs p) {
  using namespace few;
  constexpr int BNF = 128, NJ = 2;
  using R = FewRing<MB, false, BNF, BNF * 128>;
  constexpr int NS = R::NS;
  constexpr int WI = BNF / 32;  // W DMAs per wave per stage (8 rows each)
  constexpr int PER = WI + R::XI;
  static_assert(R::STAGE >= R::MP * 128, "P_s fits a ring slot");
  __shared__ __attribute__((aligned(1024))) char smem[R::LDS];
  char* ring = smem + R::FIXED;
  auto wslot = [&](int slot) { return ring + slot * R::STAGE; };
  auto xslot = [&](int slot) { return ring + slot * R::STAGE + R::WSLOT; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const FewSpan sp = few_span(p, blockIdx.x);
  const int nk = sp.nk;
  const bool two = sp.te < nk - 1;

  const __amdgpu_buffer_rsrc_t rx = few_rsrc(p.X, (int64_t)p.M * p.d_in * 2);
  // W of the block's two tiles, each resource based at the tile's first row:
  // rows past d_out lie past its end and read zero
  const int64_t r0 = (int64_t)sp.a0 * BNF, r1 = (int64_t)min(sp.a0 + 1, p.n_tiles - 1) * BNF;
  const __amdgpu_buffer_rsrc_t rw0 = few_rsrc(p.W + r0 * p.d_in, (p.d_out - r0) * p.d_in * 2);
  const __amdgpu_buffer_rsrc_t rw1 = few_rsrc(p.W + r1 * p.d_in, (p.d_out - r1) * p.d_in * 2);
  // DMA lane mapping of an NT tile: 8 rows x 128 bytes per instruction, the
  // lane lands at physical chunk lane & 7 of row lane / 8 and so fetches
  // logical chunk (lane & 7) ^ (row & 7).  Offsets at the tile's stage 0
  // (stage st adds a scalar offset).
  const int drow = lane >> 3, dpc = lane & 7;
  uint32_t vw[WI], vx[R::XI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int row = 8 * (WI * wave + i) + drow;
    vw[i] = (uint32_t)((row * p.d_in + 8 * (dpc ^ (row & 7))) * 2);
  }
#pragma unroll
  for (int i = 0; i < R::XI; ++i) {
    const int row = 8 * (wave + 4 * i) + drow;
    vx[i] = row < p.M ? (uint32_t)((row * p.d_in + 8 * (dpc ^ (row & 7))) * 2) : OOB;
  }
  auto issue = [&](int t, int slot) {
    const bool second = t > sp.te;
    const int st = second ? t - sp.te - 1 : sp.s0 + t;
    const __amdgpu_buffer_rsrc_t rw = second ? rw1 : rw0;
#pragma unroll
    for (int i = 0; i < WI; ++i) few_dma(rw, wslot(slot) + (WI * wave + i) * 1024, vw[i], st * (BK * 2));
#pragma unroll
    for (int i = 0; i < R::XI; ++i) few_dma(rx, xslot(slot) + (wave + 4 * i) * 1024, vx[i], st * (BK * 2));
  };

  // acc0: tile a0's sum once the range has moved on; accr: tile a0 + 1's
  // starting value (its rank term)
  f32x4 acc[MB][NJ], acc0[MB][NJ], accr[MB][NJ];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mb][j] = acc0[mb][j] = accr[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot) {
    const char* xs = xslot(slot);
    const char* wt = wslot(slot);
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep) {
      bf16x8 bfr[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = nt_frag(wt, 32 * wave + 16 * j, sstep, lane);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = nt_frag(xs, 16 * mb, sstep, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[mb][j] = mfma16(af, bfr[j], acc[mb][j]);
      }
    }
  };
  auto tile_done = [&](int t) {
    if (t == sp.te && two) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc0[mb][j] = acc[mb][j];
          acc[mb][j] = accr[mb][j];
        }
    }
  };

  // The rank term P_s B^T of a tile goes into the partial of the block that
  // streams the tile's first stage (tile a0 when s0 = 0, tile a0 + 1 when the
  // range reaches it).  Its B fragments (rows = the wave's columns, r8
  // contiguous) and the panel partials are loaded ahead of the DMAs, with no
  // branch; P_s goes to LDS no stage uses yet (the last ring slot) while the
  // first stages fly.
  const bool rk0 = sp.s0 == 0;
  const __amdgpu_buffer_rsrc_t rbr = few_rsrc(p.B, (int64_t)p.d_out * p.r8 * 2);
  FewPanelPre<MB, NT> pre;
  pre.load(p);
  bf16x8 bq[2][2][NJ];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int q = 32 * sstep + 8 * g, col = (sp.a0 + u) * BNF + 32 * wave + 16 * j + l16;
        const bool ok = (u ? two : rk0) && col < p.d_out && q < p.r8;
        bq[u][sstep][j] = __builtin_bit_cast(bf16x8, few_ld16(rbr, ok ? (uint32_t)((col * p.r8 + q) * 2) : OOB));
      }

  // stages 0 .. NS - 2 in flight, with no branch (as in the NF4 form)
  few_issue_order();
  few_unroll<NS - 1>([&](auto sc) { issue(min((int)decltype(sc)::value, nk - 1), decltype(sc)::value); });
  if (rk0 || two) {
    char* ps = wslot(NS - 1);
    pre.store(p, ps);
    lds_barrier();  // (LDS only: a __syncthreads would also wait for every DMA in flight)
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = nt_frag(ps, 16 * mb, sstep, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (rk0) acc[mb][j] = mfma16(af, bq[0][sstep][j], acc[mb][j]);
          if (two) accr[mb][j] = mfma16(af, bq[1][sstep][j], accr[mb][j]);
        }
      }
    // (the slot's first DMA, at stage 0, follows the loop's first barrier)
  }
  // The stage loop, unrolled so that every ring slot index is a constant.
  constexpr int U = (NS % 2) ? 2 * NS : NS;
  for (int t0 = 0; t0 < nk; t0 += U) {
    few_unroll<U>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int t = t0 + j;
      if (t >= nk) return;
      few_wait_stages<PER>(min(NS - 2, nk - 1 - t));
      lds_barrier();
      if (t + NS - 1 < nk) issue(t + NS - 1, (j + NS - 1) % NS);
      compute(j % NS);
      tile_done(t);
    });
  }

  // ---- one partial per covered tile, then the last block of a tile sums ----
  const int b = blockIdx.x, na = two ? 2 : 1;
  auto store_part = [&](const f32x4 (&v)[MB][NJ], int a) {
    float* cp = p.Cp + (int64_t)(b + a) * p.Mp * BNF;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int row = 16 * mb + 4 * g + vv;
          if (row < p.M) few_st_dev(cp + row * BNF + 32 * wave + 16 * j + l16, v[mb][j][vv]);
        }
  };
  if (two) store_part(acc0, sp.a0);
  store_part(acc, sp.a0 + na - 1);
  int* flag = reinterpret_cast<int*>(smem + R::LDS - 16);
  few_arrive(p.cnt + sp.a0, na,
             [&](int i) {
               const int a = sp.a0 + i;
               return few_blk_of(p, (a + 1) * p.nkt - 1) - few_blk_of(p, a * p.nkt) + 1;
             },
             flag);
  const int fin0 = flag[0], fin1 = na > 1 ? flag[1] : 0;
  for (int i = 0; i < na; ++i) {
    if (!(i ? fin1 : fin0)) continue;
    const int a = sp.a0 + i;
    const int lo = few_blk_of(p, a * p.nkt), hi = few_blk_of(p, (a + 1) * p.nkt - 1);
    few_finish<BNF>(p, p.Cp + (int64_t)(lo + a) * p.Mp * BNF, hi - lo + 1, a * BNF, p.d_out, p.Y,
                    p.rope != 0);
  }
}

// ---------------------------------------------------------------------------
// launch 2, backward: dX = G W + Q_s A, dB and dA.  A tile: 128 columns of d_in
// (4 waves x 32); its stages: the 64-wide steps of d_out.  Block b streams its
// range of the stage sequence (few_span); the last block to arrive at a tile
// finishes it.  dB rows of stage st come from the tile st mod n_tiles, dA
// rows of a tile from its blocks in turn.
// ---------------------------------------------------------------------------
template <int MB, bool NF4>
__global__ void __launch_bounds__(few::NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
few_bwd_kernel(const FewArgs p) {
  using namespace few;
  constexpr int NJ = 2;  // a wave's 32 columns
  // (a stage's NF4 codes: 64 rows x 64 bytes, the size of 128 rows of 32)
  using R0 = FewRing<MB, NF4, 128, 64 * 256>;
  constexpr int PT = R0::MP * 128;  // one panel tile (NT, MP rows)
  using R = FewRing<MB, NF4, 128, 64 * 256, 2 * PT>;
  constexpr int NS = R::NS;
  constexpr int WI = NF4 ? 1 : 4;  // bf16: 16 instructions of 4 rows x 256 bytes; NF4: 4 of 16 rows x 64 bytes
  constexpr int PER = WI + R::XI + (NF4 ? 1 : 0);
  static_assert(NS * R::STAGE >= 64 * 256 && (NF4 ? 2 * 64 * 256 + NF4_TAB_BYTES : NS * R::STAGE - 64 * 256) >=
                    R::MP * 128 * 4,
                "the finish reuses the ring (A tile) and the W tiles or the ring (rank tile)");
  __shared__ __attribute__((aligned(1024))) char smem[R::LDS];
  char* ring = smem + R::FIXED;
  auto wslot = [&](int slot) { return ring + slot * R::STAGE; };
  auto gslot = [&](int slot) { return ring + slot * R::STAGE + R::WSLOT; };
  char* pst = smem;       // P_s (NT)
  char* qst = smem + PT;  // Q_s (NT)
  auto wbf = [&](int b) { return smem + 2 * PT + b * (64 * 256); };  // NF4: expanded W tiles (NN)
  f32x2* tab2 = reinterpret_cast<f32x2*>(smem + 2 * PT + 2 * 64 * 256);
  const f32x2* tabl = tab2 + (threadIdx.x & 15);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const FewSpan sp = few_span(p, blockIdx.x);
  const int nk = sp.nk;
  const bool two = sp.te < nk - 1;  // the range reaches tile a0 + 1
  // NF4: the byte -> pair table entries this thread writes (entry tid + NT i:
  // {table[i], table[(tid / 16) % 16]}; the table is in the kernel's
  // arguments), written to LDS once the DMAs are out
  static_assert(!NF4 || NT == 256, "the table entries of a thread");
  const float tlo = NF4 ? tab16(p.nf4_table, (tid >> 4) & 15) : 0.f;
  // Every load of the prologue takes no branch (offsets past a resource read
  // zero) and those used after the stream's first DMAs are issued before
  // them: a load issued after the DMAs completes only after all of them, and
  // a load in a branch makes the compiler wait for every load in flight,
  // DMAs included, before its first use.
  // The P_s and Q_s tiles start as zeros (rows past Mp, columns past r8)
  for (int e = tid; e < 2 * R::MP * 8; e += NT) *reinterpret_cast<u32x4*>(smem + 16 * e) = u32x4{0u, 0u, 0u, 0u};
  // Their values: with fold, the panel partials of one 4-column item of P and
  // one of Q per thread (Mp r8 / 4 <= NT items each; at most 8 slabs each),
  // else the bf16 panels, 8 columns per item, up to 4 items of each.
  const int nP4 = p.Mp * p.r8 / 4, n8 = p.Mp * p.r8 / 8;
  f32x4 pv[2][8];
  u32x4 bv[2][4];
  if (p.fold) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int S = k ? p.Sq : p.Sp;
      const __amdgpu_buffer_rsrc_t rp = few_rsrc(k ? p.Qp : p.Pp, (int64_t)S * p.Mp * p.r8 * 4);
#pragma unroll
      for (int z = 0; z < 8; ++z)
        pv[k][z] = __builtin_bit_cast(
            f32x4, few_ld16(rp, tid < nP4 && z < S ? (uint32_t)(((int64_t)z * p.Mp * p.r8 + 4 * tid) * 4) : OOB));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const __amdgpu_buffer_rsrc_t rs = few_rsrc(k ? p.Qs : p.Ps, (int64_t)n8 * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int it = tid + NT * e;
        bv[k][e] = few_ld16(rs, it < n8 ? (uint32_t)(16 * it) : OOB);
      }
    }
  }
  __syncthreads();  // the zeros are written
  const uint16_t* Gm = p.rope ? p.G : p.dY;
  const __amdgpu_buffer_rsrc_t rg = few_rsrc(Gm, (int64_t)p.M * p.d_out * 2);
  // W (NF4: codes and absmax) of the block's two tiles, each resource based at
  // the tile's first column (d_in is a multiple of 128: whole tiles)
  const int64_t c0 = (int64_t)sp.a0 * 128, c1 = (int64_t)min(sp.a0 + 1, p.n_tiles - 1) * 128;
  const int64_t nel = (int64_t)p.d_out * p.d_in;
  __amdgpu_buffer_rsrc_t rw0, rw1, ram0, ram1;
  if constexpr (NF4) {
    rw0 = few_rsrc(p.codes + c0 / 2, (nel - c0) / 2);
    rw1 = few_rsrc(p.codes + c1 / 2, (nel - c1) / 2);
    ram0 = few_rsrc(p.absmax + c0 / 64, (nel - c0) / 64 * 4);
    ram1 = few_rsrc(p.absmax + c1 / 64, (nel - c1) / 64 * 4);
  } else {
    rw0 = few_rsrc(p.W + c0, (nel - c0) * 2);
    rw1 = few_rsrc(p.W + c1, (nel - c1) * 2);
  }
  const int drow = lane >> 3, dpc = lane & 7;
  // the lanes' DMA offsets at the tile's stage 0 (stage st adds a scalar
  // offset: 64 more W rows, 64 more G columns)
  uint32_t vw[WI], vam = OOB, vg[R::XI];
  if constexpr (NF4) {
    // codes: instruction j = wave moves rows 16 j .. 16 j + 15, 64 bytes
    // (128 columns) each; the lane: row 16 j + lane / 4, quarter lane & 3
    const int row = 16 * wave + (lane >> 2);
    vw[0] = (uint32_t)(row * (p.d_in / 2) + 16 * (lane & 3));
    // absmax: entries e = 32 wave + lane (lanes < 32): row e / 2, block e & 1
    const int e = 32 * wave + lane;
    if (lane < 32) vam = (uint32_t)(((e >> 1) * (p.d_in / 64) + (e & 1)) * 4);
  } else {
    // NN tile rows of 256 bytes: instruction j moves rows 4 j .. 4 j + 3; the
    // lane lands at physical chunk lane & 15 of row 4 j + lane / 16
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int row = 4 * (WI * wave + i) + (lane >> 4);
      const int pc = lane & 15, psg = pc >> 1;
      const int lsg = (psg & ~3) | ((psg ^ row) & 3);
      vw[i] = (uint32_t)((row * p.d_in + 8 * ((lsg << 1) | (pc & 1))) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < R::XI; ++i) {
    const int row = 8 * (wave + 4 * i) + drow;
    vg[i] = row < p.M ? (uint32_t)((row * p.d_out + 8 * (dpc ^ (row & 7))) * 2) : OOB;
  }
  // local stage t: tile a0 (stage s0 + t) up to te, then tile a0 + 1
  auto stage_of = [&](int t) { return t > sp.te ? t - sp.te - 1 : sp.s0 + t; };
  auto issue = [&](int t, int slot) {
    const bool second = t > sp.te;
    const int st = stage_of(t);
    char* ws = wslot(slot);
    if constexpr (NF4) {
      const __amdgpu_buffer_rsrc_t rc = second ? rw1 : rw0, ra = second ? ram1 : ram0;
      few_dma(rc, ws + wave * 1024, vw[0], st * BK * (p.d_in / 2));
      few_dma<4>(ra, ws + R::CODES + wave * 256, vam, st * BK * (p.d_in / 64) * 4);
    } else {
      const __amdgpu_buffer_rsrc_t rw = second ? rw1 : rw0;
#pragma unroll
      for (int i = 0; i < WI; ++i) few_dma(rw, ws + (WI * wave + i) * 1024, vw[i], st * BK * p.d_in * 2);
    }
    char* gs = gslot(slot);
#pragma unroll
    for (int i = 0; i < R::XI; ++i) few_dma(rg, gs + (wave + 4 * i) * 1024, vg[i], st * (BK * 2));
  };
  // NF4: codes of stage st -> bf16 NN tile b: thread t expands row t / 4,
  // columns 32 (t & 3) .. +31 (one absmax block half)
  auto expand = [&](int slot, int b) {
    if constexpr (NF4) {
      const char* ws = wslot(slot);
      const int row = tid >> 2, qt = tid & 3;
      const u32x4 c = *reinterpret_cast<const u32x4*>(ws + (row >> 4) * 1024 + (row & 15) * 64 + 16 * qt);
      const int e = 2 * row + (qt >> 1);
      const float am = *reinterpret_cast<const float*>(ws + R::CODES + (e >> 5) * 256 + (e & 31) * 4);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = few_nf4_pair(tabl, (c[w] >> (8 * q)) & 0xff, am);
        *reinterpret_cast<u32x4*>(wbf(b) + nn_off<256>(row, 4 * qt + w)) = o;
      }
    }
  };

  // acc0: tile a0's sum once the range has moved on; accr: tile a0 + 1's
  // starting value (its rank term)
  f32x4 acc[MB][NJ], acc0[MB][NJ], accr[MB][NJ];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mb][j] = acc0[mb][j] = accr[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const char* gs, const char* wt) {
    // the stage's W fragments of both 32-deep steps in one batch of reads
    bf16x8 bfr[2 * NJ];
    u32x2 ad[2 * NJ];
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int j = 0; j < NJ; ++j) ad[NJ * sstep + j] = nn_frag_addr<256>(wt, 32 * sstep, 32 * wave + 16 * j, lane);
    lds_tr_frags<2 * NJ>(bfr, ad);
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = nt_frag(gs, 16 * mb, sstep, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[mb][j] = mfma16(af, bfr[NJ * sstep + j], acc[mb][j]);
      }
    }
  };
  // dB rows of stage st (G rows i of the stage meet all M tokens here): the
  // block that streams stage st of tile st mod n_tiles writes
  // dB[i, q] = sum_t G[t, i] P_s[t, q] = (G^T P_s)[i, q], an MFMA product over
  // the tokens (zero rows past M): A = G^T read transposed from the G tile,
  // B = P_s read transposed from its NT tile.  Wave w: rows 16 w .. + 15.
  // P_s fragments for dB, read once (the tile does not change)
  constexpr int KT = R::MP / 32;
  bf16x8 pfr[KT][MAXR / 16];
  auto load_pfr = [&]() {
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      u32x2 ad[MAXR / 16];
#pragma unroll
      for (int nb = 0; nb < MAXR / 16; ++nb) ad[nb] = nt_tr_frag_addr(pst, 32 * k, 16 * nb, lane);
      lds_tr_frags<MAXR / 16>(pfr[k], ad);
    }
  };
  auto db_rows = [&](int t, int slot) {
    const int st = stage_of(t);
    if (st % p.n_tiles != sp.a0 + (t > sp.te ? 1 : 0)) return;
    const char* gs = gslot(slot);
    f32x4 d[MAXR / 16];
#pragma unroll
    for (int nb = 0; nb < MAXR / 16; ++nb) d[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 af[KT];
    u32x2 ad[KT];
#pragma unroll
    for (int k = 0; k < KT; ++k) ad[k] = nt_tr_frag_addr(gs, 32 * k, 16 * wave, lane);
    lds_tr_frags<KT>(af, ad);
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int nb = 0; nb < MAXR / 16; ++nb)
        if (16 * nb < p.r8) d[nb] = mfma16(af[k], pfr[k][nb], d[nb]);
    const int i0 = st * BK + 16 * wave;
#pragma unroll
    for (int nb = 0; nb < MAXR / 16; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = 16 * nb + l16;
        if (q < p.r8) p.dB[(int64_t)(i0 + 4 * g + v) * p.r8 + q] = d[nb][v];
      }
  };

  auto tile_done = [&](int t) {
    if (t == sp.te && two) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc0[mb][j] = acc[mb][j];
          acc[mb][j] = accr[mb][j];
        }
    }
  };

  // The rank term Q_s A of a tile goes into the partial of the block that
  // streams the tile's first stage (tile a0 when s0 = 0, tile a0 + 1 when the
  // range reaches it), computed before the stream: its A rows (q < r8, the
  // tile's 128 columns) are loaded here, ahead of the DMAs, and used once Q_s
  // is in LDS.
  const bool rk0 = sp.s0 == 0;
  const __amdgpu_buffer_rsrc_t rar = few_rsrc(p.A, (int64_t)p.r8 * p.d_in * 2);
  u32x4 av[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + NT * e, q = idx >> 4, cc = idx & 15;
      const int col = (sp.a0 + u) * 128 + 8 * cc;
      const bool ok = (u ? two : rk0) && q < p.r8 && col < p.d_in;
      av[u][e] = few_ld16(rar, ok ? (uint32_t)((q * p.d_in + col) * 2) : OOB);
    }

  // prologue: stages 0 .. NS - 2 in flight, with no branch (a range of fewer
  // stages loads its last stage again into the slots it does not use; the
  // waits below count them, and the last wait, for none in flight, sees them
  // land before the ring is reused)
  few_issue_order();
  few_unroll<NS - 1>([&](auto sc) { issue(min((int)decltype(sc)::value, nk - 1), decltype(sc)::value); });
  if constexpr (NF4) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tab2[tid + NT * i] = f32x2{p.nf4_table[i], tlo};
  }
  // P_s and Q_s into their NT tiles while the first stages fly: with fold
  // summed here (slabs in order) from launch 1's partials, else the bf16
  // panels of few_reduce_kernel
  if (p.fold) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int S = k ? p.Sq : p.Sp;
      f32x4 a = pv[k][0];
#pragma unroll
      for (int z = 1; z < 8; ++z)
        if (z < S) a += pv[k][z];
      const int off = 4 * tid, t = off / p.r8, c = off % p.r8;
      if (tid < nP4)
        *reinterpret_cast<u32x2*>((k ? qst : pst) + nt_off(t, c >> 3) + 2 * (c & 7)) =
            u32x2{pack_bf16x2(p.s * a[0], p.s * a[1]), pack_bf16x2(p.s * a[2], p.s * a[3])};
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int it = tid + NT * e, x = 8 * it;
        if (it < n8) *reinterpret_cast<u32x4*>((k ? qst : pst) + nt_off(x / p.r8, (x % p.r8) >> 3)) = bv[k][e];
      }
  }
  lds_barrier();  // the P_s and Q_s tiles are written
  load_pfr();
  // rank terms: acc (tile a0) and accr (tile a0 + 1) start from Q_s A.  The A
  // tile goes to LDS that no stage uses yet (the last ring slot, or the second
  // expanded W tile), as an NN tile read like W.
  char* at = NF4 ? wbf(1) : wslot(NS - 1);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!(u ? two : rk0)) continue;
    // (LDS-only barriers: a __syncthreads would also wait for every DMA in flight)
    if (u && rk0) lds_barrier();  // every wave is done with tile a0's A
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + NT * e;
      *reinterpret_cast<u32x4*>(at + nn_off<256>(idx >> 4, idx & 15)) = av[u][e];
    }
    lds_barrier();
    bf16x8 bfr[2 * NJ];
    u32x2 ad[2 * NJ];
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int j = 0; j < NJ; ++j) ad[NJ * sstep + j] = nn_frag_addr<256>(at, 32 * sstep, 32 * wave + 16 * j, lane);
    lds_tr_frags<2 * NJ>(bfr, ad);
#pragma unroll
    for (int sstep = 0; sstep < 2; ++sstep)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 af = nt_frag(qst, 16 * mb, sstep, lane);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (u)
            accr[mb][j] = mfma16(af, bfr[NJ * sstep + j], accr[mb][j]);
          else
            acc[mb][j] = mfma16(af, bfr[NJ * sstep + j], acc[mb][j]);
        }
      }
  }
  // (the slot's first DMA, at stage 0, follows the loop's first barrier)
  if constexpr (NF4) {
    if (nk > 0) {
      few_wait_stages<PER>(min(NS - 2, nk - 1));
      lds_barrier();
      expand(0, 0);
    }
  }
  // unrolled as in the forward: constant slot and W tile indices
  constexpr int U = (NS % 2) ? 2 * NS : NS;
  for (int t0 = 0; t0 < nk; t0 += U) {
    few_unroll<U>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int t = t0 + j;
      if (t >= nk) return;
      if constexpr (NF4) {
        if (t + 1 < nk) few_wait_stages<PER>(min(NS - 3, nk - 2 - t));
        lds_barrier();
        if (t + NS - 1 < nk) issue(t + NS - 1, (j + NS - 1) % NS);
        if (t + 1 < nk) expand((j + 1) % NS, (j + 1) & 1);
        compute(gslot(j % NS), wbf(j & 1));
      } else {
        few_wait_stages<PER>(min(NS - 2, nk - 1 - t));
        lds_barrier();
        if (t + NS - 1 < nk) issue(t + NS - 1, (j + NS - 1) % NS);
        compute(gslot(j % NS), wslot(j % NS));
      }
      db_rows(t, j % NS);
      tile_done(t);
    });
  }

  const int N = p.d_in;
  const int b = blockIdx.x, na = two ? 2 : 1;
  auto blo = [&](int a) { return few_blk_of(p, a * p.nkt); };
  auto bhi = [&](int a) { return few_blk_of(p, (a + 1) * p.nkt - 1); };

  // dA[q, j] = sum_t Q_s[t, q] X[t, j] for a covered tile's 128 columns j and
  // the 16-rank blocks nb = i, i + c, ... (the block is the tile's i-th of c):
  // (X^T Q_s)[j, q] by MFMA over the tokens, X [MP rows, 128 columns] staged
  // in the ring (NN layout, zeros past M), A = X^T and B = Q_s both read
  // transposed.  Wave w: columns 32 w .. + 31.
  for (int ia = 0; ia < na; ++ia) {
    const int a = sp.a0 + ia, n0 = a * 128;
    const int lo = blo(a), c = bhi(a) - lo + 1;
    if (16 * (b - lo) >= p.r8) continue;
    char* xt = ring;
    __syncthreads();  // every wave is done with the ring
    for (int e = tid; e < R::MP * 16; e += NT) {
      const int t = e >> 4, cc = e & 15;
      const int col = n0 + 8 * cc;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t < p.M && col < p.d_in) v = *reinterpret_cast<const u32x4*>(p.X + (int64_t)t * p.d_in + col);
      *reinterpret_cast<u32x4*>(xt + nn_off<256>(t, cc)) = v;
    }
    __syncthreads();
    for (int nb = b - lo; 16 * nb < p.r8; nb += c) {
      f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < R::MP / 32; ++k) {
        const bf16x8 bq = nt_tr_frag(qst, 32 * k, 16 * nb, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) d[j] = mfma16(nn_frag<256>(xt, 32 * k, 32 * wave + 16 * j, lane), bq, d[j]);
      }
      const int q = 16 * nb + l16;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int col = n0 + 32 * wave + 16 * j + 4 * g + v;
          if (q < p.r8 && col < p.d_in) p.dA[(int64_t)q * p.d_in + col] = d[j][v];
        }
    }
  }

  // ---- one partial per covered tile (slab b + a of tile a), then the last
  // block to arrive at a tile finishes it ----
  auto store_part = [&](const f32x4 (&v)[MB][NJ], int a) {
    float* cp = p.Cp + (int64_t)(b + a) * p.Mp * 128;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int row = 16 * mb + 4 * g + vv;
          if (row < p.M) few_st_dev(cp + row * 128 + 32 * wave + 16 * j + l16, v[mb][j][vv]);
        }
  };
  if (two) store_part(acc0, sp.a0);
  store_part(acc, sp.a0 + na - 1);
  int* flag = reinterpret_cast<int*>(smem + R::LDS - 16);
  few_arrive(p.cnt + sp.a0, na, [&](int i) { return bhi(sp.a0 + i) - blo(sp.a0 + i) + 1; }, flag);
  const int fin0 = flag[0], fin1 = na > 1 ? flag[1] : 0;

  for (int ia = 0; ia < na; ++ia) {
    if (!(ia ? fin1 : fin0)) continue;
    const int a = sp.a0 + ia, n0 = a * 128;
    // (the rank term is in the partial of the tile's first block)
    __syncthreads();
    const int lo = blo(a);
    few_finish<128>(p, p.Cp + (int64_t)(lo + a) * p.Mp * 128, bhi(a) - lo + 1, n0, N, p.dX, false);
  }
}

}  // namespace lora
