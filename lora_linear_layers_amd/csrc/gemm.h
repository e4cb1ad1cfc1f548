// gemm.h - the one MFMA GEMM template behind every contraction of the fused
// LoRA linear layer on gfx950 (CDNA4).
//
// It computes C[m, n] = sum_k Aop[m, k] * Bop[k, n] over a contraction made of
// up to two segments that feed the SAME fp32 accumulator:
//
//   segment 1: (a1, b1) over K1 elements   e.g. X and W
//   segment 2: (a2, b2) over K2 elements   e.g. the rank-r panel s*X*A^T and B
//
// which is how the low-rank update lands in the base GEMM's accumulator: the
// forward is [X | sXA^T] [W | B]^T and the input gradient is
// [dY | s dY B] [W ; A] (page "UnSloth加速微调体验…", section 算子融合: the whole
// Wx + BAx in one pass, no [M, d_out] intermediate in memory).
//
// Operand layouts (row-major):
//   Aop: always contraction-contiguous, a[m * lda + k].
//   Bop, B_NN = false: b[n * ldb + k]  (the "weight" layout, W [d_out, d_in]).
//   Bop, B_NN = true : b[k * ldb + n]  (contraction along rows: W in dX, dY in dB).
//   Bop, BL_NF4      : segment 1 is W given as NF4 codes + absmax; segment 2 plain.
//
// Tiles: BM x BN per workgroup, 128 bytes of contraction per stage (64 bf16 or
// 32 fp32), two LDS stages.  Waves form a WM x WN grid and each owns a
// (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks.
//
// Schedules.  With 8 waves (two per SIMD) the workgroup runs a ping-pong:
// waves 0-3 (one per SIMD) and waves 4-7 alternate between a compute phase
// (fragment reads + MFMAs on stage t) and a memory phase (write the stage t+1
// operand they loaded into LDS, then issue the global loads of stage t+2).
// Group 0 moves the A operand, group 1 the B operand.  Phases are separated
// by raw s_barriers (no memory fence, so loads stay in flight across them), and
// every SIMD always has one wave issuing MFMAs.  Configurations with 4 waves
// use one double-buffered loop in which every thread loads both operands.
// bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses v_mfma_f32_16x16x4_f32 (true
// fp32 products, no reduced-precision inputs).
//
// LDS rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r is stored at
// chunk c ^ (r & 7).  Measured on gfx950 (LDS bank-conflict counters): with
// this swizzle a 64-lane ds_read_b128 of 16 consecutive rows at one chunk
// takes 4 cycles with no conflicts (256 B/clk), and the loaders' row-major
// ds_write_b128 are conflict-free as well.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Epi : int {
  EPI_STORE = 0,       // C[m, n] = alpha * acc            (type T)
  EPI_STORE_T = 1,     // Ct[n, m] = alpha * acc           (type T)
  EPI_STORE_BOTH = 2,  // both of the above
  EPI_ROPE = 3,        // rotate (n, n+64) pairs of 128-wide heads, then store
  EPI_PARTIAL = 4,     // fp32 partial slab of split z: C[z][m, n] = acc
  EPI_ADD = 5,         // C[m, n] = alpha * acc + Cin[m, n]  (type T; C may be Cin)
  EPI_SWIGLU = 6,      // whole-tile kernel only: gate/up pair -> silu(g) * u (see gemm_w4.h)
  EPI_ADD_MASKED = 7,  // C[m, n] = keep(m, n) ? alpha * acc + Cin[m, n] : Cin[m, n]
  EPI_GROUP = 8        // whole-tile kernel only: several projections' GEMMs, store or RoPE per member
};

enum BLoad : int { BL_PLAIN = 0, BL_NF4 = 1 };

// A RoPE position outside [0, max_pos) names no row of the cos / sin cache:
// such a row reads no cache memory and its cos and sin are taken as zero (its
// outputs come out as zeros).
__device__ __forceinline__ bool rope_pos_ok(int32_t q, int64_t max_pos) { return q >= 0 && q < max_pos; }

constexpr int kPanelSrcMax = 8;  // row sources of a panel's Bop (a group's members)
constexpr int kGroupGemmMax = 8;  // members of one group GEMM launch

struct GemmArgs {
  const void* a1;
  const void* b1;
  int64_t lda1, ldb1, K1;
  const void* a2;
  const void* b2;
  int64_t lda2, ldb2, K2;
  int64_t m_load, m_store;  // rows of Aop that exist / rows of C written
  int64_t n_load, n_store;  // columns of Bop that exist / columns of C written
  int64_t k_split;          // EPI_PARTIAL: contraction length per blockIdx.z
  void* c;
  int64_t ldc;
  void* ct;
  int64_t ldct;
  int64_t part_stride;      // EPI_PARTIAL: elements between split slabs
  float alpha;
  int tiles_m;
  const int32_t* pos;       // EPI_ROPE
  const float* cosc;
  const float* sinc;
  int64_t max_pos;          // rows of the cos / sin cache
  const uint8_t* codes;     // BL_NF4: packed codes of W [n_load rows? see loader], bytes per row
  const float* absmax;
  int64_t codes_ld;         // bytes per W row (= d_in / 2)
  int64_t blocks_per_row;   // absmax entries per W row (= d_in / 64)
  float nf4_table[16];
  const void* cin;          // EPI_ADD: the addend, row stride ldcin
  int64_t ldcin;
  // EPI_SWIGLU: b1 / b2 are the gate's W and padded B, b1u / b2u the up's
  // (b2u row stride ldb2u); rank columns [0, k2_split) of segment 2 belong to
  // the gate, [k2_split, K2) to the up; c = silu(g) * u, and g / u are also
  // stored to cg / cu (row stride ldc) when not NULL
  const void* b1u;
  const void* b2u;
  int64_t ldb2u, k2_split;
  void* cg;
  void* cu;
  // EPI_ADD_MASKED: keep bit of (m, n) = bit n % 8 of mask[m * mask_ld + n / 8]
  const uint8_t* mask;
  int64_t mask_ld;
  // panel_dma_kernel with n_src > 0: Bop rows [rs_beg[g], rs_beg[g] + 8k) of
  // the tile (up to the next source's rs_beg, or n_store) come from rs[g],
  // its row 0 first and its rows at or past rs_rows[g] read as zeros (row
  // stride ldb1; rs_beg[0] = 0, every rs_beg a multiple of 8).  n_src = 0:
  // every row from b1.
  int n_src;
  const void* rs[kPanelSrcMax];
  int rs_beg[kPanelSrcMax];
  int rs_rows[kPanelSrcMax];
  // gemm_w4_nt_kernel<EPI_GROUP>: the forward GEMMs of n_mem projections of
  // one X in one launch.  Blocks [mem_tile0[g], mem_tile0[g + 1]) are member
  // g's whole tiles (tiles_m per 256 of its columns, in the single GEMM's
  // order); per member its W (row stride ldb1), B (row stride mem_ldb2), its
  // columns of the stacked panel (mem_a2, row stride lda2), rank mem_k2, Y
  // (mem_c, row stride mem_ldc = its column count) and the RoPE epilogue
  // (mem_rope) or the store.
  int n_mem;
  int mem_tile0[kGroupGemmMax + 1];
  const void* mem_b1[kGroupGemmMax];
  const void* mem_b2[kGroupGemmMax];
  const void* mem_a2[kGroupGemmMax];
  void* mem_c[kGroupGemmMax];
  int mem_k2[kGroupGemmMax];
  int mem_ldb2[kGroupGemmMax];
  int mem_ldc[kGroupGemmMax];
  int mem_rope[kGroupGemmMax];
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row << 7) + ((chunk ^ (row & 7)) << 4);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 32-bit LDS address of a generic pointer into LDS
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// N fragments of ds_read_b64_tr_b16 pairs (the two halves of each at a[n][0]
// and a[n][1]) in one asm block that issues the 2N reads back to back and
// waits for them before it ends (no read is in flight when the block's output
// registers are handed back).  The builtin form of the read makes the compiler
// wait first for every LDS DMA in flight, which would drain a stage ring at
// each read; callers read only slots whose DMAs their own waits and barriers
// have already seen land.
#define LDS_TR(o, a) "ds_read_b64_tr_b16 %" #o ", %" #a "\n\t"
template <int N>
__device__ __forceinline__ void lds_tr_frags(bf16x8 (&f)[N], const u32x2 (&a)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 fragments");
  u32x2 h[2 * N];
  if constexpr (N == 1) {
    asm volatile(LDS_TR(0, 2) LDS_TR(1, 3) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(h[0]), "=&v"(h[1])
                 : "v"(a[0][0]), "v"(a[0][1]));
  } else if constexpr (N == 2) {
    asm volatile(LDS_TR(0, 4) LDS_TR(1, 5) LDS_TR(2, 6) LDS_TR(3, 7) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
                 : "v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1]));
  } else {
    asm volatile(LDS_TR(0, 8) LDS_TR(1, 9) LDS_TR(2, 10) LDS_TR(3, 11) LDS_TR(4, 12) LDS_TR(5, 13)
                     LDS_TR(6, 14) LDS_TR(7, 15) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]), "=&v"(h[5]),
                   "=&v"(h[6]), "=&v"(h[7])
                 : "v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1]), "v"(a[2][0]), "v"(a[2][1]),
                   "v"(a[3][0]), "v"(a[3][1]));
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const u32x4 v = {h[2 * n][0], h[2 * n][1], h[2 * n + 1][0], h[2 * n + 1][1]};
    f[n] = __builtin_bit_cast(bf16x8, v);
  }
}
#undef LDS_TR

__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// two floats -> two bf16 (nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32 (the scalar casts of f2bf, or-ed, take three instructions)
typedef float pk_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pk_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(pk_f32x2{lo, hi}, pk_bf16x2));
}

template <typename T>
__device__ __forceinline__ void store_out(void* c, int64_t idx, float v) {
  if constexpr (sizeof(T) == 2)
    reinterpret_cast<uint16_t*>(c)[idx] = f2bf(v);
  else
    reinterpret_cast<float*>(c)[idx] = v;
}

// NF4 byte -> two bf16 (element 2j in the high nibble goes to the low half,
// i.e. first in memory).  tab2[b] = {table[b >> 4], table[b & 15]} lives in LDS.
// Each value is the fp32 product table * absmax (round to nearest even), then
// rounded to bf16 (nearest even).
__device__ __forceinline__ uint32_t nf4_byte_to_bf16x2(const float2* tab2, uint32_t b, float am) {
  float2 t = tab2[b & 0xFF];
  return pack_bf16x2(t.x * am, t.y * am);
}

// t[i] of a 16-entry table held in the kernel's arguments, for a lane's own
// i, by selects over the 16 values: indexing the argument's array with a
// lane value (or taking its address) would copy the whole argument block to
// scratch memory and read every argument from there.  Each value passes
// through readfirstlane (free on a uniform value), which keeps the compiler
// from turning the selects of loaded values into a select of addresses and
// one per-lane load from the argument segment, a memory round trip each call.
__device__ __forceinline__ float tab16(const float (&t)[16], int i) {
  auto u = [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x))); };
  float v = u(t[0]);
#pragma unroll
  for (int k = 1; k < 16; ++k) v = i == k ? u(t[k]) : v;
  return v;
}

__device__ __forceinline__ void nf4_fill_tab2(float2* tab2, const float (&table)[16], int tid, int nt) {
  for (int t = tid; t < 256; t += nt) tab2[t] = make_float2(tab16(table, t >> 4), tab16(table, t & 15));
}

template <typename T, int BM, int BN, int WM, int WN, bool B_NN, int EPI, int BL>
struct GemmCfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr bool PP = (WM * WN == 8);   // ping-pong schedule
  static constexpr int NTL = PP ? NT / 2 : NT;  // threads per loading role
  static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(T);
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr int LDS = 2 * STAGE + (BL == BL_NF4 ? 2048 : 0);
  // per loading thread
  static constexpr int CA = BM * 8 / NTL;                       // A chunks
  static constexpr int CB = BN * 8 / NTL;                       // B chunks (weight layout)
  static constexpr int NBLK = 8 * (BN / E);                     // B blocks (contraction-row layout), E x E
  static constexpr int CBN = (NBLK + NTL - 1) / NTL;
  static constexpr int NF4U = BN * 2;                           // NF4 half-row units (weight layout)
  static constexpr int CNF = (NF4U + NTL - 1) / NTL;
  static constexpr int NF4B = BN;                               // NF4 8x8 blocks (contraction-row layout)
  static constexpr int CNFB = (NF4B + NTL - 1) / NTL;
  static constexpr int PB_PLAIN = B_NN ? CBN * E : CB;          // B prefetch, 16-byte registers
  static constexpr int PB_NF4 = B_NN ? CNFB * 2 : CNF;
  static constexpr int PB = (BL == BL_NF4 && PB_NF4 > PB_PLAIN) ? PB_NF4 : PB_PLAIN;
  static constexpr int PAM = BL == BL_NF4 ? (B_NN ? CNFB * 8 : CNF) : 1;
  static constexpr int OFFB = PP ? 0 : CA;                      // B registers follow A's unless roles split
  static constexpr int PRE = PP ? (CA > PB ? CA : PB) : CA + PB;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile/wave mismatch");
  static_assert((BM * 8) % NTL == 0 && (BN * 8) % NTL == 0, "16-byte chunks must divide over the threads");
  static_assert(EPI != EPI_ROPE || TN == 128, "RoPE epilogue needs 128-wide wave columns");
  static_assert(BL == BL_PLAIN || sizeof(T) == 2, "NF4 weights feed bf16 MFMA");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Workgroup barrier for LDS hand-offs: this wave's LDS traffic is complete,
// then s_barrier.  Unlike __syncthreads() it carries no memory fence, so global
// loads already in flight stay in flight.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int BM, int BN, int WM, int WN, bool B_NN, int EPI, int BL>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const GemmArgs p) {
  using C = GemmCfg<T, BM, BN, WM, WN, B_NN, EPI, BL>;
  constexpr int NT = C::NT, NTL = C::NTL, E = C::E, BK = C::BK, FM = C::FM, FN = C::FN;
  constexpr bool BF16 = sizeof(T) == 2;
  constexpr bool PP = C::PP;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  float2* tab2 = reinterpret_cast<float2*>(smem + 2 * C::STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;
  // loading roles: with the ping-pong, waves 0..3 move A and waves 4..7 move B
  const bool role_a = PP ? tid < NTL : true;
  const bool role_b = PP ? tid >= NTL : true;
  const int lt = PP ? (tid & (NTL - 1)) : tid;

  const int bid = blockIdx.x;
  const int64_t m0 = (int64_t)(bid % p.tiles_m) * BM;
  const int64_t n0 = (int64_t)(bid / p.tiles_m) * BN;
  const int z = blockIdx.z;

  // contraction ranges
  int64_t kbeg = 0, kend = p.K1;
  if constexpr (EPI == EPI_PARTIAL) {
    kbeg = (int64_t)z * p.k_split;
    kend = kbeg + p.k_split < p.K1 ? kbeg + p.k_split : p.K1;
  }
  const int nk1 = kend > kbeg ? (int)((kend - kbeg + BK - 1) / BK) : 0;
  // with split partials only the last split runs segment 2
  const int nk2 = (EPI == EPI_PARTIAL && z + 1 < (int)gridDim.z) ? 0 : (int)((p.K2 + BK - 1) / BK);
  const int nk = nk1 + nk2;

  // ---------------- prefetch registers (shared by the two roles) ----------
  u32x4 pre[C::PRE];
  float pam[C::PAM];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Segment-1 loads of tiles that lie wholly inside the operands take a
  // wave-uniform base plus a fixed 32-bit per-lane byte offset (no masks, no
  // per-load 64-bit address arithmetic); tails and segment 2 use masked loads.
  const bool a_full = m0 + BM <= p.m_load;
  const bool b_full = n0 + BN <= p.n_load;
  const char* a1t = reinterpret_cast<const char*>(p.a1) + m0 * p.lda1 * (int64_t)sizeof(T);
  const char* b1t = reinterpret_cast<const char*>(p.b1) + (B_NN ? n0 : n0 * p.ldb1) * (int64_t)sizeof(T);
  // per-lane offsets, shared like the prefetch registers: A's first, then B's
  // (with the ping-pong each wave only holds its own role's)
  constexpr int NOB = B_NN ? C::CBN : C::CB;
  constexpr int OFFO = PP ? 0 : C::CA;
  uint32_t off[PP ? (C::CA > NOB ? C::CA : NOB) : C::CA + NOB];
  uint32_t* offa = off;
  uint32_t* offb = off + OFFO;
  if (role_a) {
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int q = lt + i * NTL;
      offa[i] = (uint32_t)(((q >> 3) * p.lda1 + (q & 7) * E) * (int64_t)sizeof(T));
    }
  }
  if (role_b) {
    if constexpr (!B_NN) {
#pragma unroll
      for (int i = 0; i < C::CB; ++i) {
        const int q = lt + i * NTL;
        offb[i] = (uint32_t)(((q >> 3) * p.ldb1 + (q & 7) * E) * (int64_t)sizeof(T));
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::CBN; ++i) {
        const int q = lt + i * NTL;
        offb[i] = (uint32_t)(((q & 7) * E * p.ldb1 + (q >> 3) * E) * (int64_t)sizeof(T));
      }
    }
  }

  // ---- A role: global -> registers ----
  auto load_a = [&](int t) {
    const bool seg1 = t < nk1;
    const int64_t kb = seg1 ? kbeg + (int64_t)t * BK : (int64_t)(t - nk1) * BK;
    if (seg1 && a_full && kb + BK <= kend) {
      const char* base = a1t + kb * (int64_t)sizeof(T);
#pragma unroll
      for (int i = 0; i < C::CA; ++i) pre[i] = *reinterpret_cast<const u32x4*>(base + offa[i]);
      return;
    }
    const T* A = reinterpret_cast<const T*>(seg1 ? p.a1 : p.a2);
    const int64_t lda = seg1 ? p.lda1 : p.lda2;
    const int64_t kv = seg1 ? kend : p.K2;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int q = lt + i * NTL;
      const int64_t gm = m0 + (q >> 3), gk = kb + (q & 7) * E;
      u32x4 v = zero4;
      if (gm < p.m_load && gk < kv) v = *reinterpret_cast<const u32x4*>(A + gm * lda + gk);
      pre[i] = v;
    }
  };

  // ---- B role: global -> registers ----
  auto load_b = [&](int t) {
    u32x4* rb = pre + C::OFFB;
    const bool seg1 = t < nk1;
    const int64_t kb = seg1 ? kbeg + (int64_t)t * BK : (int64_t)(t - nk1) * BK;
    const int64_t kv = seg1 ? kend : p.K2;
    if constexpr (BL == BL_NF4) {
      if (seg1) {
        if constexpr (!B_NN) {
          // W rows n, 64 contraction elements = one NF4 block per row per stage
#pragma unroll
          for (int i = 0; i < C::CNF; ++i) {
            const int u = lt + i * NTL;
            const int row = u >> 1, half = u & 1;
            const int64_t gn = n0 + row;
            u32x4 v = zero4;
            float am = 0.f;
            if (u < C::NF4U && gn < p.n_load && kb < kv) {
              v = *reinterpret_cast<const u32x4*>(p.codes + gn * p.codes_ld + (kb >> 1) + half * 16);
              am = p.absmax[gn * p.blocks_per_row + (kb >> 6)];
            }
            rb[i] = v;
            pam[i] = am;
          }
        } else {
          // W rows = contraction (d_out), columns = n (d_in): 8x8 blocks
#pragma unroll
          for (int i = 0; i < C::CNFB; ++i) {
            const int q = lt + i * NTL;
            const int kbk = q & 7, nb = q >> 3;
            const int64_t gn = n0 + nb * 8;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
              const int64_t gk = kb + kbk * 8 + rr;
              uint32_t v = 0;
              float am = 0.f;
              if (q < C::NF4B && gn < p.n_load && gk < kv) {
                v = *reinterpret_cast<const uint32_t*>(p.codes + gk * p.codes_ld + (gn >> 1));
                am = p.absmax[gk * p.blocks_per_row + (gn >> 6)];
              }
              rb[i * 2 + (rr >> 2)][rr & 3] = v;
              pam[i * 8 + rr] = am;
            }
          }
        }
        return;
      }
    }
    if (BL == BL_PLAIN && seg1 && b_full && kb + BK <= kend) {
      if constexpr (!B_NN) {
        const char* base = b1t + kb * (int64_t)sizeof(T);
#pragma unroll
        for (int i = 0; i < C::CB; ++i) rb[i] = *reinterpret_cast<const u32x4*>(base + offb[i]);
      } else {
#pragma unroll
        for (int i = 0; i < C::CBN; ++i) {
          const int q = lt + i * NTL;
#pragma unroll
          for (int rr = 0; rr < E; ++rr) {
            const char* base = b1t + (kb + rr) * p.ldb1 * (int64_t)sizeof(T);
            u32x4 v = zero4;
            if (q < C::NBLK) v = *reinterpret_cast<const u32x4*>(base + offb[i]);
            rb[i * E + rr] = v;
          }
        }
      }
      return;
    }
    const T* B = reinterpret_cast<const T*>(seg1 ? p.b1 : p.b2);
    const int64_t ldb = seg1 ? p.ldb1 : p.ldb2;
    if constexpr (!B_NN) {
#pragma unroll
      for (int i = 0; i < C::CB; ++i) {
        const int q = lt + i * NTL;
        const int64_t gn = n0 + (q >> 3), gk = kb + (q & 7) * E;
        u32x4 v = zero4;
        if (gn < p.n_load && gk < kv) v = *reinterpret_cast<const u32x4*>(B + gn * ldb + gk);
        rb[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::CBN; ++i) {
        const int q = lt + i * NTL;
        const int kbk = q & 7, nb = q >> 3;
        const int64_t gn = n0 + nb * E;
#pragma unroll
        for (int rr = 0; rr < E; ++rr) {
          const int64_t gk = kb + kbk * E + rr;
          u32x4 v = zero4;
          if (q < C::NBLK && gn < p.n_load && gk < kv) v = *reinterpret_cast<const u32x4*>(B + gk * ldb + gn);
          rb[i * E + rr] = v;
        }
      }
    }
  };

  // ---- A role: registers -> LDS stage s ----
  auto store_a = [&](int s) {
    char* sA = smem + s * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int q = lt + i * NTL;
      *reinterpret_cast<u32x4*>(sA + lds_off(q >> 3, q & 7)) = pre[i];
    }
  };

  // ---- B role: registers -> LDS stage s (transposing / dequantising) ----
  auto store_b = [&](int t, int s) {
    const u32x4* rb = pre + C::OFFB;
    char* sB = smem + s * C::STAGE + BM * 128;
    if constexpr (BL == BL_NF4) {
      if (t < nk1) {
        if constexpr (!B_NN) {
#pragma unroll
          for (int i = 0; i < C::CNF; ++i) {
            const int u = lt + i * NTL;
            if (u < C::NF4U) {
              const int row = u >> 1, half = u & 1;
              const u32x4 v = rb[i];
              const float am = pam[i];
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const uint32_t word = v[w];  // 4 bytes = 8 elements
                u32x4 o;
                o[0] = nf4_byte_to_bf16x2(tab2, word, am);
                o[1] = nf4_byte_to_bf16x2(tab2, word >> 8, am);
                o[2] = nf4_byte_to_bf16x2(tab2, word >> 16, am);
                o[3] = nf4_byte_to_bf16x2(tab2, word >> 24, am);
                *reinterpret_cast<u32x4*>(sB + lds_off(row, half * 4 + w)) = o;
              }
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < C::CNFB; ++i) {
            const int q = lt + i * NTL;
            if (q < C::NF4B) {
              const int kbk = q & 7, nb = q >> 3;
              // dequantise the 8x8 block: rows rr (contraction), columns j (n)
              uint32_t pk[8][4];  // [rr][byte] -> bf16x2 of columns 2b, 2b+1
#pragma unroll
              for (int rr = 0; rr < 8; ++rr) {
                const uint32_t word = rb[i * 2 + (rr >> 2)][rr & 3];
                const float am = pam[i * 8 + rr];
#pragma unroll
                for (int b = 0; b < 4; ++b) pk[rr][b] = nf4_byte_to_bf16x2(tab2, word >> (8 * b), am);
              }
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                u32x4 o;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                  const uint32_t x0 = pk[2 * pp][j >> 1], x1 = pk[2 * pp + 1][j >> 1];
                  o[pp] = (j & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
                }
                *reinterpret_cast<u32x4*>(sB + lds_off(nb * 8 + j, kbk)) = o;
              }
            }
          }
        }
        return;
      }
    }
    if constexpr (!B_NN) {
#pragma unroll
      for (int i = 0; i < C::CB; ++i) {
        const int q = lt + i * NTL;
        *reinterpret_cast<u32x4*>(sB + lds_off(q >> 3, q & 7)) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::CBN; ++i) {
        const int q = lt + i * NTL;
        if (q < C::NBLK) {
          const int kbk = q & 7, nb = q >> 3;
          if constexpr (BF16) {
            // 8x8 transpose of 16-bit values: column j of the block becomes
            // one 16-byte LDS chunk holding rows 0..7.
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              u32x4 o;
#pragma unroll
              for (int pp = 0; pp < 4; ++pp) {
                const uint32_t x0 = rb[i * 8 + 2 * pp][j >> 1];
                const uint32_t x1 = rb[i * 8 + 2 * pp + 1][j >> 1];
                o[pp] = (j & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
              }
              *reinterpret_cast<u32x4*>(sB + lds_off(nb * 8 + j, kbk)) = o;
            }
          } else {
            // 4x4 transpose of 32-bit values
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              u32x4 o;
              o[0] = rb[i * 4 + 0][j];
              o[1] = rb[i * 4 + 1][j];
              o[2] = rb[i * 4 + 2][j];
              o[3] = rb[i * 4 + 3][j];
              *reinterpret_cast<u32x4*>(sB + lds_off(nb * 4 + j, kbk)) = o;
            }
          }
        }
      }
    }
  };

  auto load_role = [&](int t) {
    if (role_a) load_a(t);
    if (role_b) load_b(t);
  };
  auto store_role = [&](int t, int s) {
    if (role_a) store_a(s);
    if (role_b) store_b(t, s);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_stage = [&](int s) {
    const char* sA = smem + s * C::STAGE;
    const char* sB = sA + BM * 128;
    if constexpr (BF16) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                 sA + lds_off(wm * C::TM + i * 16 + l16, kk * 4 + g)));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                  sB + lds_off(wn * C::TN + j * 16 + l16, kk * 4 + g)));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // each lane group g owns contraction elements 8g .. 8g+7 of the stage
      float af[FM][8], bfr[FN][8];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * C::TM + i * 16 + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + lds_off(row, 2 * g));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + lds_off(row, 2 * g + 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t ul = lo[e], uh = hi[e];  // copy out of the vector before the bit cast
          af[i][e] = __builtin_bit_cast(float, ul);
          af[i][4 + e] = __builtin_bit_cast(float, uh);
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * C::TN + j * 16 + l16;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(sB + lds_off(row, 2 * g));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(sB + lds_off(row, 2 * g + 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t ul = lo[e], uh = hi[e];
          bfr[j][e] = __builtin_bit_cast(float, ul);
          bfr[j][4 + e] = __builtin_bit_cast(float, uh);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][kk], bfr[j][kk], acc[i][j], 0, 0, 0);
    }
  };

  // ---------------- main loop ----------------
  if (nk > 0) {
    if constexpr (BL == BL_NF4) {
      nf4_fill_tab2(tab2, p.nf4_table, tid, NT);
      __syncthreads();  // tab2 ready before the first dequantising store
    }
    load_role(0);
    store_role(0, 0);
    if constexpr (PP) {
      if (nk > 1) load_role(1);
      lds_barrier();
      const bool first = wave < WM * WN / 2;  // computes in the first phase of each stage
      for (int t = 0; t < nk; ++t) {
        if (first) {
          compute_stage(t & 1);
          lds_barrier();
          if (t + 1 < nk) store_role(t + 1, (t + 1) & 1);
          if (t + 2 < nk) load_role(t + 2);
          lds_barrier();
        } else {
          if (t + 1 < nk) store_role(t + 1, (t + 1) & 1);
          if (t + 2 < nk) load_role(t + 2);
          lds_barrier();
          compute_stage(t & 1);
          lds_barrier();
        }
      }
    } else {
      __syncthreads();
      for (int t = 0; t < nk; ++t) {
        if (t + 1 < nk) load_role(t + 1);
        compute_stage(t & 1);
        if (t + 1 < nk) store_role(t + 1, (t + 1) & 1);
        __syncthreads();
      }
    }
  }

  // ---------------- epilogue ----------------
  // acc[i][j][v] holds C[row, col] with
  //   row = m0 + wm*TM + 16 i + 4 g + v,  col = n0 + wn*TN + 16 j + l16.
  const int64_t rbase = m0 + wm * C::TM + 4 * g;
  const int64_t cbase = n0 + wn * C::TN + l16;
  if constexpr (EPI == EPI_PARTIAL) {
    float* out = reinterpret_cast<float*>(p.c) + (int64_t)z * p.part_stride;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = rbase + i * 16 + v;
        if (row >= p.m_store) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = cbase + j * 16;
          if (col < p.n_store) out[row * p.ldc + col] = acc[i][j][v];
        }
      }
  } else if constexpr (EPI == EPI_ROPE) {
    // 128-wide wave columns are whole heads: column 16j + l16 (j < 4) pairs
    // with 16(j+4) + l16, both in this lane.  cos/sin row = positions[row].
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = rbase + i * 16 + v;
        if (row >= p.m_store) continue;
        const int32_t q = p.pos[row];
        const bool ok = rope_pos_ok(q, p.max_pos);
        const int64_t prow = ok ? (int64_t)q * 64 : 0;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int f = j * 16 + l16;
          const int64_t col = cbase + j * 16;
          if (col >= p.n_store) continue;
          const float cs = ok ? p.cosc[prow + f] : 0.f, sn = ok ? p.sinc[prow + f] : 0.f;
          const float z1 = acc[i][j][v] * p.alpha, z2 = acc[i][j + FN / 2][v] * p.alpha;
          store_out<T>(p.c, row * p.ldc + col, z1 * cs - z2 * sn);
          store_out<T>(p.c, row * p.ldc + col + 64, z2 * cs + z1 * sn);
        }
      }
  } else if constexpr (EPI == EPI_ADD || EPI == EPI_ADD_MASKED) {
    // Staged through LDS in blocks of RB rows (fp32, row pitch BN + 4 floats:
    // the 16x16 output layout writes without bank conflicts), then each thread
    // adds 8 consecutive outputs to the addend with 16-byte accesses and one
    // keep byte per 8 columns (n_store is a multiple of 8).
    constexpr int PITCH = BN + 4;
    constexpr int RB0 = C::LDS / (PITCH * 4);
    constexpr int RB = RB0 >= BM ? BM : (RB0 / C::TM) * C::TM;
    static_assert(RB >= C::TM, "the LDS holds at least one wave's rows");
    float* stile = reinterpret_cast<float*>(smem);
    __syncthreads();
    for (int rb = 0; rb < BM; rb += RB) {
      if (wm * C::TM >= rb && wm * C::TM < rb + RB) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              stile[(wm * C::TM + i * 16 + 4 * g + v - rb) * PITCH + wn * C::TN + j * 16 + l16] =
                  acc[i][j][v] * p.alpha;
      }
      __syncthreads();
      const int rows_here = BM - rb < RB ? BM - rb : RB;  // the tile's last block may be shorter
      for (int c = tid; c < rows_here * (BN / 8); c += NT) {
        const int lr = c / (BN / 8), lc = (c % (BN / 8)) * 8;
        const int64_t row = m0 + rb + lr, col = n0 + lc;
        if (row >= p.m_store || col >= p.n_store) continue;
        const float4 y0 = *reinterpret_cast<const float4*>(stile + lr * PITCH + lc);
        const float4 y1 = *reinterpret_cast<const float4*>(stile + lr * PITCH + lc + 4);
        const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
        uint32_t keep = 0xFFu;
        if constexpr (EPI == EPI_ADD_MASKED) keep = p.mask[row * p.mask_ld + (col >> 3)];
        if constexpr (BF16) {
          const u32x4 in = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.cin) + row * p.ldcin + col);
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float lo = __builtin_bit_cast(float, in[q] << 16), hi = __builtin_bit_cast(float, in[q] & 0xFFFF0000u);
            if ((keep >> (2 * q)) & 1u) lo += y[2 * q];
            if ((keep >> (2 * q + 1)) & 1u) hi += y[2 * q + 1];
            o[q] = pack_bf16x2(lo, hi);
          }
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.c) + row * p.ldc + col) = o;
        } else {
          const float* in = reinterpret_cast<const float*>(p.cin) + row * p.ldcin + col;
          float4 a = *reinterpret_cast<const float4*>(in), b = *reinterpret_cast<const float4*>(in + 4);
          float o[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if ((keep >> e) & 1u) o[e] += y[e];
          float* out = reinterpret_cast<float*>(p.c) + row * p.ldc + col;
          *reinterpret_cast<float4*>(out) = make_float4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<float4*>(out + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = rbase + i * 16 + v;
        if (row >= p.m_store) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = cbase + j * 16;
          if (col >= p.n_store) continue;
          const float y = acc[i][j][v] * p.alpha;
          if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_BOTH) store_out<T>(p.c, row * p.ldc + col, y);
          if constexpr (EPI == EPI_STORE_T || EPI == EPI_STORE_BOTH) store_out<T>(p.ct, col * p.ldct + row, y);
        }
      }
  }
}

}  // namespace lora
