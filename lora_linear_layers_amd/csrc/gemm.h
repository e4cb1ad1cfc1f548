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
// 32 fp32), two LDS stages, one barrier per stage.  Waves form a WM x WN grid
// and each owns a (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks.
// bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses v_mfma_f32_16x16x4_f32 (true
// fp32 products, no reduced-precision inputs).
//
// LDS rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r is stored at
// chunk c ^ ((r & 7) ^ ((r >> 3) & 1)), which spreads both the 16-byte stores
// of the loaders and the 16-byte fragment reads of 16 consecutive rows over
// distinct banks.
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
  EPI_PARTIAL = 4      // fp32 partial slab of split z: C[z][m, n] = acc
};

enum BLoad : int { BL_PLAIN = 0, BL_NF4 = 1 };

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
  const uint8_t* codes;     // BL_NF4: packed codes of W [n_load rows? see loader], bytes per row
  const float* absmax;
  int64_t codes_ld;         // bytes per W row (= d_in / 2)
  int64_t blocks_per_row;   // absmax entries per W row (= d_in / 64)
  float nf4_table[16];
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return (row << 7) + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
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

__device__ __forceinline__ void nf4_fill_tab2(float2* tab2, const float* table, int tid, int nt) {
  for (int t = tid; t < 256; t += nt) tab2[t] = make_float2(table[t >> 4], table[t & 15]);
}

template <typename T, int BM, int BN, int WM, int WN, bool B_NN, int EPI, int BL>
struct GemmCfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(T);
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr int LDS = 2 * STAGE + (BL == BL_NF4 ? 2048 : 0);
  // per-thread load counts
  static constexpr int CA = (BM * 8 + NT - 1) / NT;             // A chunks
  static constexpr int CB = (BN * 8 + NT - 1) / NT;             // B chunks (NT layout)
  static constexpr int NBLK = 8 * (BN / E);                     // B blocks (NN layout), E x E each
  static constexpr int CBN = (NBLK + NT - 1) / NT;
  static constexpr int NF4U = BN * 2;                           // NF4 half-row units (NT layout)
  static constexpr int CNF = (NF4U + NT - 1) / NT;
  static constexpr int NF4B = 8 * (BN / 8);                     // NF4 8x8 blocks (NN layout)
  static constexpr int CNFB = (NF4B + NT - 1) / NT;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile/wave mismatch");
  static_assert(EPI != EPI_ROPE || TN == 128, "RoPE epilogue needs 128-wide wave columns");
  static_assert(BL == BL_PLAIN || sizeof(T) == 2, "NF4 weights feed bf16 MFMA");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <typename T, int BM, int BN, int WM, int WN, bool B_NN, int EPI, int BL>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const GemmArgs p) {
  using C = GemmCfg<T, BM, BN, WM, WN, B_NN, EPI, BL>;
  constexpr int NT = C::NT, E = C::E, BK = C::BK, FM = C::FM, FN = C::FN;
  constexpr bool BF16 = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  float2* tab2 = reinterpret_cast<float2*>(smem + 2 * C::STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l16 = lane & 15, g = lane >> 4;

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
  const int nk2 = (EPI == EPI_PARTIAL) ? 0 : (int)((p.K2 + BK - 1) / BK);
  const int nk = nk1 + nk2;

  if constexpr (BL == BL_NF4) {
    nf4_fill_tab2(tab2, p.nf4_table, tid, NT);
  }

  // ---------------- prefetch registers ----------------
  u32x4 ra[C::CA];
  u32x4 rb[B_NN ? 1 : C::CB];
  u32x4 rbn[B_NN ? C::CBN * E : 1];
  u32x4 rnf[BL == BL_NF4 && !B_NN ? C::CNF : 1];
  float ramf[BL == BL_NF4 && !B_NN ? C::CNF : 1];
  uint32_t rnfb[BL == BL_NF4 && B_NN ? C::CNFB * 8 : 1];
  float ramb[BL == BL_NF4 && B_NN ? C::CNFB * 8 : 1];

  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  auto load_stage = [&](int t) {
    const bool seg1 = t < nk1;
    const T* A = reinterpret_cast<const T*>(seg1 ? p.a1 : p.a2);
    const T* B = reinterpret_cast<const T*>(seg1 ? p.b1 : p.b2);
    const int64_t lda = seg1 ? p.lda1 : p.lda2;
    const int64_t ldb = seg1 ? p.ldb1 : p.ldb2;
    const int64_t kb = seg1 ? kbeg + (int64_t)t * BK : (int64_t)(t - nk1) * BK;
    const int64_t kv = seg1 ? kend : p.K2;
    // A: BM rows x 8 chunks
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int q = tid + i * NT;
      const int row = q >> 3, c = q & 7;
      const int64_t gm = m0 + row, gk = kb + c * E;
      u32x4 v = zero4;
      if (q < BM * 8 && gm < p.m_load && gk < kv)
        v = *reinterpret_cast<const u32x4*>(A + gm * lda + gk);
      ra[i] = v;
    }
    if constexpr (BL == BL_NF4) {
      if (seg1) {
        if constexpr (!B_NN) {
          // W rows n, 64 contraction elements = one NF4 block per row per stage
#pragma unroll
          for (int i = 0; i < C::CNF; ++i) {
            const int u = tid + i * NT;
            const int row = u >> 1, half = u & 1;
            const int64_t gn = n0 + row;
            u32x4 v = zero4;
            float am = 0.f;
            if (u < C::NF4U && gn < p.n_load && kb < kv) {
              v = *reinterpret_cast<const u32x4*>(p.codes + gn * p.codes_ld + (kb >> 1) + half * 16);
              am = p.absmax[gn * p.blocks_per_row + (kb >> 6)];
            }
            rnf[i] = v;
            ramf[i] = am;
          }
        } else {
          // W rows = contraction (d_out), columns = n (d_in): 8x8 blocks
#pragma unroll
          for (int i = 0; i < C::CNFB; ++i) {
            const int q = tid + i * NT;
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
              rnfb[i * 8 + rr] = v;
              ramb[i * 8 + rr] = am;
            }
          }
        }
        return;
      }
    }
    if constexpr (!B_NN) {
#pragma unroll
      for (int i = 0; i < C::CB; ++i) {
        const int q = tid + i * NT;
        const int row = q >> 3, c = q & 7;
        const int64_t gn = n0 + row, gk = kb + c * E;
        u32x4 v = zero4;
        if (q < BN * 8 && gn < p.n_load && gk < kv)
          v = *reinterpret_cast<const u32x4*>(B + gn * ldb + gk);
        rb[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::CBN; ++i) {
        const int q = tid + i * NT;
        const int kbk = q & 7, nb = q >> 3;
        const int64_t gn = n0 + nb * E;
#pragma unroll
        for (int rr = 0; rr < E; ++rr) {
          const int64_t gk = kb + kbk * E + rr;
          u32x4 v = zero4;
          if (q < C::NBLK && gn < p.n_load && gk < kv)
            v = *reinterpret_cast<const u32x4*>(B + gk * ldb + gn);
          rbn[i * E + rr] = v;
        }
      }
    }
  };

  auto store_stage = [&](int t, int s) {
    char* sA = smem + s * C::STAGE;
    char* sB = sA + BM * 128;
#pragma unroll
    for (int i = 0; i < C::CA; ++i) {
      const int q = tid + i * NT;
      if (q < BM * 8) *reinterpret_cast<u32x4*>(sA + lds_off(q >> 3, q & 7)) = ra[i];
    }
    if constexpr (BL == BL_NF4) {
      if (t < nk1) {
        if constexpr (!B_NN) {
#pragma unroll
          for (int i = 0; i < C::CNF; ++i) {
            const int u = tid + i * NT;
            if (u < C::NF4U) {
              const int row = u >> 1, half = u & 1;
              const u32x4 v = rnf[i];
              const float am = ramf[i];
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
            const int q = tid + i * NT;
            if (q < C::NF4B) {
              const int kbk = q & 7, nb = q >> 3;
              // dequantise the 8x8 block: rows rr (contraction), columns j (n)
              uint32_t pk[8][4];  // [rr][byte] -> bf16x2 of columns 2b, 2b+1
#pragma unroll
              for (int rr = 0; rr < 8; ++rr) {
                const uint32_t word = rnfb[i * 8 + rr];
                const float am = ramb[i * 8 + rr];
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
        const int q = tid + i * NT;
        if (q < BN * 8) *reinterpret_cast<u32x4*>(sB + lds_off(q >> 3, q & 7)) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::CBN; ++i) {
        const int q = tid + i * NT;
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
                const uint32_t x0 = rbn[i * 8 + 2 * pp][j >> 1];
                const uint32_t x1 = rbn[i * 8 + 2 * pp + 1][j >> 1];
                o[pp] = (j & 1) ? ((x0 >> 16) | (x1 & 0xFFFF0000u)) : ((x0 & 0xFFFFu) | (x1 << 16));
              }
              *reinterpret_cast<u32x4*>(sB + lds_off(nb * 8 + j, kbk)) = o;
            }
          } else {
            // 4x4 transpose of 32-bit values
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              u32x4 o;
              o[0] = rbn[i * 4 + 0][j];
              o[1] = rbn[i * 4 + 1][j];
              o[2] = rbn[i * 4 + 2][j];
              o[3] = rbn[i * 4 + 3][j];
              *reinterpret_cast<u32x4*>(sB + lds_off(nb * 4 + j, kbk)) = o;
            }
          }
        }
      }
    }
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

  // ---------------- main loop: two LDS stages, one barrier per stage -------
  if (nk > 0) {
    load_stage(0);
    if constexpr (BL == BL_NF4) __syncthreads();  // tab2 ready
    store_stage(0, 0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      if (t + 1 < nk) load_stage(t + 1);
      compute_stage(t & 1);
      if (t + 1 < nk) store_stage(t + 1, (t + 1) & 1);
      __syncthreads();
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
        const int64_t prow = (int64_t)p.pos[row] * 64;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int f = j * 16 + l16;
          const int64_t col = cbase + j * 16;
          if (col >= p.n_store) continue;
          const float cs = p.cosc[prow + f], sn = p.sinc[prow + f];
          const float z1 = acc[i][j][v] * p.alpha, z2 = acc[i][j + FN / 2][v] * p.alpha;
          store_out<T>(p.c, row * p.ldc + col, z1 * cs - z2 * sn);
          store_out<T>(p.c, row * p.ldc + col + 64, z2 * cs + z1 * sn);
        }
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
