// few_args.h - the launch arguments and tile constants of the few-token path
// (kernels in few.h), shared by the host code that plans and launches it.
#pragma once

#include <stdint.h>

namespace lora {

namespace few {
constexpr int NT = 256;                // threads per block
constexpr int NW4 = 8;                 // waves of the NF4 forward's W-streaming block
constexpr int NT4 = 64 * NW4;          // its threads
constexpr int BN = 128;                // output columns per block (one RoPE head)
constexpr int BK = 64;                 // contraction per stage
constexpr int MAXMB = 8;               // 16-row blocks of tokens (M <= 128)
constexpr int MAXR = 64;               // rank (a multiple of 8)
constexpr int GRID = 256;              // blocks of the W-streaming launch: one per MI355X CU
constexpr uint32_t OOB = 0x80000000u;  // lane offset past every resource: reads zero
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }
}  // namespace few

struct FewArgs {
  int M, Mp;   // tokens; rows padded to 16 MB
  int d_in, d_out, r8;
  float s;
  const uint16_t* X;     // [M, d_in]
  const uint16_t* W;     // [d_out, d_in] bf16, or NULL with codes / absmax (NF4)
  const uint8_t* codes;  // [d_out, d_in / 2]
  const float* absmax;   // [d_out, d_in / 64]
  float nf4_table[16];
  const uint16_t* A;     // [r8, d_in]
  const uint16_t* B;     // [d_out, r8]
  const uint16_t* dY;    // [M, d_out]
  uint16_t* G;           // RoPE backward: launch 1 stores R(-angle) dY here, launch 2 reads it
  uint16_t* Y;           // [M, d_out]
  uint16_t* dX;          // [M, d_in]
  float* dA;             // [r8, d_in]
  float* dB;             // [d_out, r8]
  const int32_t* pos;    // RoPE (rope != 0): position of each token
  const float* cosc;
  const float* sinc;
  int64_t max_pos;
  int rope;
  float* Pp;  // [Sp][Mp][r8] fp32 partials of X A^T
  float* Qp;  // [Sq][Mp][r8] fp32 partials of G B
  float* Cp;  // [nblk + n_tiles - 1][Mp][BN] fp32 partials of the main product, one per (block, tile)
  int* cnt;   // [n_tiles] arrival counters of launch 2 (cleared by launch 1)
  uint16_t* Ps;  // backward: bf16(s P) [Mp, r8] (few_reduce_kernel)
  uint16_t* Qs;  // backward: bf16(s Q) [Mp, r8]
  int Sp, Kp;  // P: chunks of d_in of Kp (a multiple of 32)
  int pg;      // P: 16-row groups of tokens per chunk, a block each (1: one block takes every row)
  int Sq, Kq;  // Q: chunks of d_out of Kq (a multiple of 128)
  // launch 2: n_tiles column tiles of BN, nkt stages of BK each; block b of
  // nblk takes the stages [b T / nblk, (b + 1) T / nblk) of the T = n_tiles nkt
  int n_tiles, nkt, T, nblk;
  int fold;  // backward: the W stream sums P and Q from the partials itself (no few_reduce_kernel)
};

}  // namespace lora
