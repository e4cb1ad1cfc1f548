/*
 * lora_linear.h - C ABI of the MI355X (gfx950) fused LoRA linear layer.
 *
 * The layer (page "UnSloth加速微调体验：在LoRA基础上再提速3倍的秘密", section
 * 算子融合, equation y = Wx + ΔWx = Wx + BAx, with B in R^{d x r} and
 * A in R^{r x k}) computes, for every token x (one row of X):
 *
 *     y = W x + s * B (A x),        s = alpha / r (the caller passes s)
 *
 * with the base weight W frozen.  Row-major, one token per row:
 *
 *     X  [M, d_in]     W  [d_out, d_in]     A [r, d_in]     B [d_out, r]
 *     Y  [M, d_out]    dY [M, d_out]        dX [M, d_in]
 *     dA [r, d_in] fp32                     dB [d_out, r] fp32
 *
 * Backward (section 反向传播优化 of the same page; its printed gradient formulas
 * are garbled, these follow the chain rule):
 *
 *     dX = dY W + s (dY B) A,   dB = s dY^T (X A^T),   dA = s (dY B)^T X
 *
 * X A^T is recomputed, never stored by the forward.  No dW is ever formed:
 * only the adapters train (page "Unsloth教程：本地微调大模型速度提升数倍，显存
 * 节省60%", section 显存优化策略, 4-bit QLoRA paragraph).
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers (caller-owned, e.g. torch allocations) unless
 *    an argument says "host".  The library never allocates or frees device
 *    memory; scratch space comes from the caller's workspace `ws` of
 *    `ws_bytes` bytes, sized by lora_workspace_bytes().  The workspace holds
 *    nothing between calls.
 *  - bf16 tensors are passed as their 16-bit patterns.  Accumulation is fp32.
 *    dA and dB are always fp32 and are OVERWRITTEN (not accumulated into).
 *  - `stream` is a hipStream_t (NULL = default stream).  Calls only enqueue
 *    work on it and never synchronise.  The library is re-entrant; calls that
 *    share a workspace must be ordered by the caller.
 *  - Every pointer must be 16-byte aligned; d_in and d_out must be multiples
 *    of 8; 1 <= r <= 256; M >= 0 (M = 0 gives empty Y/dX and zero dA, dB; the
 *    pointers to the M-row tensors X, Y, dY, dX and positions may then be NULL).
 *  - Validation happens before any HIP call: on error nothing is launched and
 *    no output is touched.  A failed launch returns LORA_ERR_DEVICE.  No
 *    exception crosses the ABI and nothing is printed.
 *  - A shape the kernels do not support returns LORA_ERR_SHAPE; there is no
 *    slower fallback path.
 */
#ifndef LORA_LINEAR_H
#define LORA_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 1

/* Largest RoPE cache (rows) the q/k projections accept: 2^23 - 1, so that a
 * row's byte offset (256 bytes a row) stays below 2^31. */
#define LORA_ROPE_MAX_POS ((1 << 23) - 1)

/* element types of X, W, A, B, Y, dY, dX */
enum { LORA_F32 = 0, LORA_BF16 = 1 };

/* return codes */
enum {
  LORA_OK = 0,
  LORA_ERR_NULL = -1,      /* a required pointer is NULL */
  LORA_ERR_SHAPE = -2,     /* a size is out of range or breaks a divisibility rule */
  LORA_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
  LORA_ERR_DTYPE = -4,     /* unknown dtype, or a dtype the entry point does not take */
  LORA_ERR_WORKSPACE = -5, /* ws_bytes < lora_workspace_bytes(...) or ws NULL when needed */
  LORA_ERR_DEVICE = -6,    /* current device is not gfx950, or a launch failed */
  LORA_ERR_SCRATCH = -7    /* lora_linear_fwd_noalloc: the problem needs more than the static scratch */
};

/* operation ids for lora_workspace_bytes */
enum {
  LORA_OP_FWD = 0,
  LORA_OP_BWD = 1,
  LORA_OP_ROPE_FWD = 2,
  LORA_OP_ROPE_BWD = 3,
  LORA_OP_NF4_FWD = 4,
  LORA_OP_NF4_BWD = 5,
  LORA_OP_MERGE = 6,
  LORA_OP_DROPOUT_FWD = 7,
  LORA_OP_DROPOUT_BWD = 8
};

/* Library version; equals LORA_ABI_VERSION of the header it was built from. */
int lora_abi_version(void);

/* Static description of a return code ("ok", "null pointer", ...). */
const char* lora_strerror(int code);

/*
 * Bytes of workspace that entry point `op` needs for these sizes (0 if none).
 * Pure host arithmetic; no device query.  Returns 0 for invalid arguments
 * (the entry point itself then reports the error).
 */
size_t lora_workspace_bytes(int op, int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r);

/*
 * Forward: Y = X W^T + s (X A^T) B^T.
 * Page "UnSloth加速微调体验…", section 算子融合: W x and the low-rank update are
 * produced by one fused pass; the rank-r panel s X A^T is added into the same
 * fp32 accumulator as X W^T, so no intermediate of size [M, d_out] exists.
 * dtype: LORA_F32 or LORA_BF16 (X, W, A, B, Y all of that type).
 */
int lora_linear_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                    const void* X, const void* W, const void* A, const void* B, void* Y,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * lora_linear_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same result as lora_linear_fwd, bit for bit, with no workspace
 * argument.  Its scratch is a static device array inside the library,
 * LORA_STATIC_SCRATCH_BYTES (32 MiB) per GPU, held by every GPU the library
 * runs on until the process ends; the call itself never allocates or frees
 * memory.  The caller still passes X, W, A, B and Y.  Problems whose
 * workspace (lora_workspace_bytes(LORA_OP_FWD, ...)) exceeds that size
 * return LORA_ERR_SCRATCH before any launch (bf16 at r = 64 fits up to about
 * 87000 tokens at the large-weight shapes).  All calls on one GPU share its array, which keeps the last
 * call's contents: calls that overlap on one GPU (different streams, or
 * threads without ordering) race and must be serialised by the caller.
 */
#define LORA_STATIC_SCRATCH_BYTES (32u << 20)
int lora_linear_fwd_noalloc(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                            const void* X, const void* W, const void* A, const void* B, void* Y,
                            void* stream);

/*
 * Backward: dX = dY W + s (dY B) A (skipped when dX is NULL),
 *           dB = s dY^T (X A^T),  dA = s (dY B)^T X  (fp32, overwritten).
 * Page "UnSloth加速微调体验…", section 反向传播优化: X A^T is recomputed here
 * instead of being kept from the forward.  No dW.
 */
int lora_linear_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                    const void* X, const void* W, const void* A, const void* B, const void* dY,
                    void* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/*
 * Fill the RoPE cache: cos_cache[p * head_dim/2 + i] = cos(p * theta^(-2i/head_dim)),
 * sin_cache likewise, for p < max_pos and i < head_dim/2, computed in fp64 and
 * rounded to fp32.  Page "UnSloth加速微调体验…", section RoPE缓存集成: the cos/sin
 * values live in one contiguous block and a position selects a row by a
 * pointer offset.  Both arrays are device fp32 [max_pos, head_dim/2].
 */
int lora_rope_cache(int64_t max_pos, int head_dim, double theta, float* cos_cache,
                    float* sin_cache, void* stream);

/*
 * q/k projection with the RoPE rotation as the forward epilogue
 * (section RoPE缓存集成: the rotation is applied while q_proj(x) + lora_q(x) is
 * produced).  Within every head of width head_dim (must be 128, and d_out a
 * multiple of it), element i pairs with i + 64 and rotates by the angle whose
 * cos/sin sit in row positions[t] of the caches (rotate-half pairing):
 *     y_i = z_i cos - z_{i+64} sin,   y_{i+64} = z_{i+64} cos + z_i sin,
 * where z is the fused LoRA output.  1 <= max_pos <= LORA_ROPE_MAX_POS
 * (2^23 - 1; else LORA_ERR_SHAPE).  positions: device int32 [M], each meant to lie in
 * [0, max_pos).  The host cannot read them before the launch;
 * the kernels check each one against max_pos and read no cache row for a
 * position outside that range: such a row of y comes out as zeros (and in
 * the backward its gradient is taken as zero), so a bad position never reads
 * outside the caches.
 */
int lora_qk_rope_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                     const void* X, const void* W, const void* A, const void* B, int head_dim,
                     const int32_t* positions, const float* cos_cache, const float* sin_cache,
                     int64_t max_pos, void* Y, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of lora_qk_rope_fwd: the inverse rotation (the transpose, angle
 * negated) is applied to dY, then the LoRA backward runs on the result.
 * Outputs as lora_linear_bwd.
 */
int lora_qk_rope_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                     const void* X, const void* W, const void* A, const void* B, int head_dim,
                     const int32_t* positions, const float* cos_cache, const float* sin_cache,
                     int64_t max_pos, const void* dY, void* dX, float* dA, float* dB, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Forward with an NF4 base weight (QLoRA; page "Unsloth教程…", section 显存优化策略;
 * page "Unsloth自动化优化：无需手动调参的实现原理", section 5: NF4 is the default).
 * W_nf4: device uint8 [d_out * d_in / 2], element e = i*d_in + j of W in byte
 * e/2, high nibble for even e.  absmax: device fp32 [d_out * d_in / blocksize],
 * one per block of `blocksize` consecutive elements.  table16: HOST pointer to
 * the 16 fp32 code values (copied into the launch).  The weight used is
 *     W[e] = bf16_rne(fp32_rne(table16[code_e] * absmax[e / blocksize])).
 * Below LORA_NF4_DEQUANT_MIN_TOKENS tokens (M) it is formed inside the GEMM's
 * load stage and never written to memory: there the GEMM is bound by reading
 * W, and the codes are a quarter of its bf16 bytes.  From that M on, either
 * the whole-tile GEMM expands W in its load stage (M and d_out multiples of
 * 256), or the same routine writes W once per call into the workspace
 * (2 * d_out * d_in bytes, included in lora_workspace_bytes) and the bf16
 * GEMMs read it; lora_set_nf4_fwd_path picks between them.  Every path gives
 * the same W bit for bit.
 * blocksize must be 64 and d_in a multiple of 64.  X, A, B, Y are bf16.
 */
#define LORA_NF4_DEQUANT_MIN_TOKENS 512

/*
 * Which NF4 forward path runs from LORA_NF4_DEQUANT_MIN_TOKENS tokens on, for
 * every later call in the process (a measurement and test control):
 *   LORA_NF4_PATH_AUTO        the library's choice by shape (the default);
 *   LORA_NF4_PATH_DEQUANT     W dequantised once per call, then the bf16 GEMM;
 *   LORA_NF4_PATH_LOAD_STAGE  the whole-tile GEMM expanding W in its load
 *                             stage wherever M and d_out are multiples of 256.
 * lora_workspace_bytes depends on it: size the workspace after setting it,
 * and do not change it while a call that was sized under another mode is
 * pending.  Returns the previous mode, or LORA_ERR_SHAPE for another value
 * (no change).  No HIP call.
 */
#define LORA_NF4_PATH_AUTO 0
#define LORA_NF4_PATH_DEQUANT 1
#define LORA_NF4_PATH_LOAD_STAGE 2
int lora_set_nf4_fwd_path(int mode);
int nf4_lora_linear_fwd(int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                        const void* X, const uint8_t* W_nf4, const float* absmax, int blocksize,
                        const float* table16, const void* A, const void* B, void* Y, void* ws,
                        size_t ws_bytes, void* stream);

/* Backward with the NF4 base weight; outputs as lora_linear_bwd.  Never forms dW. */
int nf4_lora_linear_bwd(int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                        const void* X, const uint8_t* W_nf4, const float* absmax, int blocksize,
                        const float* table16, const void* A, const void* B, const void* dY,
                        void* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/*
 * Dequantise n NF4 elements to bf16 bit patterns with the same device routine
 * the NF4 GEMMs use in their load stage (exposed so it can be checked bit for
 * bit).  n must be a multiple of blocksize (64).  table16 is a HOST pointer.
 */
int nf4_dequant(const uint8_t* W_nf4, const float* absmax, int blocksize, int64_t n,
                const float* table16, uint16_t* out_bf16, void* stream);

/*
 * LoRA dropout on the adapter's input (page "微调太慢？试试Unsloth…", section
 * 3.3, configuration E trains with dropout 0.05; page "Unsloth框架：高效LLM微调
 * 与LoRA优化实践", section 2.2, passes lora_dropout = 0.1): inverted dropout
 * D = X * keep / (1 - p) feeds only the rank-r branch, the base path sees X:
 *     Y  = X W^T + s (D A^T) B^T
 *     dX = G W + s ((G B) A) * keep / (1 - p),  dA = s (G B)^T D,  dB = s G^T (D A^T).
 * keep: device bit mask [M, d_in / 8] bytes, bit b of byte (i, j) keeps element
 * (i, 8 j + b); the caller draws it (the library has no random generator) and
 * passes the same mask to the backward.  0 <= p < 1.  The masked copy of X is
 * exact and 1 / (1 - p) joins s in the rank-r panels; the masked rank-r term
 * of dX is a separate rank-r GEMM added into dX.  Other arguments, workspace
 * (op LORA_OP_DROPOUT_FWD / _BWD) and errors as lora_linear_fwd / _bwd;
 * LORA_ERR_SHAPE if p is outside [0, 1).
 */
int lora_dropout_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                     const uint8_t* keep, const void* X, const void* W, const void* A, const void* B, void* Y,
                     void* ws, size_t ws_bytes, void* stream);
int lora_dropout_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                     const uint8_t* keep, const void* X, const void* W, const void* A, const void* B,
                     const void* dY, void* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream);

/*
 * The dropout keep mask drawn on the device from the counter-based generator
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 * as 1, 2, 3", SC'11, section 4), so that a backward regenerates its forward's
 * mask from the same (seed, offset) instead of keeping it.  Element e of the
 * row-major [M, d_in] input takes word e mod 4 of the generator's block for
 * the counter (lo32(e / 4), hi32(e / 4), lo32(offset), hi32(offset)) under the
 * key (lo32(seed), hi32(seed)), and is kept iff that word >= floor(p 2^32).
 * keep: device output [M, d_in / 8] bytes in lora_dropout_fwd's bit order.
 * Needs d_in % 8 == 0 and 0 <= p < 1 (else LORA_ERR_SHAPE); asynchronous.
 */
int lora_dropout_mask(int64_t M, int64_t d_in, float p, uint64_t seed, uint64_t offset, uint8_t* keep,
                      void* stream);

/*
 * lora_dropout_fwd / _bwd with the mask drawn on the device as
 * lora_dropout_mask(M, d_in, p, seed, offset) draws it (one pass over X
 * writes the masked copy and, in the backward, the bits); the same
 * (seed, offset) in the forward and the backward gives the same mask.
 * Results equal lora_dropout_fwd / _bwd given that mask.  Workspace: ops
 * LORA_OP_DROPOUT_FWD / _BWD; errors as there.
 */
int lora_dropout_philox_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                            uint64_t seed, uint64_t offset, const void* X, const void* W, const void* A,
                            const void* B, void* Y, void* ws, size_t ws_bytes, void* stream);
int lora_dropout_philox_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                            uint64_t seed, uint64_t offset, const void* X, const void* W, const void* A,
                            const void* B, const void* dY, void* dX, float* dA, float* dB, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Merge for inference: W_out = W + scale * B A, one GEMM over the rank (fp32
 * accumulation) whose epilogue adds W and rounds once to the output type.
 * Page "微调太慢？试试Unsloth：实测训练速度翻倍，显存占用减半", section 5.1: for
 * inference the adapter is folded into the main weight, so no rank-r branch
 * runs per token; page "Unsloth自动化优化：无需手动调参的实现原理", section 3.2:
 * the adapter product and the original weight combined in one kernel.
 * Unmerge is the same call with -scale (it restores W up to the output type's
 * rounding, since the merge rounded).  W_out may be W (in place: every element
 * is read and written by the same thread, and by no other).  dtype LORA_F32 or
 * LORA_BF16; W, W_out [d_out, d_in], A [r, d_in], B [d_out, r]; workspace of
 * lora_workspace_bytes(LORA_OP_MERGE, dtype, 0, d_in, d_out, r) bytes (a
 * padded copy of B when r is not a multiple of 8, else none).  An NF4 weight
 * cannot absorb the adapter without re-quantising; there is no NF4 merge.
 */
int lora_merge(int dtype, int64_t d_out, int64_t d_in, int64_t r, float scale, const void* W, const void* A,
               const void* B, void* W_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Groups of projections that read the same input X: q/k/v of attention,
 * gate/up of the MLP.  Page "UnSloth加速微调体验…", section RoPE缓存集成 fuses
 * q_proj with its LoRA branch; page "Unsloth框架：高效LLM微调与LoRA优化实践",
 * section 3.1 (graph rewriting), merges adjacent linear layers; page
 * "Unsloth自动化优化：无需手动调参的实现原理", section 3.3, walks the layer as
 * the segments q, k, v, o, gate, up, down.  A group call runs the
 * rank-r panels of all its members in ONE pass over X, with A_1 .. A_n stacked:
 * the forward panel s X A^T, the backward's recomputation of X A^T and the dA
 * contraction over X.  Everything else runs per member exactly as in the
 * single-projection entry points, so every member's outputs equal that
 * member's single call up to rounding order.  (fp32 groups run their members
 * one after another.)
 *
 * `members` is a HOST array of n (1 <= n <= LORA_GROUP_MAX) descriptions whose
 * pointers are device pointers.  Per member: d_out, r and the pointer rules
 * are those of one projection; `scale` is its s; `rope` = 1 gives it the RoPE
 * epilogue of lora_qk_rope_fwd with the group's head_dim / positions / caches
 * (then head_dim must be 128 and d_out a multiple of it); `W_nf4` (with
 * `absmax`, blocksize 64, d_in a multiple of 64, bf16 only, no RoPE) replaces W
 * by an NF4 base weight decoded with the HOST table `table16` as in
 * nf4_lora_linear_fwd.  Forward writes every member's Y.  Backward writes
 * every member's dA, dB and, where dX is not NULL, the member's own input
 * gradient (not summed over the group).  The rope and table arguments may be
 * NULL when no member needs them.
 * On MI355X the whole-tile GEMM reads W^T (rows of W's input dimension)
 * about 12 % faster than W with its contraction rows, so the bf16 backward
 * forms dX = G W from W^T: from `W_t` when the caller keeps one (W is frozen,
 * so one lora_transpose serves every step), else from a per-call transpose
 * in the workspace.
 */
#define LORA_GROUP_MAX 8
typedef struct lora_group_member {
  int64_t d_out, r;
  float scale;
  int rope;
  const void* W;          /* [d_out, d_in], or NULL when W_nf4 is given */
  const uint8_t* W_nf4;   /* NF4 codes [d_out * d_in / 2], or NULL */
  const float* absmax;    /* [d_out * d_in / 64] with W_nf4 */
  const void* A;          /* [r, d_in] */
  const void* B;          /* [d_out, r] */
  void* Y;                /* forward output [M, d_out] */
  const void* dY;         /* backward input [M, d_out] */
  void* dX;               /* backward output [M, d_in], or NULL */
  float* dA;              /* backward output [r, d_in] fp32 */
  float* dB;              /* backward output [d_out, r] fp32 */
  const void* W_t;        /* optional W^T [d_in, d_out] (bf16, e.g. from lora_transpose): the
                             backward's input gradient reads it instead of transposing W per call */
} lora_group_member;

/* Workspace bytes of lora_group_fwd (backward = 0) or lora_group_bwd (1); 0 for
 * invalid arguments. */
size_t lora_group_workspace_bytes(int backward, int dtype, int64_t M, int64_t d_in, int n,
                                  const lora_group_member* members);

int lora_group_fwd(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* members,
                   const void* X, int head_dim, const int32_t* positions, const float* cos_cache,
                   const float* sin_cache, int64_t max_pos, const float* table16, void* ws,
                   size_t ws_bytes, void* stream);

int lora_group_bwd(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* members,
                   const void* X, int head_dim, const int32_t* positions, const float* cos_cache,
                   const float* sin_cache, int64_t max_pos, const float* table16, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * SwiGLU on a gate / up pair that reads the same X (the gated unit of the
 * Llama MLP): G and U are the two fused LoRA projections of X (each as
 * lora_linear_fwd or nf4_lora_linear_fwd), H = silu(G) * U elementwise,
 * silu(z) = z / (1 + e^-z).  Page "Unsloth框架：高效LLM微调与LoRA优化实践",
 * section 3.1: the graph rewriter merges adjacent linear layers with their
 * activation function; page "Unsloth自动化优化：无需手动调参的实现原理",
 * section 1: SwiGLU is one of the module types it optimises.
 * members[0] is the gate and members[1] the up projection (lora_group_member
 * with equal d_out, rope = 0, W or W_nf4 as in the group calls); their rank-r
 * panels run in one pass over X as in lora_group_fwd.  With bf16, M a multiple
 * of 256, d_out of 128, d_in of 64 (and for an NF4 member M >= 512, where its
 * weight is dequantised once), gate and up run as ONE GEMM whose epilogue
 * forms H from the fp32 accumulators; other shapes form G and U with the group
 * path and H in an elementwise pass from G and U rounded to the dtype.
 * H: [M, d_out] in the dtype.  members[g].Y, when not NULL, receives G (g = 0)
 * and U (g = 1) in the dtype, as the backward needs them.
 */
int lora_swiglu_fwd(int dtype, int64_t M, int64_t d_in, const lora_group_member* members, const void* X,
                    const float* table16, void* H, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of lora_swiglu_fwd for the upstream gradient dH [M, d_out]:
 * dG = dH * U * silu'(G) and dU = dH * silu(G) (G, U as the forward stored
 * them; silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z)), then the LoRA
 * backward of both projections with their panels shared as in lora_group_bwd.
 * dX [M, d_in] (NULL: skipped) receives the SUM of the two input gradients;
 * members[g].dA and .dB receive each adapter's gradients (fp32, overwritten);
 * members[g].dY, .dX and .Y are not used.
 */
int lora_swiglu_bwd(int dtype, int64_t M, int64_t d_in, const lora_group_member* members, const void* X,
                    const float* table16, const void* dH, const void* G, const void* U, void* dX, void* ws,
                    size_t ws_bytes, void* stream);

/* Workspace bytes of lora_swiglu_fwd (backward = 0) or lora_swiglu_bwd (1); 0
 * for invalid arguments. */
size_t lora_swiglu_workspace_bytes(int backward, int dtype, int64_t M, int64_t d_in,
                                   const lora_group_member* members);

/*
 * dst [cols, rows] = src [rows, cols]^T for bf16 matrices (rows and cols
 * multiples of 8), e.g. the frozen W^T that the backward can take as
 * lora_group_member.W_t.  Asynchronous on `stream`.
 */
int lora_transpose(const void* src, int64_t rows, int64_t cols, void* dst, void* stream);

/*
 * Launch profiling (measurement hook, not part of the layer's arithmetic).
 * Between lora_profile_begin and lora_profile_end every kernel the library
 * launches is bracketed by two HIP events on its stream, and the launch's
 * algorithmic FLOP and minimum HBM bytes are recorded with its kind.  At most
 * max_launches launches are recorded (later ones are not).  Query after the
 * stream has been synchronised.  Kinds are numbered 0 .. lora_profile_kinds()-1.
 *   lora_profile_begin: LORA_ERR_SHAPE if max_launches < 1; LORA_ERR_DEVICE if
 *     event creation fails.
 *   lora_profile_query: totals over the recorded launches of `kind`:
 *     summed event time in ms, launch count, summed FLOP, summed bytes.
 *   lora_profile_only: from now on record only launches of `kind` (-1: every
 *     kind, the state at load); the others run without events, so a timed run
 *     can bracket one kernel kind without slowing the rest.  LORA_ERR_SHAPE if
 *     kind is outside [-1, lora_profile_kinds()).  No HIP call.
 */
int lora_profile_begin(int max_launches);
int lora_profile_end(void);
int lora_profile_only(int kind);
int lora_profile_kinds(void);
const char* lora_profile_kind_name(int kind);
int lora_profile_query(int kind, double* total_ms, int* count, double* total_flop, double* total_bytes);

/*
 * MFMA rate probe (measurement hook, not part of the layer's arithmetic): an
 * asynchronous launch of `blocks` workgroups of 4 waves (one per SIMD), each
 * wave running `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
 * register operands, so the work is blocks * 4 * iters * 8 * 32768 FLOP; the
 * caller times it on `stream`.  This is the dense bf16 rate the chip sustains
 * under its own power and clock limits, next to the published peak.  out:
 * device fp32 [blocks * 256].  LORA_ERR_SHAPE if iters or blocks < 1.
 */
int lora_mfma_rate(int iters, int blocks, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LORA_LINEAR_H */
