"""Oracle for the fused LoRA linear layer (float64, numpy, CPU).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the HIP library.  It shares no code
with the GPU path.

Every function is the plain definition written out; numpy's float64 matmul is
the only library primitive used.  Page citations name the page title and the
section or equation on it:

  [P1] "UnSloth加速微调体验：在LoRA基础上再提速3倍的秘密"
       - section 算子融合 (operator fusion), equation y = Wx + ΔWx = Wx + BAx
         with B ∈ R^{d×r}, A ∈ R^{r×k};
       - section 反向传播优化 (backward optimisation): gradients of A and B,
         intermediates Ax, BAx recomputed rather than stored;
       - section RoPE缓存集成 (RoPE cache): cos/sin as one contiguous cache,
         the rotation applied inside the q/k projection.
  [P2] "微调太慢？试试Unsloth：实测训练速度翻倍，显存占用减半", section 5.1:
       for inference the LoRA weights are merged into the main weight.
  [P2] section 3.3, configuration E: LoRA dropout 0.05 (a weak effect on the
       loss); [P4] section 2.2: get_peft_model(..., lora_dropout=0.1).
  [P3] "Unsloth教程：本地微调大模型速度提升数倍，显存节省60%", section
       显存优化策略, 4-bit QLoRA paragraph: base weight in NormalFloat4, only
       the LoRA adapters train (no dW).
  [P4] "Unsloth框架：高效LLM微调与LoRA优化实践", section 3.1: the graph
       rewriter merges adjacent linear layers with their activation function.
  [P5] "Unsloth自动化优化：无需手动调参的实现原理", section 3.2: the fused
       kernel is equivalent to A@B added to the original weight; section 5:
       NF4 is the default 4-bit format, and fusion changes the order of the
       gradient arithmetic, so results are equal up to rounding only;
       section 1: the layer types it recognises include SwiGLU.

Readings where the pages are silent or garbled (each also listed in the design
notes):
  * scale s = alpha / r multiplies the low-rank branch ([P1] prints no scale);
  * the gradient formulas printed in [P1] 反向传播优化 are dimensionally
    inconsistent; the chain rule of Y = X W^T + s (X A^T) B^T gives
    dX = G W + s (G B) A,  dB = s G^T (X A^T),  dA = s (G B)^T X;
  * RoPE pairs element i with i + D/2 inside each head of width D
    ("rotate-half"), angle pos * theta^(-2i/D), theta = 5e5;
  * NF4: blocks of 64 consecutive elements of row-major W [d_out, d_in];
    element 2j in the high nibble of byte j; value = bf16(f32(table[c] * absmax));
  * LoRA dropout (a rate on the pages, not a definition): inverted dropout on
    the adapter's input only, D(x) = x * keep / (1 - p) with keep ~ Bernoulli(1 - p)
    per element of X; the base path W x sees x unchanged.  The keep mask is an
    input (bit-packed, bit b of byte [i, j] keeps element (i, 8 j + b)), or is
    drawn from a Philox4x32-10 stream keyed by a seed (dropout_mask_philox);
  * SwiGLU (named, not defined, on the pages): the Llama MLP's gated unit
    h = silu(g) * u elementwise, g and u the gate and up projections of the
    same x, silu(z) = z / (1 + e^-z).

Layout: row-major, one token per row.  X [M, d_in], W [d_out, d_in],
A [r, d_in], B [d_out, r], Y and dY [M, d_out].
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor: widen exactly
        import torch

        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# forward, backward ([P1] 算子融合, 反向传播优化)
# ---------------------------------------------------------------------------

def lora_panel(X, A) -> np.ndarray:
    """P = X A^T [M, r]: the rank-r projection A x of every token ([P1] 算子融合)."""
    return _f64(X) @ _f64(A).T


def lora_forward(X, W, A, B, s: float) -> np.ndarray:
    """Y = X W^T + s (X A^T) B^T: per token y = W x + s B (A x) ([P1] 算子融合, eq. y = Wx + BAx)."""
    X, W, A, B = map(_f64, (X, W, A, B))
    P = X @ A.T
    return X @ W.T + s * (P @ B.T)


def lora_grad_x(W, A, B, s: float, G) -> np.ndarray:
    """dX = G W + s (G B) A: the input gradient (row-wise in G)."""
    W, A, B, G = map(_f64, (W, A, B, G))
    return G @ W + s * ((G @ B) @ A)


def lora_grad_ab(X, A, B, s: float, G):
    """(dA, dB) = (s (G B)^T X, s G^T (X A^T)), with X A^T recomputed ([P1] 反向传播优化)."""
    X, A, B, G = map(_f64, (X, A, B, G))
    P = X @ A.T
    Q = G @ B
    return s * (Q.T @ X), s * (G.T @ P)


def lora_backward(X, W, A, B, s: float, G):
    """(dX, dA, dB) for upstream gradient G = dL/dY; no dW (W is frozen, [P3] QLoRA paragraph).

    Chain rule of Y = X W^T + s P B^T with P = X A^T (recomputed, [P1] 反向传播优化):
      dX = G W + s (G B) A
      dB = s G^T P
      dA = s (G B)^T X
    """
    dX = lora_grad_x(W, A, B, s, G)
    dA, dB = lora_grad_ab(X, A, B, s, G)
    return dX, dA, dB


def merged_weight(W, A, B, s: float) -> np.ndarray:
    """W' = W + s B A: the LoRA branch folded into the base weight ([P2] 5.1, [P5] 3.2)."""
    return _f64(W) + s * (_f64(B) @ _f64(A))


# ---------------------------------------------------------------------------
# RoPE epilogue ([P1] RoPE缓存集成)
# ---------------------------------------------------------------------------

def rope_angles(pos, head_dim: int, theta: float) -> np.ndarray:
    """Angle pos[t] * theta^(-2i/D) for t < M, i < D/2, in float64 ([M, D/2])."""
    pos = np.asarray(pos, dtype=np.float64)
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-(2.0 * i) / head_dim)
    return pos[:, None] * inv_freq[None, :]


def rope_rotate(Z, pos, head_dim: int, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate each pair (i, i + D/2) of every width-D head of each row by +angle
    (or by -angle when inverse=True, which is the transpose of the rotation)."""
    Z = _f64(Z)
    M, d = Z.shape
    if d % head_dim:
        raise ValueError("d_out must be a multiple of head_dim")
    half = head_dim // 2
    a = rope_angles(pos, head_dim, theta)
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    if inverse:
        s = -s
    Zh = Z.reshape(M, d // head_dim, head_dim)
    z1, z2 = Zh[..., :half], Zh[..., half:]
    out = np.concatenate([z1 * c - z2 * s, z2 * c + z1 * s], axis=-1)
    return out.reshape(M, d)


def qk_rope_forward(X, W, A, B, s, pos, head_dim=128, theta=500000.0) -> np.ndarray:
    """Y = RoPE(X W^T + s (X A^T) B^T): q/k projection with the rotation applied to its output."""
    return rope_rotate(lora_forward(X, W, A, B, s), pos, head_dim, theta)


def qk_rope_backward(X, W, A, B, s, pos, dY, head_dim=128, theta=500000.0):
    """Backward of qk_rope_forward: G = R(-angle) dY, then the LoRA backward with G."""
    G = rope_rotate(dY, pos, head_dim, theta, inverse=True)
    return lora_backward(X, W, A, B, s, G)


# ---------------------------------------------------------------------------
# rounding and NF4 ([P3] QLoRA paragraph, [P5] section 5)
# ---------------------------------------------------------------------------

def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest fp32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round fp32-representable values to bfloat16, nearest with ties to even.

    bfloat16 keeps the top 16 bits of an fp32 word; the dropped low 16 bits
    decide the rounding.  NaN stays NaN.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    hi = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((hi & 1) == 1))
    hi = hi + up.astype(np.uint64)
    out = (hi << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def nf4_unpack(codes, n_elems: int) -> np.ndarray:
    """4-bit codes of n_elems elements; element 2j is the high nibble of byte j."""
    b = np.asarray(codes.cpu() if hasattr(codes, "cpu") else codes, dtype=np.uint8)
    out = np.empty(n_elems, dtype=np.int64)
    out[0::2] = b[: n_elems // 2] >> 4
    out[1::2] = b[: n_elems // 2] & 0xF
    return out


def nf4_dequant(codes, absmax, table, d_out: int, d_in: int, blocksize: int = 64) -> np.ndarray:
    """W [d_out, d_in] from NF4 codes: W[e] = bf16(f32(table[c_e] * absmax[e // blocksize])).

    The float64 product of two fp32 values is exact, so rounding it once to
    fp32 equals an fp32 multiply with round-to-nearest-even.
    """
    n = d_out * d_in
    c = nf4_unpack(codes, n)
    tab = _f64(table)
    am = _f64(absmax)
    e = np.arange(n)
    w = round_bf16(round_f32(tab[c] * am[e // blocksize]))
    return w.reshape(d_out, d_in)


def nf4_encode(W, table, blocksize: int = 64):
    """Quantise W [d_out, d_in] to (packed codes uint8, absmax fp32); used by tests.

    absmax = max |w| of each block (fp32); each w / absmax goes to the nearest
    table value, ties to the lower code; an all-zero block gets absmax 0 and
    the code of 0.0.
    """
    W = _f64(W).reshape(-1)
    tab = _f64(table)
    n = W.size
    blocks = W.reshape(-1, blocksize)
    am = round_f32(np.abs(blocks).max(axis=1))
    safe = np.where(am > 0, am, 1.0)
    norm = blocks / safe[:, None]
    dist = np.abs(norm[..., None] - tab[None, None, :])
    codes = np.argmin(dist, axis=-1)  # first minimum = lower code on ties
    zero_code = int(np.argmin(np.abs(tab)))
    codes[am == 0] = zero_code
    codes = codes.reshape(n)
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    return packed, am.astype(np.float32)


# ---------------------------------------------------------------------------
# LoRA dropout on the adapter's input ([P2] 3.3, [P4] 2.2)
# ---------------------------------------------------------------------------

def dropout_keep(bits, M: int, d_in: int) -> np.ndarray:
    """bool [M, d_in] keep mask from the packed bytes [M, d_in / 8]: bit b
    (least significant first) of byte (i, j) is element (i, 8 j + b)."""
    b = np.asarray(bits, dtype=np.uint8).reshape(M, d_in // 8)
    out = np.zeros((M, d_in), dtype=bool)
    for bit in range(8):
        out[:, bit::8] = (b >> bit) & 1
    return out


# Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
# random numbers: as easy as 1, 2, 3", SC'11, section 4): a counter-based
# generator whose output block is a keyed bijection of a 128-bit counter.  The
# dropout mask is drawn from it so that the backward regenerates the forward's
# mask from (seed, offset) instead of storing it.

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57  # round multipliers
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85  # key schedule increments (Weyl)
_U32 = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One output block: four 32-bit words from four counter words and two key
    words, ten rounds.  A round multiplies words 0 and 2 by the two constants
    (full 64-bit products), then the new words are (hi of product 1) xor word 1
    xor key 0, (lo of product 1), (hi of product 0) xor word 3 xor key 1,
    (lo of product 0); the key advances by the increments between rounds."""
    x = [int(c) & _U32 for c in counter]
    k0, k1 = int(key[0]) & _U32, int(key[1]) & _U32
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + PHILOX_W0) & _U32, (k1 + PHILOX_W1) & _U32
        p0, p1 = PHILOX_M0 * x[0], PHILOX_M1 * x[2]
        x = [(p1 >> 32) ^ x[1] ^ k0, p1 & _U32, (p0 >> 32) ^ x[3] ^ k1, p0 & _U32]
    return x


def dropout_threshold(p: float) -> int:
    """A word w keeps its element iff w >= floor(p 2^32), with p taken as the
    float32 the C interface receives (so P(keep) = 1 - p up to 2^-32)."""
    return int(np.floor(float(np.float32(p)) * 4294967296.0))


def dropout_mask_philox(n: int, p: float, seed: int, offset: int) -> np.ndarray:
    """bool keep mask of n elements (the row-major flattening of X [M, d_in]).
    Element e takes word e mod 4 of the block whose counter is
    (lo32(e // 4), hi32(e // 4), lo32(offset), hi32(offset)) under the key
    (lo32(seed), hi32(seed)).  Plain loop over blocks: small n only."""
    thr = dropout_threshold(p)
    key = (seed & _U32, (seed >> 32) & _U32)
    keep = np.zeros(n, dtype=bool)
    for g in range((n + 3) // 4):
        w = philox4x32_10((g & _U32, g >> 32, offset & _U32, (offset >> 32) & _U32), key)
        for j in range(4):
            if 4 * g + j < n:
                keep[4 * g + j] = w[j] >= thr
    return keep


def dropout_mask_philox_np(n: int, p: float, seed: int, offset: int) -> np.ndarray:
    """The same mask as dropout_mask_philox, the ten rounds evaluated on every
    block at once in uint64 numpy arithmetic (for sizes where the loop is slow)."""
    thr = dropout_threshold(p)
    nb = (n + 3) // 4
    g = np.arange(nb, dtype=np.uint64)
    m32 = np.uint64(_U32)
    x0, x1 = g & m32, g >> np.uint64(32)
    x2 = np.full(nb, offset & _U32, dtype=np.uint64)
    x3 = np.full(nb, (offset >> 32) & _U32, dtype=np.uint64)
    k0, k1 = seed & _U32, (seed >> 32) & _U32
    for rnd in range(10):
        if rnd:
            k0, k1 = (k0 + PHILOX_W0) & _U32, (k1 + PHILOX_W1) & _U32
        p0, p1 = x0 * np.uint64(PHILOX_M0), x2 * np.uint64(PHILOX_M1)
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ np.uint64(k0), p1 & m32,
                          (p0 >> np.uint64(32)) ^ x3 ^ np.uint64(k1), p0 & m32)
    words = np.stack([x0, x1, x2, x3], axis=1).reshape(-1)[:n]
    return words >= np.uint64(thr)


def dropout_pack(keep) -> np.ndarray:
    """Packed bytes of a bool mask with 8 | n: bit b of byte j is element 8 j + b."""
    k = np.asarray(keep, dtype=bool).reshape(-1, 8).astype(np.uint8)
    return (k << np.arange(8, dtype=np.uint8)).sum(axis=1).astype(np.uint8)


def lora_dropout_forward(X, W, A, B, s: float, p: float, keep) -> np.ndarray:
    """Y = X W^T + s (D A^T) B^T with D = X * keep / (1 - p)."""
    X, W, A, B = map(_f64, (X, W, A, B))
    D = X * np.asarray(keep, dtype=np.float64) / (1.0 - p)
    return X @ W.T + s * ((D @ A.T) @ B.T)


def lora_dropout_backward(X, W, A, B, s: float, p: float, keep, G):
    """(dX, dA, dB) of lora_dropout_forward for upstream G:
      dX = G W + s ((G B) A) * keep / (1 - p)   (the adapter's path passes the mask)
      dA = s (G B)^T D,  dB = s G^T (D A^T)."""
    X, W, A, B, G = map(_f64, (X, W, A, B, G))
    k = np.asarray(keep, dtype=np.float64) / (1.0 - p)
    D = X * k
    Q = G @ B
    return G @ W + s * (Q @ A) * k, s * (Q.T @ D), s * (G.T @ (D @ A.T))


# ---------------------------------------------------------------------------
# SwiGLU on the gate / up pair ([P4] 3.1, [P5] section 1)
# ---------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu_forward(X, Wg, Ag, Bg, sg, Wu, Au, Bu, su):
    """(H, G, U): G and U the two LoRA projections of X, H = silu(G) * U."""
    G = lora_forward(X, Wg, Ag, Bg, sg)
    U = lora_forward(X, Wu, Au, Bu, su)
    return silu(G) * U, G, U


def swiglu_grad(dH, G, U):
    """(dG, dU) of H = silu(G) * U: dU = dH silu(G), dG = dH U silu'(G) with
    silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    dH, G, U = map(_f64, (dH, G, U))
    sg = 1.0 / (1.0 + np.exp(-G))
    return dH * U * sg * (1.0 + G * (1.0 - sg)), dH * G * sg


def swiglu_backward(X, Wg, Ag, Bg, sg, Wu, Au, Bu, su, dH, G=None, U=None):
    """(dX, dAg, dBg, dAu, dBu) of H = silu(G) U: the two LoRA backwards with
    upstream gradients dG and dU, input gradients summed.  G and U default to
    the exact forward values."""
    if G is None or U is None:
        _, G, U = swiglu_forward(X, Wg, Ag, Bg, sg, Wu, Au, Bu, su)
    dG, dU = swiglu_grad(dH, G, U)
    dXg, dAg, dBg = lora_backward(X, Wg, Ag, Bg, sg, dG)
    dXu, dAu, dBu = lora_backward(X, Wu, Au, Bu, su, dU)
    return dXg + dXu, dAg, dBg, dAu, dBu


def nf4_lora_forward(X, codes, absmax, table, A, B, s, d_out, d_in, blocksize=64):
    """Forward with the NF4-dequantised frozen base weight."""
    W = nf4_dequant(codes, absmax, table, d_out, d_in, blocksize)
    return lora_forward(X, W, A, B, s)


def nf4_lora_backward(X, codes, absmax, table, A, B, s, dY, d_out, d_in, blocksize=64):
    """Backward with the NF4-dequantised frozen base weight; never forms dW."""
    W = nf4_dequant(codes, absmax, table, d_out, d_in, blocksize)
    return lora_backward(X, W, A, B, s, dY)


# ---------------------------------------------------------------------------
# comparison
# ---------------------------------------------------------------------------

def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero)."""
    got, ref = _f64(got), _f64(ref)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
