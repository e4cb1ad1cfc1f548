// api.cpp - the C ABI declared in include/lora_linear.h: argument validation
// (before any HIP call), workspace layout, tile choice and the sequence of
// launches for each entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/lora_linear.h"
#include "few_args.h"
#include "launch.h"
#include "skinny.h"

using namespace lora;

namespace {

constexpr int64_t kMaxRank = 256;
constexpr int64_t kMaxDim = int64_t(1) << 31;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == LORA_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// device check: gfx950 only, checked once per device
// ---------------------------------------------------------------------------
std::atomic<int> g_dev_state[64];  // 0 unknown, 1 ok, 2 bad
std::mutex g_dev_mu;

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LORA_ERR_DEVICE;
  int s = g_dev_state[dev].load(std::memory_order_acquire);
  if (s == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LORA_ERR_DEVICE;
      s = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      g_dev_state[dev].store(s, std::memory_order_release);
    }
  }
  return s == 1 ? LORA_OK : LORA_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// few-token plan (few.h): two launches per direction for 1 <= M <= 128
// ---------------------------------------------------------------------------
struct FewPlan {
  bool ok = false;
  int MB = 0, Mp = 0, Sp = 0, Kp = 0, pg = 1, Sq = 0, Kq = 0, n_tiles = 0, nkt = 0, T = 0, nblk = 0;
  bool fold = false;  // backward in two launches: the W stream sums the panels
  size_t pp = 0, qp = 0, cp = 0, cnt = 0, g = 0, ps = 0, qs = 0, total = 0;
};

// bf16, 1 <= M <= 128, r a multiple of 8 up to 64, d_in and d_out multiples
// of 64 (d_in of 128 in the backward, whole column tiles, and with NF4; d_out
// of 128 with RoPE),
// every byte offset of an operand below 2^30.  Launch 2: the column tiles (128
// of d_out forward, of d_in backward) times their 64-wide contraction stages,
// cut into few::GRID equal contiguous ranges, one block each (at most as
// many tiles as blocks, so a range covers one tile or two).  P in at most 16
// chunks of d_in (the forward's finishing blocks sum them with every load in
// flight); Q in chunks of d_out of whole 128-row heads, about 32 of them but
// at most 512 rows each, one head per wave (measured: a wave with two heads
// in turn, on d_out = 27392, cost 3-7 us; fewer blocks with every wave busy,
// on d_out = 4096, cost 3 us more than 32 blocks with one); summed with P
// between the backward's launches, 32 slabs' loads in flight.
FewPlan few_plan(bool bwd, bool nf4, bool rope, int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
  FewPlan F;
  if (M < 1 || M > 16 * few::MAXMB || r % 8 || r > few::MAXR || d_in % 64 || d_out % 64) return F;
  if ((rope && d_out % 128) || ((bwd || nf4) && d_in % 128)) return F;
  const int64_t lim = int64_t(1) << 30;
  if (d_in * d_out * 2 >= lim || M * std::max(d_in, d_out) * 2 >= lim) return F;
  // taken where it measured faster on MI355X than the skinny and split-GEMM
  // paths: the backward; the forward with NF4; the forward with a bf16 W up
  // to 64 tokens wherever the one-launch skinny kernel (one block per 16
  // output columns, each forming the whole rank panel) underfills the chip or
  // re-reads much of A: RoPE (4 skinny blocks per head), more than 16 tokens,
  // a rank above 16, or W of 2^25 elements or more.  Small plain problems keep
  // skinny's single launch (4096 x 4096, r = 16, 1 token: 16.6 us against 20.7).
  if (!bwd && !nf4 && !(M <= 64 && (rope || M > 16 || r > 16 || d_in * d_out >= (int64_t(1) << 25)))) return F;
  F.MB = M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 64 ? 4 : 8));
  F.Mp = 16 * F.MB;
  const int64_t ncols = bwd ? d_in : d_out, K = bwd ? d_out : d_in;
  F.n_tiles = (int)cdiv(ncols, few::BN);
  if (F.n_tiles > few::GRID) return F;
  F.nkt = (int)(K / (nf4 && !bwd ? 2 * few::BK : few::BK));  // the NF4 forward's stages are 128 deep
  F.T = F.n_tiles * F.nkt;
  F.nblk = std::min(few::GRID, F.T);
  // the backward's W stream sums the panel partials itself (no launch
  // between) when the panels are small, Mp r8 <= 1024: each block then loads
  // at most 64 KB of partials, 8 chunks of each panel, from L2.  Launch 1 then
  // has 8 chunks per panel, each block a chunk of the contraction times
  // (Mp + r8): taken while those stay within 64K elements (128 KB)
  auto chunk8 = [](int64_t K) { return std::max<int64_t>(128, rup(cdiv(K, 8), 128)); };
  F.fold = bwd && F.Mp * r <= 1024 && std::max(chunk8(d_in), chunk8(d_out)) * (F.Mp + r) <= 65536;
  // the forward's stream blocks each load every P slab for their items (16
  // tokens x 4 columns each, ahead of their DMAs): at most 16 loads a thread,
  // so fewer slabs as the tokens grow, and launch 1 then takes each slab in
  // 16-row groups of tokens, a block each
  const int64_t fwd_slabs = 16 / cdiv(F.Mp * 16, nf4 ? few::NT4 : few::NT);
  F.Kp = (int)std::max<int64_t>(128, rup(cdiv(d_in, bwd ? (F.fold ? 8 : 16) : fwd_slabs), 128));
  F.Sp = (int)cdiv(d_in, F.Kp);
  F.pg = bwd ? 1 : F.MB;
  if (bwd) {
    F.Kq = (int)(F.fold ? std::max<int64_t>(128, rup(cdiv(d_out, 8), 128))
                        : std::min<int64_t>(512, std::max<int64_t>(128, rup(cdiv(d_out, 32), 128))));
    F.Sq = (int)cdiv(d_out, F.Kq);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  F.pp = take(size_t(F.Sp) * F.Mp * r * 4);
  F.qp = take(size_t(F.Sq) * F.Mp * r * 4);
  F.cp = take(size_t(F.nblk + F.n_tiles - 1) * F.Mp * few::BN * 4);
  F.cnt = take(size_t(F.n_tiles) * 4);
  if (bwd && rope) F.g = take(size_t(M) * d_out * 2);
  if (bwd) {
    F.ps = take(size_t(F.Mp) * r * 2);
    F.qs = take(size_t(F.Mp) * r * 2);
  }
  F.total = off;
  F.ok = true;
  return F;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct Layout {
  int64_t r8 = 0, M8 = 0;
  size_t bpad = 0, bt = 0, p = 0, g = 0, pt = 0, qs = 0, qt = 0, part = 0, ppart = 0, wdq = 0, spart = 0, xm = 0,
         keep = 0, total = 0;
  int splits_main = 1;  // contraction splits of the Y (forward) or dX (backward) GEMM
  int64_t ksplit_main = 0;
  bool dequant = false;  // NF4: W dequantised once into wdq, then the bf16 GEMMs
  bool nf4_whole = false;  // NF4 forward: whole-tile GEMM expanding W in its load stage
  // dX on whole tiles: W^T [d_in, d_out] and A^T [d_in, r8] in the workspace,
  // and the input gradient runs through the forward-orientation kernel
  bool dx_nt = false;
  size_t wt = 0, at = 0;
  int splits_dA = 1, splits_dB = 1;
  int64_t ksplit_dA = 0, ksplit_dB = 0;
  int splits_p = 1, splits_q = 1;  // bf16 rank-r panels: P = X A^T, Q = G B
  int64_t ksplit_p = 0, ksplit_q = 0;
  size_t partb = 0;  // bf16: the dB partials, apart from dA's so one launch sums both
  FewPlan few;       // few tokens: the two-launch path (its regions from offset 0)
};

// 256x256 tiles when they still give at least one tile per CU, else 128x128.
bool use_big(int64_t M, int64_t N) { return cdiv(M, 256) * cdiv(N, 256) >= 256; }

// Split of the contraction of a bf16 rank-r panel: up to 128 columns, 256-row
// tiles with every column (panel_dma_kernel) and about one block per CU;
// wider panels, 256 x 64 tiles and about 1.5 per CU.  At most 32 splits, each
// a multiple of 64 and at least 8 stages long (4 when a few tokens leave
// fewer than 16 tiles).
void panel_split(int64_t M, int64_t K, int64_t r8, int* splits, int64_t* ksplit) {
  // up to 256 columns: one 128-row tile holds every column and one block per
  // CU runs (up to 160 KB of LDS each); wider panels take 64-column tiles
  int64_t tiles = r8 <= 256 ? cdiv(M, PANEL_BM) : cdiv(M, 256) * cdiv(r8, 64);
  if (tiles < 1) tiles = 1;
  int64_t s = cdiv(r8 <= 256 ? 256 : 384, tiles);
  int64_t smax = tiles < 16 ? K / 256 : K / 512;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  const int64_t ks = rup(cdiv(K, s), 64);
  *ksplit = ks;
  *splits = (int)cdiv(K, ks);
}

// Split of the token contraction for dA / dB ([rows, N] outputs), each split
// a multiple of 64 tokens and at least 256 long.  bf16 (dma) up to 128 rows:
// splitnn_dma_kernel, every row in a 256-column tile: up to 64 rows and 32+
// tiles two blocks per CU (512 slots), else one (256); wider or fp32: 64 x 256
// tiles, two blocks per CU.  The split count rounds down so that every block
// runs in the first round (560 blocks for 512 slots measured 25 % slower than
// 504).  More splits mean more fp32 partials to sum: with 16 tiles the
// two-per-CU form's 32 splits cost more in the sum than they gain.
void choose_split(int64_t M, int64_t rows, int64_t N, bool dma, int* splits, int64_t* ksplit) {
  const bool one = dma && rows <= 128;
  const int64_t tiles = one ? cdiv(N, 256) : cdiv(rows, 64) * cdiv(N, 256);
  const int64_t slots = one && (rows > 64 || tiles < 32) ? 256 : 512;
  int64_t s = slots / tiles;
  const int64_t smax = cdiv(M, 256);
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  int64_t ks = rup(cdiv(M, s), 64);
  if (ks < 64) ks = 64;
  *ksplit = ks;
  *splits = (int)cdiv(M, ks);
  if (*splits < 1) *splits = 1;
}

// Contraction split of the layer's Y or dX GEMM [M, N] over K when its
// 128x128 tiles cannot give every CU one (few tokens): about two workgroups
// per CU, at most 16 splits, each a multiple of 64 and at least 256 long.
// bf16 only; 1 = no split.
void main_split(int64_t M, int64_t N, int64_t K, int* splits, int64_t* ksplit) {
  *splits = 1;
  *ksplit = K;
  const int64_t tiles = cdiv(M, 128) * cdiv(N, 128);
  if (M == 0 || tiles >= 256) return;
  int64_t s = cdiv(512, tiles);
  if (s > K / 256) s = K / 256;
  if (s > 16) s = 16;
  if (s < 2) return;
  const int64_t ks = rup(cdiv(K, s), 64);
  *ksplit = ks;
  *splits = (int)cdiv(K, ks);
}

// NF4 forward from LORA_NF4_DEQUANT_MIN_TOKENS tokens on: W expanded in the
// whole-tile GEMM's load stage, or dequantised once per call into the
// workspace for the bf16 GEMM (lora_set_nf4_fwd_path).  Automatic: the load
// stage only for 128 to 255 whole 256 x 256 tiles.  Measured on MI355X
// (r = 64, Qwen1.5-32B shapes): with 256 tiles or more the dequantised W runs
// the bf16 whole-tile kernel and wins (gate 5120 -> 27392 at 8192 tokens:
// 1.81 against 2.82 ms; the expansion's permutes, products and LDS writes
// slow every stage); below 256 the bf16 path falls back to 128 x 128 tiles
// and the load stage wins down to about 128 tiles (gate at 512 tokens, 214
// tiles: 0.25 against 0.40 ms; down 27392 -> 5120 at 2048, 160 tiles: 1.03
// against 1.34 ms); with fewer tiles its stages wait on the codes' latency
// (80 tiles: 1.01 against 0.76 ms).
std::atomic<int> g_nf4_fwd_path{LORA_NF4_PATH_AUTO};

bool nf4_fwd_whole(int64_t M, int64_t d_in, int64_t d_out) {
  const int mode = g_nf4_fwd_path.load();
  if (mode == LORA_NF4_PATH_DEQUANT) return false;
  const bool fits = M >= LORA_NF4_DEQUANT_MIN_TOKENS && M % 256 == 0 && d_out % 256 == 0 && d_in % 64 == 0 &&
                    whole_ld_fits(d_in);
  if (mode == LORA_NF4_PATH_LOAD_STAGE) return fits;
  const int64_t tiles = (M / 256) * (d_out / 256);
  return fits && tiles >= 128 && tiles < 256;
}

// have_wt: the caller supplies W^T, so the backward needs no room for it.
Layout make_layout(int op, int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, bool have_wt = false) {
  Layout L;
  const size_t eb = elem_bytes(dtype);
  L.r8 = rup(r, 8);
  L.M8 = rup(M, 8);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (op == LORA_OP_MERGE) {
    if (r % 8) L.bpad = take(size_t(d_out) * L.r8 * eb);
    L.total = off;
    return L;
  }
  const bool drop = op == LORA_OP_DROPOUT_FWD || op == LORA_OP_DROPOUT_BWD;
  const bool bwd = op == LORA_OP_BWD || op == LORA_OP_ROPE_BWD || op == LORA_OP_NF4_BWD || op == LORA_OP_DROPOUT_BWD;
  if (op == LORA_OP_NF4_FWD && nf4_fwd_whole(M, d_in, d_out)) {
    L.nf4_whole = true;
  } else if ((op == LORA_OP_NF4_FWD || op == LORA_OP_NF4_BWD) && M >= LORA_NF4_DEQUANT_MIN_TOKENS) {
    L.dequant = true;
    L.wdq = take(size_t(d_out) * d_in * 2);
  }
  if (r % 8) L.bpad = take(size_t(d_out) * L.r8 * eb);
  if (eb == 2) {
    panel_split(M, d_in, L.r8, &L.splits_p, &L.ksplit_p);
    int sp = L.splits_p;
    if (bwd) {
      panel_split(M, d_out, L.r8, &L.splits_q, &L.ksplit_q);
      if (L.splits_q > sp) sp = L.splits_q;
    }
    L.ppart = take(size_t(sp) * L.M8 * L.r8 * 4);
  }
  if (eb == 2) {
    if (bwd)
      main_split(M, d_in, d_out, &L.splits_main, &L.ksplit_main);
    else
      main_split(M, d_out, d_in, &L.splits_main, &L.ksplit_main);
  }
  const size_t sp = L.splits_main > 1 ? size_t(L.splits_main) * M * (bwd ? d_in : d_out) * 4 : 0;
  const bool nf4op = op == LORA_OP_NF4_BWD;
  if (bwd && eb == 2 && L.splits_main == 1 && (!nf4op || L.dequant) && M % 256 == 0 && d_in % 256 == 0 &&
      d_out % 64 == 0 && use_big(M, d_in)) {
    L.dx_nt = true;
    if (!have_wt) L.wt = take(size_t(d_in) * d_out * 2);
    L.at = take(size_t(d_in) * L.r8 * 2);
  }
  if (!bwd) {
    L.p = take(size_t(M) * L.r8 * eb);
    if (sp) L.spart = take(sp);
  } else {
    if (op == LORA_OP_ROPE_BWD) L.g = take(size_t(M) * d_out * eb);
    if (eb == 2) L.bt = take(size_t(L.r8) * d_out * eb);
    L.pt = take(size_t(L.r8) * L.M8 * eb);
    L.qs = take(size_t(L.M8) * L.r8 * eb);
    L.qt = take(size_t(L.r8) * L.M8 * eb);
    choose_split(M, L.r8, d_in, eb == 2, &L.splits_dA, &L.ksplit_dA);
    choose_split(M, L.r8, d_out, eb == 2, &L.splits_dB, &L.ksplit_dB);
    size_t pa = size_t(L.splits_dA) * L.r8 * d_in * 4;
    size_t pb = size_t(L.splits_dB) * L.r8 * d_out * 4;
    if (sp > pa) pa = sp;  // the dX partials are reduced before dB and dA start
    if (eb == 2) {
      L.part = take(pa);
      L.partb = take(pb);
    } else {
      L.part = take(pa > pb ? pa : pb);
    }
    L.spart = L.part;
  }
  if (drop) L.xm = take(size_t(M) * d_in * eb);
  // the backward's keep bits when it draws them itself (Philox entry point)
  if (op == LORA_OP_DROPOUT_BWD) L.keep = take(size_t(M) * d_in / 8);
  L.total = off;
  if (eb == 2 && !drop) {
    const bool rope = op == LORA_OP_ROPE_FWD || op == LORA_OP_ROPE_BWD;
    const bool nf4 = op == LORA_OP_NF4_FWD || op == LORA_OP_NF4_BWD;
    L.few = few_plan(bwd, nf4, rope, M, d_in, d_out, r);
    if (L.few.ok && L.few.total > L.total) L.total = L.few.total;
  }
  return L;
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
int check_sizes(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
  if (M < 0 || M >= kMaxDim) return LORA_ERR_SHAPE;
  if (d_in < 8 || d_out < 8 || d_in % 8 || d_out % 8 || d_in >= kMaxDim || d_out >= kMaxDim) return LORA_ERR_SHAPE;
  if (r < 1 || r > kMaxRank) return LORA_ERR_SHAPE;
  return LORA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (!q) return LORA_ERR_NULL;
  for (const void* q : ps)
    if (!aligned16(q)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

int check_ws(const Layout& L, const void* ws, size_t ws_bytes) {
  if (L.total == 0) return LORA_OK;
  if (!ws || ws_bytes < L.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

#define TRY(x)                       \
  do {                               \
    int _rc = (x);                   \
    if (_rc != LORA_OK) return _rc;  \
  } while (0)

#define HIPTRY(x)                                  \
  do {                                             \
    if ((x) != hipSuccess) return LORA_ERR_DEVICE; \
  } while (0)

// ---------------------------------------------------------------------------
// launch profiling: HIP events around every launch while enabled
// ---------------------------------------------------------------------------
enum ProfKind : int {
  K_PAD = G_KIND_COUNT,
  K_ROPE_INV,
  K_REDUCE,
  K_FILL,
  K_ROPE_CACHE,
  K_NF4_DEQ,
  K_PANEL,
  K_TRANSPOSE,
  K_FINISH,
  K_SWIGLU,
  K_MASK,
  K_TRANSPOSE_W,
  K_SKINNY,
  K_FEW_PANEL,
  K_FEW_FWD,
  K_FEW_BWD,
  K_TINY,
  K_PROF_COUNT
};

const char* kind_name(int k) {
  static const char* names[] = {
      "gemm_bf16_256x256_nt_store", "gemm_bf16_256x256_nt_rope", "gemm_bf16_128x128_nt_store",
      "gemm_bf16_128x128_nt_rope",  "gemm_bf16_256x256_nn_store", "gemm_bf16_128x128_nn_store",
      "gemm_nf4_256x256_nt_store",  "gemm_nf4_128x128_nt_store",  "gemm_nf4_256x256_nn_store",
      "gemm_nf4_128x128_nn_store",  "split_bf16_nn_partial",      "gemm_f32_64x128_nt_store",
      "gemm_f32_64x128_nt_rope",    "gemm_f32_64x128_nn_store",   "panel_f32_nt_store",
      "panel_f32_nt_store_t",       "panel_f32_nn_both",          "split_f32_nn_partial",
      "panel_bf16_split",           "gemm_bf16_128x128_nt_split", "gemm_bf16_128x128_nn_split",
      "gemm_nf4_128x128_nt_split",  "gemm_nf4_128x128_nn_split",  "merge_bf16_128x128",
      "merge_f32_64x128",           "gemm_bf16_256x256_swiglu",   "dropout_dx_bf16_128x128",
      "dropout_dx_f32_64x128",      "gemm_bf16_256x256_nt_group", "gemm_nf4_256x256_nt_whole",
      "pad_cols",
      "rope_inverse",
      "reduce_splits",              "fill_zero",                  "rope_cache",
      "nf4_dequant",                "panel_reduce",               "transpose_ab",
      "split_finish",               "swiglu_elementwise",
      "dropout_mask_copy",          "transpose_w",                "skinny_fwd",
      "few_panel",                  "few_fwd",                    "few_bwd",
      "tiny_f32"};
  static_assert(sizeof(names) / sizeof(names[0]) == K_PROF_COUNT, "one name per launch kind");
  return (k >= 0 && k < K_PROF_COUNT) ? names[k] : "unknown";
}

struct ProfEntry {
  int kind;
  double flop, bytes;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per slot
  std::vector<ProfEntry> ent;
  size_t n = 0;
  int only = -1;  // record only this kind (-1: all)
} g_prof;

template <class F>
hipError_t timed(int kind, double flop, double bytes, hipStream_t st, F&& f) {
  if (!g_prof.on) return f();
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on || g_prof.n >= g_prof.ent.size() || (g_prof.only >= 0 && kind != g_prof.only)) return f();
  const size_t i = g_prof.n++;
  if (hipEventRecord(g_prof.ev[2 * i], st) != hipSuccess) return hipErrorUnknown;
  hipError_t e = f();
  if (hipEventRecord(g_prof.ev[2 * i + 1], st) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  g_prof.ent[i] = ProfEntry{kind, flop, bytes};
  return e;
}

hipError_t gemm(GemmKind k, const GemmArgs& a, int splits, hipStream_t st, double flop, double bytes) {
  return timed(k, flop, bytes, st, [&] { return launch_gemm(k, a, splits, st); });
}

// ---------------------------------------------------------------------------
// tile choice
// ---------------------------------------------------------------------------

GemmArgs blank() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.alpha = 1.f;
  return a;
}

// bf16 rank-r panel v = alpha * X R^T over a contraction of K: split partials
// (256 x 64 tiles) into part, then the fixed-order reduction into out
// (row-major [rows, ldo]) and/or outt (transposed [r8, ldot]); rows in
// [M, rows) and columns in [r, r8) are zeros.
// Rows of a group's stacked R taken straight from each member's (n = 0: R
// itself is the stacked matrix).
struct PanelSrc {
  int n = 0;
  const void* rs[kPanelSrcMax] = {};
  int beg[kPanelSrcMax] = {};
  int rows[kPanelSrcMax] = {};
};

int panel_bf16(const void* X, int64_t ldx, const void* R, int64_t ldr, int64_t M, int64_t rows, int64_t K, int64_t r,
               int64_t r8, int splits, int64_t ksplit, const ColScale& cs, float* part, uint16_t* out, int64_t ldo,
               uint16_t* outt, int64_t ldot, hipStream_t st, const PanelSrc* src = nullptr) {
  GemmArgs a = blank();
  a.a1 = X; a.lda1 = ldx; a.b1 = R; a.ldb1 = ldr; a.K1 = K;
  if (src) {
    a.n_src = src->n;
    for (int g = 0; g < src->n; ++g) {
      a.rs[g] = src->rs[g];
      a.rs_beg[g] = src->beg[g];
      a.rs_rows[g] = src->rows[g];
    }
  }
  a.m_load = M; a.m_store = rows; a.n_load = r; a.n_store = r8;
  a.k_split = ksplit; a.c = part; a.ldc = r8; a.part_stride = rows * r8;
  const double Md = double(M), kd = double(K), rd = double(r);
  HIPTRY(gemm(G_BF16_PANEL_SPLIT_NT, a, splits, st, 2 * Md * rd * kd,
              (Md * kd + rd * kd) * 2 + 4.0 * splits * rows * r8));
  HIPTRY(timed(K_PANEL, double(splits) * rows * r8, 4.0 * splits * rows * r8 + 2.0 * rows * r8 * ((out ? 1 : 0) + (outt ? 1 : 0)),
               st, [&] { return launch_panel_reduce(part, splits, rows * r8, r8, rows, r8, cs, out, ldo, outt, ldot, st); }));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// forward (shared by the plain, RoPE and NF4 entry points)
// ---------------------------------------------------------------------------
struct Nf4W {
  const uint8_t* codes;
  const float* absmax;
  const float* table;  // host
};

struct Rope {
  const int32_t* pos;
  const float* cosc;
  const float* sinc;
  int64_t max_pos;  // rows of the cache: a position outside [0, max_pos) gives zeros
};

// W [n] bf16 from NF4 codes with the load stage's own routine (one pass).
int dequant_w(const Nf4W& q, int64_t n, void* out, hipStream_t st) {
  HIPTRY(timed(K_NF4_DEQ, 2.0 * n, n / 2.0 + n / 16.0 + 2.0 * n, st, [&] {
    return launch_nf4_dequant(q.codes, q.absmax, n, q.table, static_cast<uint16_t*>(out), st);
  }));
  return LORA_OK;
}

// The few-token path (few.h): launch 1 (panel partials, counters cleared),
// launch 2 (the streamed W product; the last block of each column tile adds
// the rank term and stores).
FewArgs few_args(const FewPlan& F, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                 const void* W, const Nf4W* nf4, const void* A, const void* B, const Rope* rope, char* w) {
  FewArgs a;
  memset(&a, 0, sizeof(a));
  a.M = (int)M; a.Mp = F.Mp; a.d_in = (int)d_in; a.d_out = (int)d_out; a.r8 = (int)r; a.s = scale;
  a.X = static_cast<const uint16_t*>(X);
  a.W = static_cast<const uint16_t*>(W);
  if (nf4) {
    a.codes = nf4->codes; a.absmax = nf4->absmax;
    for (int i = 0; i < 16; ++i) a.nf4_table[i] = nf4->table[i];
    a.W = nullptr;
  }
  a.A = static_cast<const uint16_t*>(A); a.B = static_cast<const uint16_t*>(B);
  if (rope) { a.rope = 1; a.pos = rope->pos; a.cosc = rope->cosc; a.sinc = rope->sinc; a.max_pos = rope->max_pos; }
  a.Pp = reinterpret_cast<float*>(w + F.pp);
  a.Qp = reinterpret_cast<float*>(w + F.qp);
  a.Cp = reinterpret_cast<float*>(w + F.cp);
  a.cnt = reinterpret_cast<int*>(w + F.cnt);
  a.Sp = F.Sp; a.Kp = F.Kp; a.pg = F.pg; a.Sq = F.Sq; a.Kq = F.Kq;
  a.n_tiles = F.n_tiles; a.nkt = F.nkt; a.T = F.T; a.nblk = F.nblk; a.fold = F.fold ? 1 : 0;
  return a;
}

int few_forward(const FewPlan& F, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                const void* W, const Nf4W* nf4, const void* A, const void* B, const Rope* rope, void* Y, char* w,
                hipStream_t st) {
  FewArgs a = few_args(F, M, d_in, d_out, r, scale, X, W, nf4, A, B, rope, w);
  a.Y = static_cast<uint16_t*>(Y);
  const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r);
  const double wb = nf4 ? ko * ki * (0.5 + 1.0 / 16) : 2.0 * ko * ki;
  HIPTRY(timed(K_FEW_PANEL, 2 * Md * rr * ki, (Md + rr) * ki * 2 + 4.0 * F.Sp * F.Mp * rr, st,
               [&] { return launch_few_panel(a, F.MB, st); }));
  HIPTRY(timed(K_FEW_FWD, 2 * Md * ko * (ki + rr), wb + (Md * ki + ko * rr + Md * ko) * 2, st,
               [&] { return launch_few_fwd(a, F.MB, nf4 != nullptr, st); }));
  return LORA_OK;
}

int few_backward(const FewPlan& F, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                 const void* W, const Nf4W* nf4, const void* A, const void* B, const Rope* rope, const void* dY,
                 void* dX, float* dA, float* dB, char* w, hipStream_t st) {
  FewArgs a = few_args(F, M, d_in, d_out, r, scale, X, W, nf4, A, B, rope, w);
  a.dY = static_cast<const uint16_t*>(dY);
  a.G = rope ? reinterpret_cast<uint16_t*>(w + F.g) : nullptr;
  a.dX = static_cast<uint16_t*>(dX);
  a.dA = dA;
  a.dB = dB;
  a.Ps = reinterpret_cast<uint16_t*>(w + F.ps);
  a.Qs = reinterpret_cast<uint16_t*>(w + F.qs);
  const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r);
  const double wb = nf4 ? ko * ki * (0.5 + 1.0 / 16) : 2.0 * ko * ki;
  HIPTRY(timed(K_FEW_PANEL, 2 * Md * rr * (ki + ko), (Md + rr) * (ki + ko) * 2 + 4.0 * (F.Sp + F.Sq) * F.Mp * rr,
               st, [&] { return launch_few_panel(a, F.MB, st); }));
  if (!F.fold)
    HIPTRY(timed(K_FEW_PANEL, 0, 4.0 * (F.Sp + F.Sq) * F.Mp * rr + 4.0 * F.Mp * rr, st,
                 [&] { return launch_few_reduce(a, st); }));
  HIPTRY(timed(K_FEW_BWD, 2 * Md * ki * (ko + rr) + 4 * Md * rr * (ki + ko),
               wb + (Md * ko + Md * ki + rr * ki + ko * rr + Md * ki) * 2 + 4.0 * rr * (ki + ko), st,
               [&] { return launch_few_bwd(a, F.MB, nf4 != nullptr, st); }));
  return LORA_OK;
}

// Pext: when not NULL, the panel s X A^T is already in Pext (row stride
// ldpext, columns r..r8 zero) and is not computed here (group calls).
int forward_impl(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                 const void* W, const Nf4W* nf4, const void* A, const void* B, const Rope* rope, void* Y, void* ws,
                 const Layout& L, hipStream_t st, const void* Pext = nullptr, int64_t ldpext = 0,
                 const void* Xa = nullptr) {
  // Xa: the adapter's input when it differs from X (LoRA dropout)
  const void* Xp = Xa ? Xa : X;
  if (M == 0) return LORA_OK;
  const bool f32 = dtype == LORA_F32;
  const int eb = elem_bytes(dtype);
  char* w = static_cast<char*>(ws);
  if (!f32 && L.few.ok && !Pext && !Xa)
    return few_forward(L.few, M, d_in, d_out, r, scale, X, W, nf4, A, B, rope, Y, w, st);
  // tiny fp32 problems: the whole forward in one launch
  if (f32 && !rope && !Pext && !Xa && tiny_fits(M, d_in, d_out, r)) {
    const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r);
    HIPTRY(timed(K_TINY, 2 * Md * ko * ki + 2 * Md * rr * (ki + ko),
                 4 * (Md * ki + ko * ki + rr * ki + ko * rr + Md * ko), st, [&] {
                   return launch_tiny(false, static_cast<const float*>(X), static_cast<const float*>(W),
                                      static_cast<const float*>(A), static_cast<const float*>(B), nullptr,
                                      static_cast<float*>(Y), nullptr, nullptr, nullptr, nullptr, nullptr, M, d_in,
                                      d_out, r, scale, st);
                 }));
    return LORA_OK;
  }
  // few tokens: panel, GEMM, rank term and epilogue in one launch
  // (bf16 W; an NF4 W keeps the split path's load-stage dequantisation)
  const int smode = rope ? sk::ROPE : sk::PLAIN;
  if (!f32 && !nf4 && !Pext && !Xa && skinny_fits(M, d_in, d_out, r, smode)) {
    SkinnyArgs sa;
    memset(&sa, 0, sizeof(sa));
    sa.X = static_cast<const uint16_t*>(X); sa.ldx = d_in;
    sa.W = static_cast<const uint16_t*>(W); sa.ldw = d_in;
    sa.A = static_cast<const uint16_t*>(A); sa.B = static_cast<const uint16_t*>(B);
    sa.Y = static_cast<uint16_t*>(Y);
    sa.M = (int)M; sa.N = (int)d_out; sa.K = (int)d_in; sa.r = (int)r; sa.s = scale;
    if (rope) { sa.pos = rope->pos; sa.cosc = rope->cosc; sa.sinc = rope->sinc; sa.max_pos = rope->max_pos; }
    const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r);
    HIPTRY(timed(K_SKINNY, 2 * Md * ko * ki + 2 * Md * rr * (ki + ko),
                 (ko * ki + Md * ki + rr * ki + ko * rr + Md * ko) * 2 + (rope ? Md * 64 * 8 : 0), st,
                 [&] { return launch_skinny_fwd(sa, smode, st); }));
    return LORA_OK;
  }
  if (nf4 && L.dequant) {
    TRY(dequant_w(*nf4, d_out * d_in, w + L.wdq, st));
    W = w + L.wdq;
    nf4 = nullptr;
  }
  const void* Bsrc = B;
  if (r % 8) {
    HIPTRY(timed(K_PAD, 0, 2.0 * d_out * L.r8 * eb, st,
                 [&] { return launch_pad_cols(eb, B, w + L.bpad, d_out, r, L.r8, st); }));
    Bsrc = w + L.bpad;
  }
  const void* P = Pext ? Pext : static_cast<const void*>(w + L.p);
  const int64_t ldp = Pext ? ldpext : L.r8;
  const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r), e = double(eb);
  // panel: P = s * X A^T  [M, r8] (columns r..r8 are exact zeros)
  if (Pext) {
    // computed by the caller
  } else if (f32) {
    GemmArgs a = blank();
    a.a1 = Xp; a.lda1 = d_in; a.b1 = A; a.ldb1 = d_in; a.K1 = d_in;
    a.m_load = M; a.m_store = M; a.n_load = r; a.n_store = L.r8;
    a.c = w + L.p; a.ldc = L.r8; a.alpha = scale;
    HIPTRY(gemm(G_F32_PANEL_NT_STORE, a, 1, st, 2 * Md * rr * ki, (Md * ki + rr * ki + Md * L.r8) * e));
  } else {
    TRY(panel_bf16(Xp, d_in, A, d_in, M, M, d_in, r, L.r8, L.splits_p, L.ksplit_p, col_scale(scale),
                   reinterpret_cast<float*>(w + L.ppart), reinterpret_cast<uint16_t*>(w + L.p), L.r8, nullptr, 0, st));
  }
  // main: Y = [X | P] [W | B]^T, optional RoPE epilogue
  GemmArgs a = blank();
  a.a1 = X; a.lda1 = d_in; a.b1 = W; a.ldb1 = d_in; a.K1 = d_in;
  a.a2 = P; a.lda2 = ldp; a.b2 = Bsrc; a.ldb2 = L.r8; a.K2 = r;
  a.m_load = M; a.m_store = M; a.n_load = d_out; a.n_store = d_out;
  a.c = Y; a.ldc = d_out;
  GemmKind k;
  const bool big = use_big(M, d_out);
  if (nf4 && L.nf4_whole) {
    // whole tiles, W expanded from its codes in the load stage
    a.codes = nf4->codes; a.absmax = nf4->absmax; a.codes_ld = d_in / 2; a.blocks_per_row = d_in / 64;
    for (int i = 0; i < 16; ++i) a.nf4_table[i] = nf4->table[i];
    const double flop = 2 * Md * ko * (ki + rr);
    const double bytes = (Md * ki + Md * rr + ko * rr + Md * ko) * e + ko * ki * (0.5 + 1.0 / 16);
    HIPTRY(gemm(G_NF4_WHOLE_NT_STORE, a, 1, st, flop, bytes));
    return LORA_OK;
  }
  if (nf4) {
    a.codes = nf4->codes; a.absmax = nf4->absmax; a.codes_ld = d_in / 2; a.blocks_per_row = d_in / 64;
    for (int i = 0; i < 16; ++i) a.nf4_table[i] = nf4->table[i];
    k = big ? G_NF4_BIG_NT_STORE : G_NF4_MED_NT_STORE;
  } else if (rope) {
    a.pos = rope->pos; a.cosc = rope->cosc; a.sinc = rope->sinc; a.max_pos = rope->max_pos;
    k = f32 ? G_F32_NT_ROPE : (big ? G_BF16_BIG_NT_ROPE : G_BF16_MED_NT_ROPE);
  } else {
    k = f32 ? G_F32_NT_STORE : (big ? G_BF16_BIG_NT_STORE : G_BF16_MED_NT_STORE);
  }
  const double wbytes = nf4 ? ko * ki / 2 + ko * ki / 64 * 4 : ko * ki * e;
  const double flop = 2 * Md * ko * (ki + rr), bytes = (Md * ki + Md * rr + ko * rr + Md * ko) * e + wbytes;
  if (!f32 && L.splits_main > 1) {
    // few tokens: split partials over d_in (the rank-r segment in the last
    // split), then the fixed-order sum with the store / RoPE epilogue
    const int S = L.splits_main;
    float* part = reinterpret_cast<float*>(w + L.spart);
    a.k_split = L.ksplit_main; a.c = part; a.ldc = d_out; a.part_stride = M * d_out;
    HIPTRY(gemm(nf4 ? G_NF4_MED_NT_PARTIAL : G_BF16_MED_NT_PARTIAL, a, S, st, flop,
                bytes - Md * ko * e + 4.0 * S * Md * ko));
    HIPTRY(timed(K_FINISH, double(S) * Md * ko, 4.0 * S * Md * ko + Md * ko * e, st, [&] {
      return launch_split_finish(part, S, M * d_out, M, d_out, static_cast<uint16_t*>(Y), d_out,
                                 rope ? rope->pos : nullptr, rope ? rope->cosc : nullptr,
                                 rope ? rope->sinc : nullptr, rope ? rope->max_pos : 0, st);
    }));
    return LORA_OK;
  }
  HIPTRY(gemm(k, a, 1, st, flop, bytes));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// Rank-r panels of one member of a bf16 group: Pt (= (s X A^T)^T, rows of
// stride M8) is already computed; Q = s G B is written into the group's
// arrays (Qs row stride ldqs, Qt row stride M8); dA is left to the group.
struct PanelSlices {
  const void* Pt;
  void* Qs;
  int64_t ldqs;
  void* Qt;
  // the group's: B^T and A^T made for every member in one launch (NULL:
  // made here), the member's own dB partials, and the batch that sums them
  // with every member's dA after the group's dA contraction
  const void* Bt = nullptr;
  const void* At = nullptr;
  float* partb = nullptr;
  ReduceBatch* red = nullptr;
};

int backward_impl(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                  const void* W, const Nf4W* nf4, const void* A, const void* B, const Rope* rope, const void* dY,
                  void* dX, float* dA, float* dB, void* ws, const Layout& L, hipStream_t st,
                  const PanelSlices* ov = nullptr, const void* Xa = nullptr, const uint8_t* keep = nullptr,
                  const void* Wt_in = nullptr) {
  // LoRA dropout: Xa is the adapter's (masked) input and `keep` the mask that
  // the rank-r term of dX passes through; X itself still feeds the base path
  const void* Xp = Xa ? Xa : X;
  if (M == 0) {
    HIPTRY(timed(K_FILL, 0, 4.0 * r * d_in, st, [&] { return launch_fill_zero(dA, r * d_in, st); }));
    HIPTRY(timed(K_FILL, 0, 4.0 * r * d_out, st, [&] { return launch_fill_zero(dB, d_out * r, st); }));
    return LORA_OK;
  }
  const bool f32 = dtype == LORA_F32;
  const int eb = elem_bytes(dtype);
  char* w = static_cast<char*>(ws);
  if (f32 && !rope && !ov && !Xa && !keep && !nf4 && tiny_fits(M, d_in, d_out, r)) {
    // tiny fp32 problems: the rank rows of every token (into the panel
    // workspace: Pt holds r8 M8 >= M r floats, Qs M8 r8), then dX, dA, dB
    const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r);
    HIPTRY(timed(K_TINY, (dX ? 2 * Md * ki * ko : 0) + 6 * Md * rr * (ki + ko),
                 4 * (Md * ki + ko * ki + rr * ki + ko * rr + Md * ko + (dX ? Md * ki : 0)), st, [&] {
                   return launch_tiny(true, static_cast<const float*>(X), static_cast<const float*>(W),
                                      static_cast<const float*>(A), static_cast<const float*>(B),
                                      static_cast<const float*>(dY), nullptr, static_cast<float*>(dX), dA, dB,
                                      reinterpret_cast<float*>(w + L.pt), reinterpret_cast<float*>(w + L.qs), M,
                                      d_in, d_out, r, scale, st);
                 }));
    return LORA_OK;
  }
  if (!f32 && L.few.ok && dX && !ov && !Xa && !keep)
    return few_backward(L.few, M, d_in, d_out, r, scale, X, W, nf4, A, B, rope, dY, dX, dA, dB, w, st);
  if (nf4 && L.dequant && L.dx_nt && dX && !Wt_in) {
    // the backward reads W only as W^T: dequantise straight into it
    HIPTRY(timed(K_NF4_DEQ, 2.0 * d_out * d_in, (0.5 + 1.0 / 16 + 2.0) * d_out * d_in, st, [&] {
      return launch_nf4_dequant_t(nf4->codes, nf4->absmax, d_out, d_in, nf4->table,
                                  reinterpret_cast<uint16_t*>(w + L.wt), st);
    }));
    Wt_in = w + L.wt;
    nf4 = nullptr;
  } else if (nf4 && L.dequant && dX) {
    TRY(dequant_w(*nf4, d_out * d_in, w + L.wdq, st));
    W = w + L.wdq;
    nf4 = nullptr;
  }
  const void* Bsrc = B;
  if (r % 8) {
    HIPTRY(timed(K_PAD, 0, 2.0 * d_out * L.r8 * eb, st,
                 [&] { return launch_pad_cols(eb, B, w + L.bpad, d_out, r, L.r8, st); }));
    Bsrc = w + L.bpad;
  }
  const double Md = double(M), ki = double(d_in), ko = double(d_out), rr = double(r), e = double(eb);
  const void* G = dY;
  if (rope) {
    HIPTRY(timed(K_ROPE_INV, 3.0 * Md * ko, 2 * Md * ko * e + Md * 64 * 8, st, [&] {
      return launch_rope_inverse(eb, dY, w + L.g, M, d_out, rope->pos, rope->cosc, rope->sinc, rope->max_pos, st);
    }));
    G = w + L.g;
  }
  const void* Pt = ov ? ov->Pt : w + L.pt;
  void* Qs = ov ? ov->Qs : w + L.qs;
  const int64_t ldqs = ov ? ov->ldqs : L.r8;
  void* Qt = ov ? ov->Qt : w + L.qt;
  float* part = reinterpret_cast<float*>(w + L.part);
  bool at_done = false;  // A^T made with B^T (bf16)
  if (f32) {
    // Pt = (s X A^T)^T  [r8, M8]  (recomputed; pads are zeros)
    {
      GemmArgs a = blank();
      a.a1 = Xp; a.lda1 = d_in; a.b1 = A; a.ldb1 = d_in; a.K1 = d_in;
      a.m_load = M; a.m_store = L.M8; a.n_load = r; a.n_store = L.r8;
      a.ct = w + L.pt; a.ldct = L.M8; a.alpha = scale;
      HIPTRY(gemm(G_F32_PANEL_NT_STORE_T, a, 1, st, 2 * Md * rr * ki, (Md * ki + rr * ki + Md * L.r8) * e));
    }
    // Qs = s G B [M8, r8] and Qt = Qs^T [r8, M8]
    {
      GemmArgs a = blank();
      a.a1 = G; a.lda1 = d_out; a.b1 = Bsrc; a.ldb1 = L.r8; a.K1 = d_out;
      a.m_load = M; a.m_store = L.M8; a.n_load = L.r8; a.n_store = L.r8;
      a.c = Qs; a.ldc = L.r8; a.ct = Qt; a.ldct = L.M8; a.alpha = scale;
      HIPTRY(gemm(G_F32_PANEL_NN_BOTH, a, 1, st, 2 * Md * rr * ko, (Md * ko + rr * ko + 2 * Md * L.r8) * e));
    }
  } else {
    // Pt = (s X A^T)^T  [r8, M8], recomputed from X (rows M..M8 and columns r..r8 are zeros)
    float* pp = reinterpret_cast<float*>(w + L.ppart);
    if (!ov)
      TRY(panel_bf16(Xp, d_in, A, d_in, M, L.M8, d_in, r, L.r8, L.splits_p, L.ksplit_p, col_scale(scale), pp,
                     nullptr, 0, reinterpret_cast<uint16_t*>(w + L.pt), L.M8, st));
    // Bt = B^T [r8, d_out] (and A^T for the whole-tile dX below, in the same
    // launch); then Qs = s G B [M8, r8] and Qt = Qs^T [r8, M8]
    const void* Bt = ov ? ov->Bt : nullptr;
    if (!Bt) {
      uint16_t* bt = reinterpret_cast<uint16_t*>(w + L.bt);
      Bt = bt;
      const bool with_at = dX && L.dx_nt && !(ov && ov->At);
      if (r == L.r8) {
        // the tiled transpose (16-byte accesses); r a multiple of 8, no pad rows
        TransposeBatch tb;
        HIPTRY(tb.add(static_cast<const uint16_t*>(B), r, d_out, r, bt, d_out, d_out));
        if (with_at)
          HIPTRY(tb.add(static_cast<const uint16_t*>(A), d_in, r, d_in, reinterpret_cast<uint16_t*>(w + L.at), L.r8,
                        L.r8));
        HIPTRY(timed(K_TRANSPOSE, 0, 4.0 * rr * (d_out + (with_at ? d_in : 0)), st,
                     [&] { return launch_transpose_batch(tb, st); }));
        at_done = with_at;
      } else {
        HIPTRY(timed(K_TRANSPOSE, 0, 2.0 * d_out * (rr + L.r8) * e / 2, st, [&] {
          return launch_transpose_pad(static_cast<const uint16_t*>(B), bt, d_out, r, L.r8, st);
        }));
      }
    }
    TRY(panel_bf16(G, d_out, Bt, d_out, M, L.M8, d_out, r, L.r8, L.splits_q, L.ksplit_q, col_scale(scale), pp,
                   static_cast<uint16_t*>(Qs), ldqs, static_cast<uint16_t*>(Qt), L.M8, st));
  }
  // dX = [G | Qs] [W ; A]; with a dropout mask the rank-r term is added
  // separately, masked: dX = G W, then dX += keep * (Qs A)
  if (dX && L.dx_nt) {
    // W read with its contraction rows costs the whole-tile kernel ~12 % more
    // than the same product read as W^T, which one transposing pass gives
    const void* Wt = Wt_in;
    const void* At = ov && ov->At ? ov->At : w + L.at;
    if (!Wt) {
      uint16_t* wt = reinterpret_cast<uint16_t*>(w + L.wt);
      HIPTRY(timed(K_TRANSPOSE_W, 0, 4.0 * ko * ki, st, [&] {
        return launch_transpose_tile(static_cast<const uint16_t*>(W), d_in, d_out, d_in, wt, d_out, d_out, st);
      }));
      Wt = wt;
    }
    if (!(ov && ov->At) && !at_done)
      HIPTRY(timed(K_TRANSPOSE_W, 0, 2.0 * rr * ki + 2.0 * ki * L.r8, st, [&] {
        return launch_transpose_tile(static_cast<const uint16_t*>(A), d_in, r, d_in,
                                     reinterpret_cast<uint16_t*>(w + L.at), L.r8, L.r8, st);
      }));
    GemmArgs a = blank();
    a.a1 = G; a.lda1 = d_out; a.b1 = Wt; a.ldb1 = d_out; a.K1 = d_out;
    a.a2 = Qs; a.lda2 = ldqs; a.b2 = At; a.ldb2 = L.r8; a.K2 = keep ? 0 : r;
    a.m_load = M; a.m_store = M; a.n_load = d_in; a.n_store = d_in;
    a.c = dX; a.ldc = d_in;
    HIPTRY(gemm(G_BF16_BIG_NT_STORE, a, 1, st, 2 * Md * ki * (ko + rr),
                (Md * ko + Md * rr + rr * ki + Md * ki + ko * ki) * e));
  } else if (dX) {
    GemmArgs a = blank();
    a.a1 = G; a.lda1 = d_out; a.b1 = W; a.ldb1 = d_in; a.K1 = d_out;
    a.a2 = Qs; a.lda2 = ldqs; a.b2 = A; a.ldb2 = d_in; a.K2 = keep ? 0 : r;
    a.m_load = M; a.m_store = M; a.n_load = d_in; a.n_store = d_in;
    a.c = dX; a.ldc = d_in;
    GemmKind k;
    const bool big = use_big(M, d_in);
    if (nf4) {
      a.codes = nf4->codes; a.absmax = nf4->absmax; a.codes_ld = d_in / 2; a.blocks_per_row = d_in / 64;
      for (int i = 0; i < 16; ++i) a.nf4_table[i] = nf4->table[i];
      k = big ? G_NF4_BIG_NN_STORE : G_NF4_MED_NN_STORE;
    } else {
      k = f32 ? G_F32_NN_STORE : (big ? G_BF16_BIG_NN_STORE : G_BF16_MED_NN_STORE);
    }
    const double wbytes = nf4 ? ko * ki / 2 + ko * ki / 64 * 4 : ko * ki * e;
    const double flop = 2 * Md * ki * (ko + rr), bytes = (Md * ko + Md * rr + rr * ki + Md * ki) * e + wbytes;
    if (!f32 && L.splits_main > 1) {
      // few tokens: split partials over d_out (the rank-r segment in the last
      // split), then the fixed-order sum
      const int S = L.splits_main;
      float* sp = reinterpret_cast<float*>(w + L.spart);
      a.k_split = L.ksplit_main; a.c = sp; a.ldc = d_in; a.part_stride = M * d_in;
      HIPTRY(gemm(nf4 ? G_NF4_MED_NN_PARTIAL : G_BF16_MED_NN_PARTIAL, a, S, st, flop,
                  bytes - Md * ki * e + 4.0 * S * Md * ki));
      HIPTRY(timed(K_FINISH, double(S) * Md * ki, 4.0 * S * Md * ki + Md * ki * e, st, [&] {
        return launch_split_finish(sp, S, M * d_in, M, d_in, static_cast<uint16_t*>(dX), d_in, nullptr, nullptr,
                                   nullptr, 0, st);
      }));
    } else {
      HIPTRY(gemm(k, a, 1, st, flop, bytes));
    }
  }
  if (dX && keep) {
    GemmArgs b = blank();
    b.a1 = Qs; b.lda1 = ldqs; b.b1 = A; b.ldb1 = d_in; b.K1 = r;
    b.m_load = M; b.m_store = M; b.n_load = d_in; b.n_store = d_in;
    b.c = dX; b.ldc = d_in; b.cin = dX; b.ldcin = d_in; b.mask = keep; b.mask_ld = d_in / 8;
    HIPTRY(gemm(f32 ? G_F32_NN_ADD_MASKED : G_BF16_MED_NN_ADD_MASKED, b, 1, st, 2 * Md * ki * rr,
                (Md * rr + rr * ki + 2 * Md * ki) * e + Md * ki / 8));
  }
  const GemmKind ksplit = f32 ? G_F32_SPLIT_NN_PARTIAL : G_BF16_SPLIT_NN_PARTIAL;
  // bf16: the dB partials have their own buffer and both sums run as one
  // launch (a group's: one for all its members, after the group's dA)
  float* partb = f32 ? part : (ov && ov->partb ? ov->partb : reinterpret_cast<float*>(w + L.partb));
  ReduceBatch own;
  ReduceBatch* red = f32 ? nullptr : (ov && ov->red ? ov->red : &own);
  // dB^T = Pt G  -> partials [splits][r8, d_out] -> dB [d_out, r]
  {
    GemmArgs a = blank();
    a.a1 = Pt; a.lda1 = L.M8; a.b1 = G; a.ldb1 = d_out; a.K1 = M;
    a.m_load = L.r8; a.m_store = L.r8; a.n_load = d_out; a.n_store = d_out;
    a.k_split = L.ksplit_dB; a.c = partb; a.ldc = d_out; a.part_stride = L.r8 * d_out;
    HIPTRY(gemm(ksplit, a, L.splits_dB, st, 2 * rr * ko * Md,
                (rr * Md + Md * ko) * e + 4.0 * L.splits_dB * L.r8 * ko));
    if (red)
      HIPTRY(red->add(partb, L.splits_dB, r, d_out, L.r8 * d_out, true, dB));
    else
      HIPTRY(timed(K_REDUCE, double(L.splits_dB) * rr * ko, 4.0 * (L.splits_dB + 1) * rr * ko, st, [&] {
        return launch_reduce_splits(partb, L.splits_dB, r, d_out, L.r8 * d_out, true, dB, st);
      }));
  }
  // dA = Qt X -> partials [splits][r8, d_in] -> dA [r, d_in]
  if (!ov) {
    GemmArgs a = blank();
    a.a1 = Qt; a.lda1 = L.M8; a.b1 = Xp; a.ldb1 = d_in; a.K1 = M;
    a.m_load = L.r8; a.m_store = L.r8; a.n_load = d_in; a.n_store = d_in;
    a.k_split = L.ksplit_dA; a.c = part; a.ldc = d_in; a.part_stride = L.r8 * d_in;
    HIPTRY(gemm(ksplit, a, L.splits_dA, st, 2 * rr * ki * Md,
                (rr * Md + Md * ki) * e + 4.0 * L.splits_dA * L.r8 * ki));
    if (red)
      HIPTRY(red->add(part, L.splits_dA, r, d_in, L.r8 * d_in, false, dA));
    else
      HIPTRY(timed(K_REDUCE, double(L.splits_dA) * rr * ki, 4.0 * (L.splits_dA + 1) * rr * ki, st, [&] {
        return launch_reduce_splits(part, L.splits_dA, r, d_in, L.r8 * d_in, false, dA, st);
      }));
  }
  if (red == &own)
    HIPTRY(timed(K_REDUCE, double(L.splits_dB) * rr * ko + (ov ? 0.0 : double(L.splits_dA) * rr * ki),
                 4.0 * (L.splits_dB + 1) * rr * ko + (ov ? 0.0 : 4.0 * (L.splits_dA + 1) * rr * ki), st,
                 [&] { return launch_reduce_batch(own, st); }));
  return LORA_OK;
}

int check_rope(int head_dim, int64_t d_out, int64_t M, const int32_t* pos, const float* c, const float* s,
               int64_t max_pos) {
  if (head_dim != 128 || d_out % 128) return LORA_ERR_SHAPE;
  // cache rows are addressed with 32-bit byte offsets (256 bytes a row)
  if (max_pos < 1 || max_pos > LORA_ROPE_MAX_POS) return LORA_ERR_SHAPE;
  TRY(check_ptrs({c, s}));
  return M > 0 ? check_ptrs({pos}) : LORA_OK;
}

int check_nf4(int64_t d_in, int blocksize, const uint8_t* codes, const float* absmax, const float* table) {
  if (blocksize != 64 || d_in % 64) return LORA_ERR_SHAPE;
  if (!table) return LORA_ERR_NULL;
  return check_ptrs({codes, absmax});
}

// ---------------------------------------------------------------------------
// groups of projections sharing X
// ---------------------------------------------------------------------------
// bf16: the members' rank rows stacked, each padded to r8_g (rt = sum r8_g,
// member g at row off[g]), in sub-groups of consecutive members within the
// DMA kernels' row limits (a wider member alone): each panel sub-group (up
// to 256 rows) is one pass over X for the forward panel and one for the
// backward's recomputation, each dA sub-group (up to 128) one pass for dA,
// reading each member's A in place.  Workspace: forward the panel P = [s_1 X A_1^T | ..] [M, rt];
// backward Pt [rt, M8], Qs [M8, rt], Qt [rt, M8] and per member B^T, A^T
// and its dB partials (kept until the group's batched transposes and sums).
// One shared region follows, used in turn by the panels' split partials,
// each member's own scratch, and the sub-groups' dA partials.
struct GroupLayout {
  int64_t rt = 0, M8 = 0, off[LORA_GROUP_MAX + 1] = {};
  size_t p = 0, pt = 0, qs = 0, qt = 0, shared = 0, total = 0;
  size_t bt[LORA_GROUP_MAX] = {}, at[LORA_GROUP_MAX] = {}, partb[LORA_GROUP_MAX] = {};
  // panel sub-groups (at most 256 rows: panel_dma_kernel) and dA sub-groups
  // (at most 128: splitnn_dma_kernel); s: members [g0[s], g0[s + 1])
  int nsub = 0, sub_g0[LORA_GROUP_MAX + 1] = {};
  int nasub = 0, asub_g0[LORA_GROUP_MAX + 1] = {};
  int splits_p[LORA_GROUP_MAX] = {}, splits_a[LORA_GROUP_MAX] = {};
  int64_t ksplit_p[LORA_GROUP_MAX] = {}, ksplit_a[LORA_GROUP_MAX] = {};
  size_t part_a[LORA_GROUP_MAX] = {};  // floats from the shared region to dA sub-group s's partials
  Layout mem[LORA_GROUP_MAX];
};

int member_op(bool bwd, const lora_group_member& m) {
  if (m.W_nf4) return bwd ? LORA_OP_NF4_BWD : LORA_OP_NF4_FWD;
  if (m.rope) return bwd ? LORA_OP_ROPE_BWD : LORA_OP_ROPE_FWD;
  return bwd ? LORA_OP_BWD : LORA_OP_FWD;
}

GroupLayout make_group_layout(bool bwd, int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* mb) {
  GroupLayout G;
  const size_t eb = elem_bytes(dtype);
  G.M8 = rup(M, 8);
  size_t shared = 0;
  for (int g = 0; g < n; ++g) {
    G.off[g] = G.rt;
    G.rt += rup(mb[g].r, 8);
    G.mem[g] = make_layout(member_op(bwd, mb[g]), dtype, M, d_in, mb[g].d_out, mb[g].r,
                           mb[g].W_t != nullptr && !mb[g].W_nf4);
    if (G.mem[g].total > shared) shared = G.mem[g].total;
  }
  G.off[n] = G.rt;
  // (operands too wide for the panel DMA kernel: every member alone)
  const bool stack = panel_dma_fits(256, d_in, d_in);
  for (int g = 0; g < n; ++g) {
    if (g == 0 || !stack || G.off[g + 1] - G.off[G.sub_g0[G.nsub - 1]] > 256) G.sub_g0[G.nsub++] = g;
    if (g == 0 || G.off[g + 1] - G.off[G.asub_g0[G.nasub - 1]] > 128) G.asub_g0[G.nasub++] = g;
  }
  G.sub_g0[G.nsub] = n;
  G.asub_g0[G.nasub] = n;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (eb == 2) {
    for (int s = 0; s < G.nsub; ++s) {
      const int64_t rs = G.off[G.sub_g0[s + 1]] - G.off[G.sub_g0[s]];
      panel_split(M, d_in, rs, &G.splits_p[s], &G.ksplit_p[s]);
      const size_t pp = size_t(G.splits_p[s]) * G.M8 * rs * 4;  // the panels run one after another
      if (pp > shared) shared = pp;
    }
    if (!bwd) {
      G.p = take(size_t(M) * G.rt * eb);
    } else {
      G.pt = take(size_t(G.rt) * G.M8 * eb);
      G.qs = take(size_t(G.M8) * G.rt * eb);
      G.qt = take(size_t(G.rt) * G.M8 * eb);
      for (int g = 0; g < n; ++g) {
        const Layout& L = G.mem[g];
        G.bt[g] = take(size_t(L.r8) * mb[g].d_out * eb);
        G.at[g] = take(size_t(d_in) * L.r8 * eb);
        G.partb[g] = take(size_t(L.splits_dB) * L.r8 * mb[g].d_out * 4);
      }
      size_t pa = 0;  // every sub-group's dA partials until the batched sum
      for (int s = 0; s < G.nasub; ++s) {
        const int64_t rs = G.off[G.asub_g0[s + 1]] - G.off[G.asub_g0[s]];
        choose_split(M, rs, d_in, true, &G.splits_a[s], &G.ksplit_a[s]);
        G.part_a[s] = pa / 4;
        pa = align256(pa + size_t(G.splits_a[s]) * rs * d_in * 4);
      }
      if (pa > shared) shared = pa;
    }
  }
  G.shared = take(shared);
  G.total = off;
  return G;
}

// Validation of a whole group before any launch.
int check_group(bool bwd, int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* mb, const void* X,
                int head_dim, const int32_t* pos, const float* cosc, const float* sinc, int64_t max_pos,
                const float* table16) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (!mb) return LORA_ERR_NULL;
  if (n < 1 || n > LORA_GROUP_MAX) return LORA_ERR_SHAPE;
  if (M > 0) TRY(check_ptrs({X}));
  for (int g = 0; g < n; ++g) {
    const lora_group_member& m = mb[g];
    TRY(check_sizes(M, d_in, m.d_out, m.r));
    TRY(check_ptrs({m.A, m.B}));
    if (m.W_nf4) {
      if (dtype != LORA_BF16) return LORA_ERR_DTYPE;
      if (m.rope) return LORA_ERR_SHAPE;
      TRY(check_nf4(d_in, 64, m.W_nf4, m.absmax, table16));
    } else {
      TRY(check_ptrs({m.W}));
    }
    if (m.rope) TRY(check_rope(head_dim, m.d_out, M, pos, cosc, sinc, max_pos));
    if (m.W_t && !aligned16(m.W_t)) return LORA_ERR_ALIGN;
    if (!bwd) {
      if (M > 0) TRY(check_ptrs({m.Y}));
    } else {
      TRY(check_ptrs({m.dA, m.dB}));
      if (M > 0) TRY(check_ptrs({m.dY}));
      if (m.dX && !aligned16(m.dX)) return LORA_ERR_ALIGN;
    }
  }
  return LORA_OK;
}

int check_group_ws(const GroupLayout& G, const void* ws, size_t ws_bytes) {
  if (G.total == 0) return LORA_OK;
  if (!ws || ws_bytes < G.total) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

// The group's rank-r panels s_g X A_g^T, one pass over X per sub-group, each
// member's A read in place (a wider member alone: its A is the panel's R):
// P into out (rows of `rows`, row stride rt) and/or P^T into outt ([rt, M8]).
int group_panel(int64_t M, int64_t d_in, int n, const lora_group_member* mb, const void* X, const GroupLayout& G,
                float* part, uint16_t* out, int64_t rows, uint16_t* outt, hipStream_t st) {
  for (int s = 0; s < G.nsub; ++s) {
    const int g0 = G.sub_g0[s], g1 = G.sub_g0[s + 1];
    const int64_t o0 = G.off[g0], rs = G.off[g1] - o0;
    ColScale cs{};
    cs.n = g1 - g0;
    PanelSrc src;
    src.n = g1 - g0;
    for (int g = g0; g < g1; ++g) {
      cs.end[g - g0] = G.off[g + 1] - o0;
      cs.s[g - g0] = mb[g].scale;
      src.rs[g - g0] = mb[g].A;
      src.beg[g - g0] = (int)(G.off[g] - o0);
      src.rows[g - g0] = (int)mb[g].r;
    }
    const bool multi = panel_dma_fits(rs, d_in, d_in);
    TRY(panel_bf16(X, d_in, mb[g0].A, d_in, M, rows, d_in, multi ? rs : mb[g0].r, rs, G.splits_p[s], G.ksplit_p[s],
                   cs, part, out ? out + o0 : nullptr, G.rt, outt ? outt + o0 * G.M8 : nullptr, G.M8, st,
                   multi ? &src : nullptr));
  }
  return LORA_OK;
}

// Every member's forward GEMM in one whole-tile launch: bf16 W, M a multiple
// of 256, each d_out a multiple of 256 (its tiles whole) and r of 8 (B read
// as it is).  A k or v projection of 1024 outputs alone gives 128 tiles for
// 256 CUs (and runs the 128 x 128 kernel); stacked with q and each other they
// share the launch's waves of tiles.
bool group_gemm_fits(int64_t M, int64_t d_in, int n, const lora_group_member* mb, const GroupLayout& G) {
  if (M <= 0 || M % 256 || d_in % 64 || n > kGroupGemmMax) return false;
  int64_t ld = std::max(d_in, G.rt), cols = 0;
  for (int g = 0; g < n; ++g) {
    if (mb[g].W_nf4 || mb[g].d_out % 256 || mb[g].r % 8) return false;
    ld = std::max(ld, mb[g].r);
    cols += mb[g].d_out;
  }
  // the member table holds tile numbers as int
  return whole_ld_fits(ld) && (M / 256) * (cols / 256) <= INT32_MAX;
}

int group_gemm(int64_t M, int64_t d_in, int n, const lora_group_member* mb, const void* X, const Rope* rope,
               const uint16_t* P, const GroupLayout& G, hipStream_t st) {
  GemmArgs a = blank();
  a.a1 = X; a.lda1 = d_in; a.ldb1 = d_in; a.K1 = d_in; a.lda2 = G.rt;
  a.m_load = M; a.m_store = M;
  if (rope) { a.pos = rope->pos; a.cosc = rope->cosc; a.sinc = rope->sinc; a.max_pos = rope->max_pos; }
  a.n_mem = n;
  const int64_t tiles_m = M / 256;
  int64_t cols = 0, ldb2 = 0;
  double flop = 0, bytes = 2.0 * M * d_in;
  for (int g = 0; g < n; ++g) {
    const lora_group_member& m = mb[g];
    a.mem_tile0[g] = (int)(tiles_m * (cols / 256));
    a.mem_b1[g] = m.W;
    a.mem_b2[g] = m.B;
    a.mem_ldb2[g] = (int)m.r;
    a.mem_a2[g] = P + G.off[g];
    a.mem_k2[g] = (int)m.r;
    a.mem_c[g] = m.Y;
    a.mem_ldc[g] = (int)m.d_out;
    a.mem_rope[g] = m.rope ? 1 : 0;
    cols += m.d_out;
    ldb2 = std::max(ldb2, m.r);
    const double Md = double(M), ko = double(m.d_out), ki = double(d_in), rr = double(m.r);
    flop += 2 * Md * ko * (ki + rr);
    bytes += (Md * rr + ko * rr + Md * ko + ko * ki) * 2;
  }
  a.mem_tile0[n] = (int)(tiles_m * (cols / 256));
  a.n_load = cols; a.n_store = cols;
  a.ldb2 = ldb2;  // the widest member's, for the kernel's offset-range check
  HIPTRY(gemm(G_BF16_WHOLE_GROUP, a, 1, st, flop, bytes));
  return LORA_OK;
}

int group_forward(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* mb, const void* X,
                  const Rope* rope, const float* table16, void* ws, const GroupLayout& G, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  char* sh = w + G.shared;
  const bool share = dtype == LORA_BF16 && M > 0;
  uint16_t* P = reinterpret_cast<uint16_t*>(w + G.p);
  if (share) {
    TRY(group_panel(M, d_in, n, mb, X, G, reinterpret_cast<float*>(sh), P, M, nullptr, st));
    if (group_gemm_fits(M, d_in, n, mb, G)) return group_gemm(M, d_in, n, mb, X, rope, P, G, st);
  }
  for (int g = 0; g < n; ++g) {
    const lora_group_member& m = mb[g];
    const Nf4W q{m.W_nf4, m.absmax, table16};
    TRY(forward_impl(dtype, M, d_in, m.d_out, m.r, m.scale, X, m.W, m.W_nf4 ? &q : nullptr, m.A, m.B,
                     m.rope ? rope : nullptr, m.Y, sh, G.mem[g], st, share ? P + G.off[g] : nullptr, G.rt));
  }
  return LORA_OK;
}

int group_backward(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* mb, const void* X,
                   const Rope* rope, const float* table16, void* ws, const GroupLayout& G, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  char* sh = w + G.shared;
  const bool share = dtype == LORA_BF16 && M > 0;
  uint16_t* Pt = reinterpret_cast<uint16_t*>(w + G.pt);
  uint16_t* Qs = reinterpret_cast<uint16_t*>(w + G.qs);
  uint16_t* Qt = reinterpret_cast<uint16_t*>(w + G.qt);
  if (share) {
    TRY(group_panel(M, d_in, n, mb, X, G, reinterpret_cast<float*>(sh), nullptr, G.M8, Pt, st));
  }
  // every member's B^T (r a multiple of 8) and A^T (whole-tile dX) in one launch
  TransposeBatch tb;
  bool have_bt[LORA_GROUP_MAX] = {}, have_at[LORA_GROUP_MAX] = {};
  double tbytes = 0;
  if (share) {
    for (int g = 0; g < n; ++g) {
      const lora_group_member& m = mb[g];
      const Layout& L = G.mem[g];
      if (m.r == L.r8) {
        HIPTRY(tb.add(static_cast<const uint16_t*>(m.B), m.r, m.d_out, m.r, reinterpret_cast<uint16_t*>(w + G.bt[g]),
                      m.d_out, m.d_out));
        have_bt[g] = true;
        tbytes += 4.0 * m.r * m.d_out;
        if (m.dX && L.dx_nt) {
          HIPTRY(tb.add(static_cast<const uint16_t*>(m.A), d_in, m.r, d_in, reinterpret_cast<uint16_t*>(w + G.at[g]),
                        L.r8, L.r8));
          have_at[g] = true;
          tbytes += 4.0 * m.r * d_in;
        }
      }
    }
    HIPTRY(timed(K_TRANSPOSE, 0, tbytes, st, [&] { return launch_transpose_batch(tb, st); }));
  }
  ReduceBatch red;
  for (int g = 0; g < n; ++g) {
    const lora_group_member& m = mb[g];
    const Nf4W q{m.W_nf4, m.absmax, table16};
    PanelSlices ov{Pt + G.off[g] * G.M8, Qs + G.off[g], G.rt, Qt + G.off[g] * G.M8};
    ov.Bt = have_bt[g] ? w + G.bt[g] : nullptr;
    ov.At = have_at[g] ? w + G.at[g] : nullptr;
    ov.partb = reinterpret_cast<float*>(w + G.partb[g]);
    ov.red = &red;
    TRY(backward_impl(dtype, M, d_in, m.d_out, m.r, m.scale, X, m.W, m.W_nf4 ? &q : nullptr, m.A, m.B,
                      m.rope ? rope : nullptr, m.dY, m.dX, m.dA, m.dB, sh, G.mem[g], st, share ? &ov : nullptr,
                      nullptr, nullptr, G.mem[g].dx_nt && !m.W_nf4 ? m.W_t : nullptr));
  }
  if (!share) return LORA_OK;
  // dA of every member of a sub-group in one pass over X: Qt rows X ->
  // partials [splits][rows, d_in]; then every dA and dB sum in one launch
  float* part = reinterpret_cast<float*>(sh);
  const double Md = double(M), ki = double(d_in);
  double rflop = 0, rbytes = 0;
  for (int s = 0; s < G.nasub; ++s) {
    const int g0 = G.asub_g0[s], g1 = G.asub_g0[s + 1];
    const int64_t o0 = G.off[g0], rs = G.off[g1] - o0;
    float* ps = part + G.part_a[s];
    const int S = G.splits_a[s];
    GemmArgs a = blank();
    a.a1 = Qt + o0 * G.M8; a.lda1 = G.M8; a.b1 = X; a.ldb1 = d_in; a.K1 = M;
    a.m_load = rs; a.m_store = rs; a.n_load = d_in; a.n_store = d_in;
    a.k_split = G.ksplit_a[s]; a.c = ps; a.ldc = d_in; a.part_stride = rs * d_in;
    HIPTRY(gemm(G_BF16_SPLIT_NN_PARTIAL, a, S, st, 2 * double(rs) * ki * Md,
                (double(rs) * Md + Md * ki) * 2 + 4.0 * S * rs * ki));
    for (int g = g0; g < g1; ++g) {
      const double rg = double(mb[g].r), ko = double(mb[g].d_out);
      const int sb = G.mem[g].splits_dB;
      HIPTRY(red.add(ps + (G.off[g] - o0) * d_in, S, mb[g].r, d_in, rs * d_in, false, mb[g].dA));
      rflop += double(S) * rg * ki + double(sb) * rg * ko;
      rbytes += 4.0 * (S + 1) * rg * ki + 4.0 * (sb + 1) * rg * ko;
    }
  }
  HIPTRY(timed(K_REDUCE, rflop, rbytes, st, [&] { return launch_reduce_batch(red, st); }));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// SwiGLU on a gate / up pair
// ---------------------------------------------------------------------------
// Workspace: the pair's group layout first (panels, shared scratch),
// then forward: the dequantised NF4 weights and padded B's of the fused GEMM,
// or G and U for the elementwise path; backward: dG, dU and the up's input
// gradient before it is added to dX.
struct SwigluLayout {
  GroupLayout G;
  bool fused = false;
  size_t wg = 0, wu = 0, bg = 0, bu = 0, gbuf = 0, ubuf = 0, dg = 0, du = 0, dxu = 0, total = 0;
};

bool swiglu_fusable(int dtype, int64_t M, int64_t d_in, const lora_group_member* mb) {
  const bool nf4 = mb[0].W_nf4 || mb[1].W_nf4;
  return dtype == LORA_BF16 && M > 0 && M % 256 == 0 && mb[0].d_out % 128 == 0 && d_in % 64 == 0 &&
         (!nf4 || M >= LORA_NF4_DEQUANT_MIN_TOKENS) && d_in * 2 * (256 + 64) < (int64_t(1) << 30);
}

SwigluLayout make_swiglu_layout(bool bwd, int dtype, int64_t M, int64_t d_in, const lora_group_member* mb) {
  SwigluLayout S;
  S.G = make_group_layout(bwd, dtype, M, d_in, 2, mb);
  const size_t eb = elem_bytes(dtype);
  const int64_t d = mb[0].d_out;
  size_t off = S.G.total;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (!bwd) {
    S.fused = swiglu_fusable(dtype, M, d_in, mb);
    if (S.fused) {
      if (mb[0].W_nf4) S.wg = take(size_t(d) * d_in * 2);
      if (mb[1].W_nf4) S.wu = take(size_t(d) * d_in * 2);
      if (mb[0].r % 8) S.bg = take(size_t(d) * rup(mb[0].r, 8) * 2);
      if (mb[1].r % 8) S.bu = take(size_t(d) * rup(mb[1].r, 8) * 2);
    } else {
      S.gbuf = take(size_t(M) * d * eb);
      S.ubuf = take(size_t(M) * d * eb);
    }
  } else {
    S.dg = take(size_t(M) * d * eb);
    S.du = take(size_t(M) * d * eb);
    S.dxu = take(size_t(M) * d_in * eb);
  }
  S.total = off;
  return S;
}

int check_swiglu(bool bwd, int dtype, int64_t M, int64_t d_in, const lora_group_member* mb, const void* X,
                 const float* table16) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (!mb) return LORA_ERR_NULL;
  if (M > 0) TRY(check_ptrs({X}));
  for (int g = 0; g < 2; ++g) {
    const lora_group_member& m = mb[g];
    TRY(check_sizes(M, d_in, m.d_out, m.r));
    if (m.rope || m.d_out != mb[0].d_out) return LORA_ERR_SHAPE;
    TRY(check_ptrs({m.A, m.B}));
    if (m.W_nf4) {
      if (dtype != LORA_BF16) return LORA_ERR_DTYPE;
      TRY(check_nf4(d_in, 64, m.W_nf4, m.absmax, table16));
    } else {
      TRY(check_ptrs({m.W}));
    }
    if (bwd) TRY(check_ptrs({m.dA, m.dB}));
    if (!bwd && m.Y && !aligned16(m.Y)) return LORA_ERR_ALIGN;
    if (m.W_t && !aligned16(m.W_t)) return LORA_ERR_ALIGN;
  }
  return LORA_OK;
}

int check_ws_bytes(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return LORA_OK;
  if (!ws || ws_bytes < need) return LORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LORA_ERR_ALIGN;
  return LORA_OK;
}

int swiglu_forward(int dtype, int64_t M, int64_t d_in, const lora_group_member* mb, const void* X,
                   const float* table16, void* H, void* ws, const SwigluLayout& S, hipStream_t st) {
  if (M == 0) return LORA_OK;
  char* w = static_cast<char*>(ws);
  const int64_t d = mb[0].d_out;
  const int eb = elem_bytes(dtype);
  if (!S.fused) {
    lora_group_member m[2] = {mb[0], mb[1]};
    m[0].Y = mb[0].Y ? mb[0].Y : w + S.gbuf;
    m[1].Y = mb[1].Y ? mb[1].Y : w + S.ubuf;
    TRY(group_forward(dtype, M, d_in, 2, m, X, nullptr, table16, ws, S.G, st));
    HIPTRY(timed(K_SWIGLU, 4.0 * M * d, 3.0 * M * d * eb, st,
                 [&] { return launch_swiglu_apply(eb, m[0].Y, m[1].Y, H, M * d, st); }));
    return LORA_OK;
  }
  const GroupLayout& G = S.G;
  // the pair's rank-r panels in one pass over X: P = [sg X Ag^T | su X Au^T]
  uint16_t* P = reinterpret_cast<uint16_t*>(w + G.p);
  TRY(group_panel(M, d_in, 2, mb, X, G, reinterpret_cast<float*>(w + G.shared), P, M, nullptr, st));
  const void* Wp[2];
  const void* Bp[2];
  const size_t woff[2] = {S.wg, S.wu}, boff[2] = {S.bg, S.bu};
  for (int g = 0; g < 2; ++g) {
    Wp[g] = mb[g].W;
    if (mb[g].W_nf4) {
      TRY(dequant_w(Nf4W{mb[g].W_nf4, mb[g].absmax, table16}, d * d_in, w + woff[g], st));
      Wp[g] = w + woff[g];
    }
    Bp[g] = mb[g].B;
    if (mb[g].r % 8) {
      const int64_t r8 = rup(mb[g].r, 8);
      HIPTRY(timed(K_PAD, 0, 2.0 * d * r8 * 2, st,
                   [&] { return launch_pad_cols(2, mb[g].B, w + boff[g], d, mb[g].r, r8, st); }));
      Bp[g] = w + boff[g];
    }
  }
  // gate and up as one GEMM over [X | P]: rows of Wg and Wu interleaved in
  // 32-row blocks, epilogue H = silu(g) u (and G, U when asked for)
  GemmArgs a = blank();
  a.a1 = X; a.lda1 = d_in; a.b1 = Wp[0]; a.b1u = Wp[1]; a.ldb1 = d_in; a.K1 = d_in;
  a.a2 = P; a.lda2 = G.rt; a.b2 = Bp[0]; a.ldb2 = rup(mb[0].r, 8); a.b2u = Bp[1]; a.ldb2u = rup(mb[1].r, 8);
  a.K2 = G.rt; a.k2_split = rup(mb[0].r, 8);
  a.m_load = M; a.m_store = M; a.n_load = 2 * d; a.n_store = 2 * d;
  a.c = H; a.ldc = d; a.cg = mb[0].Y; a.cu = mb[1].Y;
  const double Md = double(M), ki = double(d_in), ko = double(d), rt = double(mb[0].r + mb[1].r);
  const double outs = 1.0 + (mb[0].Y ? 1 : 0) + (mb[1].Y ? 1 : 0);
  HIPTRY(gemm(G_BF16_WHOLE_SWIGLU, a, 1, st, 2 * Md * ko * (2 * ki) + 2 * Md * ko * rt,
              (Md * ki + Md * rt + 2 * ko * ki + ko * rt) * 2 + outs * Md * ko * 2));
  return LORA_OK;
}

int swiglu_backward(int dtype, int64_t M, int64_t d_in, const lora_group_member* mb, const void* X,
                    const float* table16, const void* dH, const void* Gs, const void* Us, void* dX, void* ws,
                    const SwigluLayout& S, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  const int64_t d = mb[0].d_out;
  const int eb = elem_bytes(dtype);
  lora_group_member m[2] = {mb[0], mb[1]};
  if (M > 0)
    HIPTRY(timed(K_SWIGLU, 10.0 * M * d, 5.0 * M * d * eb, st,
                 [&] { return launch_swiglu_grad(eb, dH, Gs, Us, w + S.dg, w + S.du, M * d, st); }));
  m[0].dY = w + S.dg;
  m[1].dY = w + S.du;
  m[0].dX = dX;
  m[1].dX = dX ? w + S.dxu : nullptr;
  TRY(group_backward(dtype, M, d_in, 2, m, X, nullptr, table16, ws, S.G, st));
  if (dX && M > 0)
    HIPTRY(timed(K_SWIGLU, 1.0 * M * d_in, 3.0 * M * d_in * eb, st,
                 [&] { return launch_add_into(eb, dX, w + S.dxu, M * d_in, st); }));
  return LORA_OK;
}

// ---------------------------------------------------------------------------
// the forward without a caller workspace: a static device array per GPU
// ---------------------------------------------------------------------------
// Each device the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// copy comes from hipGetSymbolAddress, called once per device with that
// device current, and is kept here.
constexpr size_t kStaticScratchBytes = size_t(LORA_STATIC_SCRATCH_BYTES);

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` on each device (NULL: not looked up yet)

}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LORA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LORA_ERR_DEVICE;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LORA_OK;
}

}  // namespace

// ===========================================================================
// exported C ABI
// ===========================================================================
extern "C" {

int lora_abi_version(void) { return LORA_ABI_VERSION; }

const char* lora_strerror(int code) {
  switch (code) {
    case LORA_OK: return "ok";
    case LORA_ERR_NULL: return "null pointer";
    case LORA_ERR_SHAPE: return "unsupported shape";
    case LORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LORA_ERR_DTYPE: return "unsupported dtype";
    case LORA_ERR_WORKSPACE: return "workspace too small";
    case LORA_ERR_DEVICE: return "device error (not gfx950, or launch failed)";
    case LORA_ERR_SCRATCH: return "problem needs more scratch than the library's static buffer holds";
    default: return "unknown error";
  }
}

size_t lora_workspace_bytes(int op, int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
  if (op < LORA_OP_FWD || op > LORA_OP_DROPOUT_BWD) return 0;
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  if (check_sizes(M, d_in, d_out, r) != LORA_OK) return 0;
  return make_layout(op, dtype, M, d_in, d_out, r).total;
}

int lora_linear_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                    const void* W, const void* A, const void* B, void* Y, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({W, A, B}));
  if (M > 0) TRY(check_ptrs({X, Y}));
  const Layout L = make_layout(LORA_OP_FWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  return forward_impl(dtype, M, d_in, d_out, r, scale, X, W, nullptr, A, B, nullptr, Y, ws, L,
                      static_cast<hipStream_t>(stream));
}

int lora_linear_fwd_noalloc(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale,
                            const void* X, const void* W, const void* A, const void* B, void* Y, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({W, A, B}));
  if (M > 0) TRY(check_ptrs({X, Y}));
  const Layout L = make_layout(LORA_OP_FWD, dtype, M, d_in, d_out, r);
  if (L.total > kStaticScratchBytes) return LORA_ERR_SCRATCH;
  TRY(check_device());
  void* ws = nullptr;
  TRY(static_scratch(&ws));
  return forward_impl(dtype, M, d_in, d_out, r, scale, X, W, nullptr, A, B, nullptr, Y, ws, L,
                      static_cast<hipStream_t>(stream));
}

int lora_linear_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                    const void* W, const void* A, const void* B, const void* dY, void* dX, float* dA, float* dB,
                    void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({W, A, B, dA, dB}));
  if (M > 0) TRY(check_ptrs({X, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  const Layout L = make_layout(LORA_OP_BWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  return backward_impl(dtype, M, d_in, d_out, r, scale, X, W, nullptr, A, B, nullptr, dY, dX, dA, dB, ws, L,
                       static_cast<hipStream_t>(stream));
}

int lora_rope_cache(int64_t max_pos, int head_dim, double theta, float* cos_cache, float* sin_cache,
                    void* stream) {
  if (max_pos < 1 || head_dim < 2 || head_dim % 2 || !(theta > 0.0)) return LORA_ERR_SHAPE;
  TRY(check_ptrs({cos_cache, sin_cache}));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIPTRY(timed(K_ROPE_CACHE, 0, 8.0 * max_pos * (head_dim / 2), st,
               [&] { return launch_rope_cache(max_pos, head_dim, theta, cos_cache, sin_cache, st); }));
  return LORA_OK;
}

int lora_qk_rope_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                     const void* W, const void* A, const void* B, int head_dim, const int32_t* positions,
                     const float* cos_cache, const float* sin_cache, int64_t max_pos, void* Y, void* ws,
                     size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({W, A, B}));
  if (M > 0) TRY(check_ptrs({X, Y}));
  TRY(check_rope(head_dim, d_out, M, positions, cos_cache, sin_cache, max_pos));
  const Layout L = make_layout(LORA_OP_ROPE_FWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  const Rope rp{positions, cos_cache, sin_cache, max_pos};
  return forward_impl(dtype, M, d_in, d_out, r, scale, X, W, nullptr, A, B, &rp, Y, ws, L,
                      static_cast<hipStream_t>(stream));
}

int lora_qk_rope_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                     const void* W, const void* A, const void* B, int head_dim, const int32_t* positions,
                     const float* cos_cache, const float* sin_cache, int64_t max_pos, const void* dY, void* dX,
                     float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({W, A, B, dA, dB}));
  if (M > 0) TRY(check_ptrs({X, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  TRY(check_rope(head_dim, d_out, M, positions, cos_cache, sin_cache, max_pos));
  const Layout L = make_layout(LORA_OP_ROPE_BWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  const Rope rp{positions, cos_cache, sin_cache, max_pos};
  return backward_impl(dtype, M, d_in, d_out, r, scale, X, W, nullptr, A, B, &rp, dY, dX, dA, dB, ws, L,
                       static_cast<hipStream_t>(stream));
}

int nf4_lora_linear_fwd(int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                        const uint8_t* W_nf4, const float* absmax, int blocksize, const float* table16,
                        const void* A, const void* B, void* Y, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({A, B}));
  if (M > 0) TRY(check_ptrs({X, Y}));
  TRY(check_nf4(d_in, blocksize, W_nf4, absmax, table16));
  const Layout L = make_layout(LORA_OP_NF4_FWD, LORA_BF16, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  const Nf4W q{W_nf4, absmax, table16};
  return forward_impl(LORA_BF16, M, d_in, d_out, r, scale, X, nullptr, &q, A, B, nullptr, Y, ws, L,
                      static_cast<hipStream_t>(stream));
}

int nf4_lora_linear_bwd(int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, const void* X,
                        const uint8_t* W_nf4, const float* absmax, int blocksize, const float* table16,
                        const void* A, const void* B, const void* dY, void* dX, float* dA, float* dB, void* ws,
                        size_t ws_bytes, void* stream) {
  TRY(check_sizes(M, d_in, d_out, r));
  TRY(check_ptrs({A, B, dA, dB}));
  if (M > 0) TRY(check_ptrs({X, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  TRY(check_nf4(d_in, blocksize, W_nf4, absmax, table16));
  const Layout L = make_layout(LORA_OP_NF4_BWD, LORA_BF16, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  const Nf4W q{W_nf4, absmax, table16};
  return backward_impl(LORA_BF16, M, d_in, d_out, r, scale, X, nullptr, &q, A, B, nullptr, dY, dX, dA, dB, ws, L,
                       static_cast<hipStream_t>(stream));
}

int nf4_dequant(const uint8_t* W_nf4, const float* absmax, int blocksize, int64_t n, const float* table16,
                uint16_t* out_bf16, void* stream) {
  if (blocksize != 64 || n < 0 || n % 64) return LORA_ERR_SHAPE;
  if (!table16) return LORA_ERR_NULL;
  TRY(check_ptrs({W_nf4, absmax, out_bf16}));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIPTRY(timed(K_NF4_DEQ, 2.0 * n, n / 2.0 + n / 16.0 + 2.0 * n, st,
               [&] { return launch_nf4_dequant(W_nf4, absmax, n, table16, out_bf16, st); }));
  return LORA_OK;
}

size_t lora_group_workspace_bytes(int backward, int dtype, int64_t M, int64_t d_in, int n,
                                  const lora_group_member* members) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  if (!members || n < 1 || n > LORA_GROUP_MAX) return 0;
  for (int g = 0; g < n; ++g)
    if (check_sizes(M, d_in, members[g].d_out, members[g].r) != LORA_OK) return 0;
  return make_group_layout(backward != 0, dtype, M, d_in, n, members).total;
}

int lora_group_fwd(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* members, const void* X,
                   int head_dim, const int32_t* positions, const float* cos_cache, const float* sin_cache,
                   int64_t max_pos, const float* table16, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_group(false, dtype, M, d_in, n, members, X, head_dim, positions, cos_cache, sin_cache, max_pos,
                  table16));
  const GroupLayout G = make_group_layout(false, dtype, M, d_in, n, members);
  TRY(check_group_ws(G, ws, ws_bytes));
  TRY(check_device());
  const Rope rp{positions, cos_cache, sin_cache, max_pos};
  return group_forward(dtype, M, d_in, n, members, X, &rp, table16, ws, G, static_cast<hipStream_t>(stream));
}

int lora_group_bwd(int dtype, int64_t M, int64_t d_in, int n, const lora_group_member* members, const void* X,
                   int head_dim, const int32_t* positions, const float* cos_cache, const float* sin_cache,
                   int64_t max_pos, const float* table16, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_group(true, dtype, M, d_in, n, members, X, head_dim, positions, cos_cache, sin_cache, max_pos,
                  table16));
  const GroupLayout G = make_group_layout(true, dtype, M, d_in, n, members);
  TRY(check_group_ws(G, ws, ws_bytes));
  TRY(check_device());
  const Rope rp{positions, cos_cache, sin_cache, max_pos};
  return group_backward(dtype, M, d_in, n, members, X, &rp, table16, ws, G, static_cast<hipStream_t>(stream));
}

int lora_dropout_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                     const uint8_t* keep, const void* X, const void* W, const void* A, const void* B, void* Y, void* ws,
                     size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  if (!(p >= 0.f && p < 1.f)) return LORA_ERR_SHAPE;
  TRY(check_ptrs({W, A, B}));
  if (M > 0) TRY(check_ptrs({X, Y, keep}));
  const Layout L = make_layout(LORA_OP_DROPOUT_FWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* Xm = static_cast<char*>(ws) + L.xm;
  HIPTRY(timed(K_MASK, 0, (2.0 * elem_bytes(dtype) + 0.125) * M * d_in, st,
               [&] { return launch_mask_copy(elem_bytes(dtype), X, keep, Xm, M * d_in, st); }));
  return forward_impl(dtype, M, d_in, d_out, r, scale / (1.f - p), X, W, nullptr, A, B, nullptr, Y, ws, L, st,
                      nullptr, 0, Xm);
}

int lora_dropout_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                     const uint8_t* keep, const void* X, const void* W, const void* A, const void* B, const void* dY,
                     void* dX, float* dA, float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  if (!(p >= 0.f && p < 1.f)) return LORA_ERR_SHAPE;
  TRY(check_ptrs({W, A, B, dA, dB}));
  if (M > 0) TRY(check_ptrs({X, dY, keep}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  const Layout L = make_layout(LORA_OP_DROPOUT_BWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* Xm = static_cast<char*>(ws) + L.xm;
  if (M > 0)
    HIPTRY(timed(K_MASK, 0, (2.0 * elem_bytes(dtype) + 0.125) * M * d_in, st,
                 [&] { return launch_mask_copy(elem_bytes(dtype), X, keep, Xm, M * d_in, st); }));
  return backward_impl(dtype, M, d_in, d_out, r, scale / (1.f - p), X, W, nullptr, A, B, nullptr, dY, dX, dA, dB,
                       ws, L, st, nullptr, Xm, keep);
}

static uint32_t dropout_threshold(float p) { return (uint32_t)std::floor(double(p) * 4294967296.0); }

int lora_dropout_mask(int64_t M, int64_t d_in, float p, uint64_t seed, uint64_t offset, uint8_t* keep,
                      void* stream) {
  if (M < 0 || d_in <= 0 || d_in % 8) return LORA_ERR_SHAPE;
  if (!(p >= 0.f && p < 1.f)) return LORA_ERR_SHAPE;
  if (M == 0) return LORA_OK;
  TRY(check_ptrs({keep}));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIPTRY(timed(K_MASK, 0, 0.125 * M * d_in, st, [&] {
    return launch_dropout_philox(2, nullptr, nullptr, keep, M * d_in, dropout_threshold(p), seed, offset, st);
  }));
  return LORA_OK;
}

int lora_dropout_philox_fwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                            uint64_t seed, uint64_t offset, const void* X, const void* W, const void* A,
                            const void* B, void* Y, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  if (!(p >= 0.f && p < 1.f)) return LORA_ERR_SHAPE;
  TRY(check_ptrs({W, A, B}));
  if (M > 0) TRY(check_ptrs({X, Y}));
  const Layout L = make_layout(LORA_OP_DROPOUT_FWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* Xm = static_cast<char*>(ws) + L.xm;
  HIPTRY(timed(K_MASK, 0, 2.0 * elem_bytes(dtype) * M * d_in, st, [&] {
    return launch_dropout_philox(elem_bytes(dtype), X, Xm, nullptr, M * d_in, dropout_threshold(p), seed, offset,
                                 st);
  }));
  return forward_impl(dtype, M, d_in, d_out, r, scale / (1.f - p), X, W, nullptr, A, B, nullptr, Y, ws, L, st,
                      nullptr, 0, Xm);
}

int lora_dropout_philox_bwd(int dtype, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float scale, float p,
                            uint64_t seed, uint64_t offset, const void* X, const void* W, const void* A,
                            const void* B, const void* dY, void* dX, float* dA, float* dB, void* ws,
                            size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(M, d_in, d_out, r));
  if (!(p >= 0.f && p < 1.f)) return LORA_ERR_SHAPE;
  TRY(check_ptrs({W, A, B, dA, dB}));
  if (M > 0) TRY(check_ptrs({X, dY}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  const Layout L = make_layout(LORA_OP_DROPOUT_BWD, dtype, M, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* Xm = static_cast<char*>(ws) + L.xm;
  uint8_t* keep = reinterpret_cast<uint8_t*>(static_cast<char*>(ws) + L.keep);
  if (M > 0)
    HIPTRY(timed(K_MASK, 0, (2.0 * elem_bytes(dtype) + 0.125) * M * d_in, st, [&] {
      return launch_dropout_philox(elem_bytes(dtype), X, Xm, keep, M * d_in, dropout_threshold(p), seed, offset,
                                   st);
    }));
  return backward_impl(dtype, M, d_in, d_out, r, scale / (1.f - p), X, W, nullptr, A, B, nullptr, dY, dX, dA, dB,
                       ws, L, st, nullptr, Xm, keep);
}

int lora_merge(int dtype, int64_t d_out, int64_t d_in, int64_t r, float scale, const void* W, const void* A,
               const void* B, void* W_out, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return LORA_ERR_DTYPE;
  TRY(check_sizes(0, d_in, d_out, r));
  TRY(check_ptrs({W, A, B, W_out}));
  const Layout L = make_layout(LORA_OP_MERGE, dtype, 0, d_in, d_out, r);
  TRY(check_ws(L, ws, ws_bytes));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int eb = elem_bytes(dtype);
  const void* Bsrc = B;
  if (r % 8) {
    Bsrc = static_cast<char*>(ws) + L.bpad;
    HIPTRY(timed(K_PAD, 0, 2.0 * d_out * L.r8 * eb, st, [&] {
      return launch_pad_cols(eb, B, const_cast<void*>(Bsrc), d_out, r, L.r8, st);
    }));
  }
  // W_out [d_out, d_in] = scale * B [d_out, r8] A [r, d_in] + W
  GemmArgs a = blank();
  a.a1 = Bsrc; a.lda1 = L.r8; a.b1 = A; a.ldb1 = d_in; a.K1 = r;
  a.m_load = d_out; a.m_store = d_out; a.n_load = d_in; a.n_store = d_in;
  a.c = W_out; a.ldc = d_in; a.cin = W; a.ldcin = d_in; a.alpha = scale;
  const double ko = double(d_out), ki = double(d_in), rr = double(r), e = double(eb);
  HIPTRY(gemm(dtype == LORA_F32 ? G_F32_NN_ADD : G_BF16_MED_NN_ADD, a, 1, st, 2 * ko * ki * rr,
              (2 * ko * ki + ko * rr + rr * ki) * e));
  return LORA_OK;
}

size_t lora_swiglu_workspace_bytes(int backward, int dtype, int64_t M, int64_t d_in,
                                   const lora_group_member* members) {
  if (dtype != LORA_F32 && dtype != LORA_BF16) return 0;
  if (!members) return 0;
  for (int g = 0; g < 2; ++g)
    if (check_sizes(M, d_in, members[g].d_out, members[g].r) != LORA_OK || members[g].d_out != members[0].d_out)
      return 0;
  return make_swiglu_layout(backward != 0, dtype, M, d_in, members).total;
}

int lora_swiglu_fwd(int dtype, int64_t M, int64_t d_in, const lora_group_member* members, const void* X,
                    const float* table16, void* H, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_swiglu(false, dtype, M, d_in, members, X, table16));
  if (M > 0) TRY(check_ptrs({H}));
  const SwigluLayout S = make_swiglu_layout(false, dtype, M, d_in, members);
  TRY(check_ws_bytes(S.total, ws, ws_bytes));
  TRY(check_device());
  return swiglu_forward(dtype, M, d_in, members, X, table16, H, ws, S, static_cast<hipStream_t>(stream));
}

int lora_swiglu_bwd(int dtype, int64_t M, int64_t d_in, const lora_group_member* members, const void* X,
                    const float* table16, const void* dH, const void* G, const void* U, void* dX, void* ws,
                    size_t ws_bytes, void* stream) {
  TRY(check_swiglu(true, dtype, M, d_in, members, X, table16));
  if (M > 0) TRY(check_ptrs({dH, G, U}));
  if (dX && !aligned16(dX)) return LORA_ERR_ALIGN;
  const SwigluLayout S = make_swiglu_layout(true, dtype, M, d_in, members);
  TRY(check_ws_bytes(S.total, ws, ws_bytes));
  TRY(check_device());
  return swiglu_backward(dtype, M, d_in, members, X, table16, dH, G, U, dX, ws, S,
                         static_cast<hipStream_t>(stream));
}

int lora_transpose(const void* src, int64_t rows, int64_t cols, void* dst, void* stream) {
  if (rows < 8 || cols < 8 || rows % 8 || cols % 8 || rows >= kMaxDim || cols >= kMaxDim) return LORA_ERR_SHAPE;
  TRY(check_ptrs({src, dst}));
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIPTRY(timed(K_TRANSPOSE_W, 0, 4.0 * rows * cols, st, [&] {
    return launch_transpose_tile(static_cast<const uint16_t*>(src), cols, rows, cols, static_cast<uint16_t*>(dst), rows,
                                 rows, st);
  }));
  return LORA_OK;
}

int lora_mfma_rate(int iters, int blocks, float* out, void* stream) {
  if (iters < 1 || blocks < 1) return LORA_ERR_SHAPE;
  TRY(check_ptrs({out}));
  TRY(check_device());
  HIPTRY(launch_mfma_rate(iters, blocks, out, static_cast<hipStream_t>(stream)));
  return LORA_OK;
}

int lora_profile_begin(int max_launches) {
  if (max_launches < 1) return LORA_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  const size_t want = 2 * size_t(max_launches);
  while (g_prof.ev.size() < want) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return LORA_ERR_DEVICE;
    g_prof.ev.push_back(e);
  }
  g_prof.ent.assign(size_t(max_launches), ProfEntry{-1, 0, 0});
  g_prof.n = 0;
  g_prof.on = true;
  return LORA_OK;
}

int lora_profile_end(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  return LORA_OK;
}

int lora_profile_only(int kind) {
  if (kind < -1 || kind >= K_PROF_COUNT) return LORA_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.only = kind;
  return LORA_OK;
}

int lora_profile_kinds(void) { return K_PROF_COUNT; }

int lora_set_nf4_fwd_path(int mode) {
  if (mode != LORA_NF4_PATH_AUTO && mode != LORA_NF4_PATH_DEQUANT && mode != LORA_NF4_PATH_LOAD_STAGE)
    return LORA_ERR_SHAPE;
  return g_nf4_fwd_path.exchange(mode);
}

const char* lora_profile_kind_name(int kind) { return kind_name(kind); }

int lora_profile_query(int kind, double* total_ms, int* count, double* total_flop, double* total_bytes) {
  if (!total_ms || !count || !total_flop || !total_bytes) return LORA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  double ms = 0, fl = 0, by = 0;
  int c = 0;
  for (size_t i = 0; i < g_prof.n; ++i) {
    if (g_prof.ent[i].kind != kind) continue;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) return LORA_ERR_DEVICE;
    ms += t;
    fl += g_prof.ent[i].flop;
    by += g_prof.ent[i].bytes;
    ++c;
  }
  *total_ms = ms;
  *count = c;
  *total_flop = fl;
  *total_bytes = by;
  return LORA_OK;
}

}  // extern "C"
