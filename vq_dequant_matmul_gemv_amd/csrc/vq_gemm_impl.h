#pragma once
// vq_gemm_impl.h -- prefill-shaped VQ matmul on fp16 MFMA (dense and grouped
// routed-expert): kernel templates and their host launchers, instantiated per
// code width by vq_gemm_b*.hip (vq_gemm.hip holds the routing that groups
// (token, slot) pairs by expert, and dispatches).
//
// What is computed: y[t][r] = sum_c W[r][c] * x[t][c] with
// W[r][c] = fp16(codebook[code][c % d] * scale[r][c / g]) exactly as the
// dequant defines it (paper "Data-Free Vector Quantization Beats Affine
// Quantization at Matched Bytes Below 5 Bits", §2.2 and §3.4: prefill runs a
// prefill-shaped path over the same codes; model card
// "Qwen3.5-397B-A17B-VQ-2.4bpw", Methodology, for the format), fp32
// accumulation in v_mfma_f32_32x32x16_f16.
//
// Design for gfx950:
//  * Per MFMA: x (32 tokens x 16 k) times dequantized W^T (16 k x 32 rows),
//    so each half-wave's results are 32 consecutive elements of a y row.
//    A block's waves sit side by side along W rows; a wave owns MB m-blocks
//    of 32 rows and all 32*NB tokens of the tile, so every weight is
//    dequantized exactly once per token tile, straight into the B-operand
//    registers (no LDS round trip for W).  Blocks are 8 waves (two per
//    SIMD) of 64 rows each; a tile is 512 rows x 128 tokens for large token
//    counts and 512 x 32 for small ones and routed experts.
//  * Scales are fetched in 16-byte windows of 8 groups per row, once per 8
//    groups, not 2 bytes per row per super-step.
//  * The contraction order over k is free, so each lane half (lanes 32h ..
//    32h+31) takes a contiguous run of CG columns per "super-step" (CG = 32
//    for d = 2, 64 for d = 4 and 8, and for d = 2 thin tiles whose columns
//    are a multiple of 128: half as many barriers and x stages per column): a lane's codes
//    for one super-step are one small contiguous load and its x slices are
//    contiguous.
//  * x tiles (32*NB tokens x 2*CG columns) go through LDS, double-buffered,
//    one barrier per super-step; token rows are padded by 16 bytes so the
//    16-byte fragment reads hit distinct banks.
//  * On the 128-token tiles (except d = 4 with 12-bit codes) the main loop
//    is phase-offset: clusters of 4 k-steps alternate a dequant phase and an
//    MFMA phase between block barriers, half the waves one phase behind, so
//    the two waves of a SIMD take turns on the MFMA pipe.
//  * Codebook in LDS (replicated for K = 256, as in the GEMV); the gathers of
//    the next k-step are issued ahead of the current k-step's MFMAs.
//  * Tiles of a last, partial round of the grid (or of a grid with fewer
//    tiles than CUs) are split along K over the CUs and their slices added
//    atomically into a zeroed y; the number of slices weighs the rounds
//    saved against the atomic traffic, which scales with the tokens per tile.
//  * Routed experts: the routing kernel counts pairs per expert, scans,
//    scatters pair ids by expert and emits a flat list of (expert, first,
//    count) token tiles; the GEMM walks that list with gathered x rows and
//    writes y[pair] rows directly.  All on the stream, no host sync.

#include "vq_device.h"
#include "vq_kernels.h"

#include <algorithm>
#include <cstdlib>
#include <mutex>

namespace vqmi {

namespace {

// Codes of one lane for one super-step: NCL codes of B bits starting at bit
// `bit` of the row.  When NCL * B is a multiple of 32 every such run is word
// aligned; otherwise the run is read with one extra word from the word that
// holds its first bit, and shifted into place (align_lane_codes) once the
// words have arrived: `sh` is the run's bit offset in that first word.
template <int NCL, int B>
struct LaneCodes {
  static constexpr bool kAligned = (NCL * B) % 32 == 0;
  static constexpr int kWords = (NCL * B + 31) / 32;           // after alignment
  static constexpr int kLoad = kAligned ? kWords : kWords + 1;  // as loaded
  uint32_t w[kLoad];
  uint32_t sh;
};

template <int NCL, int B>
__device__ __forceinline__ void align_lane_codes(LaneCodes<NCL, B>& c) {
  if constexpr (!LaneCodes<NCL, B>::kAligned) align_words<LaneCodes<NCL, B>::kLoad>(c.w, c.sh);
}

// The lane's run of codes starting at bit `bit` of the row whose codes start
// at byte `row_off` of the buffer.
template <int NCL, int B>
__device__ __forceinline__ void load_lane_codes(LaneCodes<NCL, B>& c, rsrc_t r, uint32_t row_off, uint32_t bit) {
  constexpr int W = LaneCodes<NCL, B>::kLoad;
  const uint32_t off = row_off == kOutOfRange ? kOutOfRange : row_off + (bit >> 5) * 4u;
  c.sh = bit & 31u;
  if constexpr (!kAlignedChunks<B>) {  // widths other than 8 and 12 bits
    load_words<W>(c.w, r, off);
  } else if constexpr (W % 4 == 0) {
#pragma unroll
    for (int q = 0; q < W / 4; ++q) {
      u32x4 v = buf_load_b128(r, off + 16u * q);
      c.w[4 * q] = v.x; c.w[4 * q + 1] = v.y; c.w[4 * q + 2] = v.z; c.w[4 * q + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    u32x2 v = buf_load_b64(r, off);
    c.w[0] = v.x; c.w[1] = v.y;
  } else if constexpr (W == 6) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      u32x2 v = buf_load_b64(r, off + 8u * q);
      c.w[2 * q] = v.x; c.w[2 * q + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int q = 0; q < W; ++q) c.w[q] = buf_load_b32(r, off + 4u * q);
  }
}

template <int NCL, int B>
__device__ __forceinline__ uint32_t lane_code(const LaneCodes<NCL, B>& c, int i) {
  constexpr uint32_t mask = (1u << B) - 1u;
  const int bit = i * B;
  const int wi = bit >> 5;
  const int sh = bit & 31;
  if (sh + B <= 32) return (c.w[wi] >> sh) & mask;
  return __builtin_amdgcn_alignbit(c.w[wi + 1], c.w[wi], sh) & mask;
}

// Entry of code i of the lane's run, from the codebook at cbp (LDS, or
// device memory for large codebooks).
template <int D, int B, int NCL>
__device__ __forceinline__ Entry<D> lane_gather(const uint8_t* cbp, const LaneCodes<NCL, B>& c,
                                                int i, uint32_t lane_off) {
  using L = CodebookLayout<D, B>;
  uint32_t off;
  if constexpr (L::kReplicated) {
    off = entry_offset_byte<D, B>(c.w[i >> 2], i & 3, lane_off);
  } else {
    off = lane_code<NCL, B>(c, i) * (uint32_t)L::kEntryBytes;
  }
  return lds_entry<D>(cbp, off);
}

}  // namespace

struct GemmArgs {
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  const uint16_t* x;
  void* y;                // element type y_kind; shape per epi
  const float* route_w;   // epi == combine: router weight per pair
  int x_bf16, y_kind, epi;  // IoSpec
  // routed experts
  const int32_t* tiles;   // [max_tiles][3]: expert, first (into pair list), count
  const int32_t* n_tiles; // device scalar
  const int32_t* pairs;   // pair ids grouped by expert
  int64_t code_estride, scale_estride, cb_estride;
  int rows, cols, wr, spr;
  int T;                  // dense tokens
  int top_k, x_per_slot;
  int x_rows;             // routed: rows of x (T or T*top_k)
  int n_row_tiles, n_tok_tiles;
  // routed: a unit is (tile, row tile); n_wide of the tiles (listed first)
  // hold 128 tokens, the rest 32.  moe_slots blocks are resident at once,
  // one per CU (0: the variant runs no row halves).
  const int32_t* n_wide;  // device scalar
  int moe_slots;
  // dense grid: blocks [0, n_full) each own a whole tile; the blocks after them
  // each own one of rem_split K slices of a remaining tile and add into y
  // (zeroed beforehand) atomically.
  int n_full, rem_split;
  // dense stack of n_stack experts sharing x: the row tiles of expert e follow
  // those of expert e - 1 (n_row_tiles counts them all) and token t's outputs
  // of expert e are y row t * n_stack + e
  int n_stack;
};

// Tile t -> (row tile, token tile): groups of 4 row tiles x all token tiles,
// so neighbouring tile indices share x and W slices.
__host__ __device__ __forceinline__ void gemm_tile_coords(int tile, int n_row_tiles, int n_tok_tiles, int& rt,
                                                          int& tt) {
  const int GR = 4;
  const int grp = tile / (GR * n_tok_tiles);
  const int in = tile - grp * GR * n_tok_tiles;
  const int rows_in_grp = min(GR, n_row_tiles - grp * GR);
  rt = grp * GR + in % rows_in_grp;
  tt = in / rows_in_grp;
}

// 32x32x16 fp16 MFMA, fp32 accumulation.  Operand lanes: lane l supplies row
// (A) / column (B) l % 32 and the 8 k-values of half h = l / 32; result lane
// l holds column l % 32, rows 8*(i/4) + 4*h + (i%4), i = 0..15.  Here A is an
// x fragment (32 tokens) and B a dequantized W fragment (32 rows).
__device__ __forceinline__ float16_t mfma32(half8_t a, half8_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Block shape: WAVES waves side by side along W rows, each owning MB m-blocks
// of 32 rows and all 32*NB tokens of the tile.
template <int WAVES, int MB, int NB>
struct GemmShape {
  static constexpr int kWaves = WAVES;
  static constexpr int kMB = MB;
  static constexpr int kNB = NB;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kRows = 32 * MB * WAVES;   // W rows per block tile
  static constexpr int kTokens = 32 * NB;         // tokens per block tile
};

// Columns per lane half per super-step (a super-step is twice that): 64 for
// d = 4 and 8, whose rows are multiples of 128 (256) columns; for d = 2 (rows
// multiples of 64) 32, or 64 in the wide variant, which the host picks for
// thin tiles when the columns are a multiple of 128.
__host__ __device__ constexpr int gemm_cg(int D, bool wide) { return (D >= 4 || wide) ? 64 : 32; }

// 16-bit element `pos` (0..7) of a 16-byte window.
__device__ __forceinline__ uint32_t pick16(u32x4 v, int pos) {
  const uint32_t lo = (pos & 2) ? v.y : v.x;
  const uint32_t hi = (pos & 2) ? v.w : v.z;
  const uint32_t d = (pos & 4) ? hi : lo;
  return (pos & 1) ? d >> 16 : d & 0xffffu;
}

// Phase-offset main loop on the 128-token tiles, in clusters of
// kGemmCluster k-steps (see the kernel).
constexpr bool kGemmPhaseOffset = true;
constexpr int kGemmCluster = 4;

// LDS bytes of a tile shape's two x stages [2][tokens][row bytes + 16].
__host__ __device__ constexpr int gemm_xbuf_bytes(int D, bool wide, int tokens) {
  return 2 * tokens * (2 * gemm_cg(D, wide) * 2 + 16);
}

// Dense GEMM: one tile (or one K slice of one) per block.
template <int D, int B, int G, class SH, bool WIDE>
__global__ __launch_bounds__(SH::kThreads, 1) void vq_gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t cb_lds[CodebookLayout<D, B>::kBytes];
  __shared__ __align__(16) uint8_t xbuf[gemm_xbuf_bytes(D, WIDE, SH::kTokens)];
  const int bid = blockIdx.x;
  int tile, kslice = 0, nslices = 1;
  if (bid < a.n_full) {
    // XCD-aware order: blocks land on XCD (bid % 8) round-robin; give each
    // XCD a contiguous range of tiles so concurrently running blocks share
    // x and W slices in that XCD's L2.
    const int N = a.n_full;
    const int q = N / 8, r8 = N % 8, xcd = bid % 8, j = bid / 8;
    tile = xcd * q + min(xcd, r8) + j;
  } else {
    const int u = bid - a.n_full;
    tile = a.n_full + u / a.rem_split;
    kslice = u % a.rem_split;
    nslices = a.rem_split;
  }
  int rt, tt;
  gemm_tile_coords(tile, a.n_row_tiles, a.n_tok_tiles, rt, tt);
  const int nrt_e = a.n_row_tiles / a.n_stack;  // row tiles per expert of a stack
  const int expert = rt / nrt_e;
  rt -= expert * nrt_e;
  const int tok_base = tt * SH::kTokens;
  const int count = min(SH::kTokens, a.T - tok_base);
  using TS = SH;
  constexpr bool MOE = false, TW = WIDE;
  constexpr int first = 0;
#include "vq_gemm_tile.inc"
}

// Whether the routed kernel runs a short last round as row halves: only
// where its LDS (codebook stage and x stages) keeps a second block off the
// CU (more than half of the CU's 160 KiB).  Where two blocks share a CU, a
// short last round already runs beside the round before it.
template <int D, int B, bool WIDE, bool MIX>
__host__ __device__ constexpr bool moe_halves() {
  const int xb = gemm_xbuf_bytes(D, WIDE, kMoeTileTokens);
  const int xbw = MIX ? gemm_xbuf_bytes(D, false, kMoeWideTokens) : 0;
  return CodebookLayout<D, B>::kBytes + (xb > xbw ? xb : xbw) > 80 * 1024;
}

// Routed (grouped) GEMM over the routing kernel's tile list, one unit (tile,
// row tile of SH::kRows) per block, in list order: the 128-token tiles of hot
// experts (MIX only; the routing kernel lists them first, so they start in
// the first round), then the 32-token tiles.  The list's length is known only
// here, on the device: when the last round of units (in 32-token-tile time,
// a 128-token tile counting two) would fill at most half the resident
// blocks, its units run as two halves of SH::kRows / 2 rows each, finishing
// in about half the time.  Blocks past the units exit.
template <int D, int B, int G, class SH, bool WIDE, bool MIX>
__global__ __launch_bounds__(SH::kThreads, 1) void vq_moe_gemm_kernel(GemmArgs a) {
  using SW = GemmShape<SH::kWaves, SH::kMB, 4>;               // 128-token tiles
  using SHALF = GemmShape<SH::kWaves, SH::kMB / 2, SH::kNB>;  // half units
  static_assert(SH::kNB == 1 && SH::kMB % 2 == 0, "32-token tiles with whole row halves");
  constexpr int XB = gemm_xbuf_bytes(D, WIDE, SH::kTokens);
  constexpr int XBW = MIX ? gemm_xbuf_bytes(D, false, SW::kTokens) : 0;
  constexpr int XBYTES = XB > XBW ? XB : XBW;
  static_assert(moe_halves<D, B, WIDE, MIX>() == (CodebookLayout<D, B>::kBytes + XBYTES > 80 * 1024),
                "row halves exactly where a block's LDS keeps a second block off its CU");
  __shared__ __align__(16) uint8_t cb_lds[CodebookLayout<D, B>::kBytes];
  __shared__ __align__(16) uint8_t xbuf[XBYTES];
  const int nrt = a.n_row_tiles;
  const int n_wide = MIX ? *a.n_wide : 0;
  const int n_units = *a.n_tiles * nrt;
  const int wide_units = n_wide * nrt;
  const int thin_units = n_units - wide_units;
  const int rem = a.moe_slots > 0 ? (2 * wide_units + thin_units) % a.moe_slots : 0;
  const int split = 2 * rem <= a.moe_slots ? min(rem, thin_units) : 0;
  const int whole = n_units - split;
  const int b = blockIdx.x;
  int u, hsel = -1;
  if (b < whole) {
    u = b;
  } else if (b < whole + 2 * split) {
    u = whole + ((b - whole) >> 1);
    hsel = (b - whole) & 1;
  } else {
    return;
  }
  const int tix = u / nrt;
  const int urt = u - tix * nrt;
  const int expert = a.tiles[3 * tix + 0];
  const int first = a.tiles[3 * tix + 1];
  const int count = a.tiles[3 * tix + 2];
  constexpr bool MOE = true;
  constexpr int tok_base = 0, kslice = 0, nslices = 1;
  if (MIX && tix < n_wide) {
    if constexpr (MIX) {
      using TS = SW;
      constexpr bool TW = false;
      const int rt = urt;
#include "vq_gemm_tile.inc"
    }
  } else if (hsel >= 0) {
    if constexpr (moe_halves<D, B, WIDE, MIX>()) {
      using TS = SHALF;
      constexpr bool TW = WIDE;
      const int rt = 2 * urt + hsel;
      if (rt * TS::kRows >= a.rows) return;
#include "vq_gemm_tile.inc"
    }
  } else {
    using TS = SH;
    constexpr bool TW = WIDE;
    const int rt = urt;
#include "vq_gemm_tile.inc"
  }
}

// Zero the y region of tiles [first, first + gridDim.x), gridDim.y blocks per
// tile, 16-byte stores where the rows allow (a kernel rather than
// hipMemsetAsync, so it can sit in a graph).  Tiles and y rows of a stack of
// n_stack experts as in the dense kernel.
static __global__ __launch_bounds__(256) void vq_zero_tiles_kernel(float* y, int rows, int T, int first, int n_row_tiles,
                                                            int n_tok_tiles, int tile_rows, int tile_tokens,
                                                            int n_stack) {
  int rt, tt;
  gemm_tile_coords(first + (int)blockIdx.x, n_row_tiles, n_tok_tiles, rt, tt);
  const int nrt_e = n_row_tiles / n_stack;
  const int e = rt / nrt_e;
  rt -= e * nrt_e;
  const int r0 = rt * tile_rows, nr = min(tile_rows, rows - r0);
  const int t0 = tt * tile_tokens, nt = min(tile_tokens, T - t0);
  const bool vec = (rows & 3) == 0;  // r0 is a multiple of tile_rows (of 32)
  const int per_row = vec ? (nr + 3) / 4 : nr;
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < nt * per_row; i += gridDim.y * blockDim.x) {
    const int t = i / per_row, k = i - t * per_row;
    float* yr = y + ((int64_t)(t0 + t) * n_stack + e) * rows + r0;
    if (vec && 4 * k + 3 < nr) {
      *reinterpret_cast<float4_t*>(yr + 4 * k) = float4_t{0.f, 0.f, 0.f, 0.f};
    } else if (vec) {
      for (int c = 4 * k; c < nr; ++c) yr[c] = 0.f;
    } else {
      yr[k] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

namespace {

using GemmSmallT = GemmShape<8, 2, 1>;  // 512 rows x 32 tokens, two waves per SIMD
using GemmLargeT = GemmShape<8, 2, 4>;  // 512 rows x 128 tokens
using GemmMoe = GemmShape<8, 2, 1>;     // 512 rows x 32 tokens: routed experts mostly get a
                                        // few tokens, so thin tiles waste the least MFMA work
static_assert(GemmMoe::kTokens == kMoeTileTokens && 4 * GemmMoe::kTokens == kMoeWideTokens,
              "routing tiles match the grouped GEMM's token tiles");

// d = 2 thin tiles (32 tokens) take 128-column super-steps when the columns
// allow: half the barriers and x stages per column, 6-10 % faster there; the
// 128-token tiles gain about 1 % and keep 64.
template <int D, class SH>
bool gemm_wide(int cols) { return D == 2 && SH::kTokens <= 32 && cols % 128 == 0; }

template <int D, int B, int G, class SH>
hipError_t gemm_launch(const GemmArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (D == 2 && SH::kTokens <= 32) {
    if (gemm_wide<D, SH>(a.cols)) {
      hipLaunchKernelGGL((vq_gemm_kernel<D, B, G, SH, true>), grid, dim3(SH::kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((vq_gemm_kernel<D, B, G, SH, false>), grid, dim3(SH::kThreads), 0, s, a);
  return hipGetLastError();
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

GemmArgs base_args(const TensorView& w, const IoSpec& io, const void* x, void* y, int G, int D, int B) {
  GemmArgs a{};
  a.codes = w.codes;
  a.codebook = w.codebook;
  a.scales = w.scales;
  a.x = static_cast<const uint16_t*>(x);
  a.y = y;
  a.route_w = io.route_w;
  a.x_bf16 = io.x_bf16;
  a.y_kind = io.y_kind;
  a.epi = io.epi;
  a.code_estride = (int64_t)w.rows * w.wr;
  a.scale_estride = (int64_t)w.rows * (w.cols / G);
  a.cb_estride = w.cb_per_expert ? (int64_t)(1 << B) * D : 0;
  a.rows = w.rows;
  a.cols = w.cols;
  a.wr = w.wr;
  a.spr = w.cols / G;
  a.n_full = 0;
  a.rem_split = 1;
  a.n_stack = 1;
  return a;
}

// Time model of a dense call, fitted to calls measured on MI355X (17408x5120
// and 5120x17408, d = 2 and 4, T = 64 ... 1024, every split of 1 ... 6): a
// tile over the whole K costs 3 us plus, per column, 0.0095 us (32-token
// tiles, d = 4 and 8), 0.0147 us (32-token, d = 2), 0.0200 us (128-token, d =
// 4 and 8) or 0.0240 us (128-token, d = 2); whole rounds of tiles run one
// after another; the K slices of a last, partial round add every sum into a
// zeroed y with fp32 atomics, ~4 ps per add, plus ~5 us for the zeroing
// launch.  The atomic adds are what a flat per-slice charge missed: at T =
// 512 (17408x5120 d = 4, 136 tiles of 128 tokens) three slices took 164 us,
// one 113 us.
struct GemmPlan {
  int split;
  double us;
};

inline double gemm_tile_us(bool thin, int D, int cols) {
  const double per_col = thin ? (D == 2 ? 0.0147 : 0.0095) : (D == 2 ? 0.0240 : 0.0200);
  return 3.0 + per_col * cols;
}

// Best K split of the last partial round for tiles of `rows_t` rows x
// `tok_t` tokens (split 1 when the output cannot take atomic adds).
inline GemmPlan gemm_plan(int T, int rows, int cols, int D, bool thin, int rows_t, int tok_t, int cus,
                          bool split_ok, int n_stack) {
  const int n_row_tiles = n_stack * ((rows + rows_t - 1) / rows_t);
  const int n_tok_tiles = (T + tok_t - 1) / tok_t;
  const int tiles = n_row_tiles * n_tok_tiles;
  const double t_tile = gemm_tile_us(thin, D, cols);
  const int full = (tiles / cus) * cus, rem = tiles - full;
  GemmPlan best{1, (double)((tiles + cus - 1) / cus) * t_tile};
  if (rem == 0 || !split_ok) return best;
  // each K slice keeps at least 512 columns (1024 for d = 8)
  const int max_split = std::max(1, cols / (D == 8 ? 1024 : 512));
  const double rem_outputs = (double)rem / tiles * (double)T * rows * n_stack;  // outputs of the split tiles
  for (int sp = 2; sp <= std::min(32, max_split); ++sp) {
    const double us = (double)(full / cus) * t_tile + (double)((rem * sp + cus - 1) / cus) * t_tile / sp + 5.0 +
                      4e-6 * rem_outputs * sp;
    if (us < best.us - 1e-9) best = GemmPlan{sp, us};
  }
  return best;
}

// Whole rounds of tiles run as whole tiles; with split > 1, the tiles of a
// last, partial round are split along K over the CUs and added atomically
// into a zeroed y (their fp32 addition order then varies between runs).
template <int D, int B, int G, class SH>
hipError_t gemm_dense(GemmArgs a, int split, hipStream_t s) {
  a.n_row_tiles = a.n_stack * ((a.rows + SH::kRows - 1) / SH::kRows);
  a.n_tok_tiles = (a.T + SH::kTokens - 1) / SH::kTokens;
  const int tiles = a.n_row_tiles * a.n_tok_tiles;
  const int cus = num_cus();
  int full = (tiles / cus) * cus, rem = tiles - full;
  if (split <= 1 || rem == 0) {
    split = 1;
    full = tiles;
    rem = 0;
  }
  a.n_full = full;
  a.rem_split = split;
  if (rem > 0) {
    hipLaunchKernelGGL(vq_zero_tiles_kernel, dim3(rem, std::max(1, 2 * cus / rem)), dim3(256), 0, s,
                       static_cast<float*>(a.y), a.rows,
                       a.T, full, a.n_row_tiles, a.n_tok_tiles, SH::kRows, SH::kTokens, a.n_stack);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return gemm_launch<D, B, G, SH>(a, dim3((unsigned)(full + rem * split)), s);
}

// Up to 32 tokens the 32-token tiles; above, the tile shape and split the
// time model rates faster (32-token tiles keep winning up to a few hundred
// tokens: 17408x5120 d = 4 at T = 64 / 128 / 256 in 36 / 52 / 77 us against
// 49 / 62 / 86 us for the best split of 128-token tiles).
// The environment variable VQMI_GEMM_TILE = 32 or 128 forces a tile shape
// (the split still by the model), so each shape can be tested at sizes where
// the model would take the other.
template <int D, int B, int G>
hipError_t gemm_geom(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) {
  GemmArgs a = base_args(w, io, x, y, G, D, B);
  a.T = T;
  a.n_stack = w.num_experts;  // a stack: every expert times the same x
  const int cus = num_cus();
  const bool split_ok = io.epi == kEpiNone && io.y_kind == kOutF32;  // K slices add fp32 sums
  const char* force = getenv("VQMI_GEMM_TILE");
  const int forced = force ? atoi(force) : 0;
  const GemmPlan thin = gemm_plan(T, w.rows, w.cols, D, true, GemmSmallT::kRows, GemmSmallT::kTokens, cus, split_ok,
                                  a.n_stack);
  const GemmPlan large = gemm_plan(T, w.rows, w.cols, D, false, GemmLargeT::kRows, GemmLargeT::kTokens, cus,
                                   split_ok, a.n_stack);
  if (forced == GemmLargeT::kTokens) return gemm_dense<D, B, G, GemmLargeT>(a, large.split, s);
  if (forced == GemmSmallT::kTokens || T <= GemmSmallT::kTokens || thin.us < large.us)
    return gemm_dense<D, B, G, GemmSmallT>(a, thin.split, s);
  return gemm_dense<D, B, G, GemmLargeT>(a, large.split, s);
}

// The routed kernel variant (32-token tiles with 128-column super-steps for
// d = 2; MIX: 128-token tiles too), launched over max_units whole units plus
// room for the halves of a last round where the variant runs them.
template <int D, int B, int G, bool WIDE, bool MIX>
hipError_t moe_launch(GemmArgs a, int max_units, hipStream_t s) {
  a.moe_slots = moe_halves<D, B, WIDE, MIX>() ? num_cus() : 0;
  hipLaunchKernelGGL((vq_moe_gemm_kernel<D, B, G, GemmMoe, WIDE, MIX>), dim3((unsigned)(max_units + a.moe_slots / 2)),
                     dim3(GemmMoe::kThreads), 0, s, a);
  return hipGetLastError();
}

// Route the pairs, then the grouped GEMM over the tile list the routing
// kernel left in the workspace.  128-token tiles for hot experts pay when
// the 32-token units alone would take at least kMoeWideRounds rounds of the
// GPU even if every expert's pairs filled whole tiles: a 128-token tile
// takes about twice a 32-token one, so in shorter runs it would outlast
// the rest of the schedule.
constexpr int kMoeWideRounds = 2;

template <int D, int B, int G>
hipError_t moe_gemm_geom(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot, const int32_t* ids,
                         int T, int top_k, void* y, int32_t* ws, hipStream_t s) {
  const int npairs = T * top_k;
  const int E = w.num_experts;
  GemmArgs a = base_args(w, io, x, y, G, D, B);
  a.tiles = moe_ws_tiles(ws, E, npairs);
  a.n_tiles = moe_ws_n_tiles(ws, E);
  a.n_wide = moe_ws_n_wide(ws, E);
  a.pairs = moe_ws_pairs(ws, E);
  a.top_k = top_k;
  a.x_per_slot = x_per_slot;
  a.x_rows = x_per_slot ? npairs : T;
  a.n_row_tiles = (a.rows + GemmMoe::kRows - 1) / GemmMoe::kRows;
  const int64_t min_units = (int64_t)((npairs + kMoeTileTokens - 1) / kMoeTileTokens) * a.n_row_tiles;
  const bool mix = min_units >= (int64_t)kMoeWideRounds * num_cus();
  void* y_skip = io.epi == kEpiCombine ? nullptr : y;  // combine: skipped slots add nothing
  const int y_row_halves = (io.epi == kEpiSwiglu ? w.rows / 2 : w.rows) * (io.y_kind == kOutF32 ? 2 : 1);
  hipError_t e = launch_route(ids, npairs, E, ws, y_skip, y_row_halves, mix, s);
  if (e != hipSuccess) return e;
  const int max_units = moe_max_tiles(npairs, E) * a.n_row_tiles;
  const bool wide = gemm_wide<D, GemmMoe>(a.cols);
  if (mix) return wide ? moe_launch<D, B, G, true, true>(a, max_units, s) : moe_launch<D, B, G, false, true>(a, max_units, s);
  return wide ? moe_launch<D, B, G, true, false>(a, max_units, s) : moe_launch<D, B, G, false, false>(a, max_units, s);
}

}  // namespace

// Every (d, group) of one code width B.
template <int B>
hipError_t gemm_bits(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) {
#define X(D, G) \
  if (w.d == D && w.group == G) return gemm_geom<D, B, G>(w, io, x, T, y, s);
  X(2, 64) X(2, 128) X(4, 64) X(4, 128) X(8, 64) X(8, 128)
#undef X
  return hipErrorInvalidValue;
}

template <int B>
hipError_t moe_gemm_bits(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot, const int32_t* ids,
                         int T, int top_k, void* y, int32_t* ws, hipStream_t s) {
#define X(D, G) \
  if (w.d == D && w.group == G) return moe_gemm_geom<D, B, G>(w, io, x, x_per_slot, ids, T, top_k, y, ws, s);
  X(2, 64) X(2, 128) X(4, 64) X(4, 128) X(8, 64) X(8, 128)
#undef X
  return hipErrorInvalidValue;
}

// The entry points of one code width's translation unit (vq_gemm_bNN.hip).
#define VQMI_GEMM_UNIT(B)                                                                                    \
  hipError_t gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) { \
    return gemm_bits<B>(w, io, x, T, y, s);                                                                  \
  }                                                                                                          \
  hipError_t moe_gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot,           \
                           const int32_t* ids, int T, int top_k, void* y, int32_t* ws, hipStream_t s) {     \
    return moe_gemm_bits<B>(w, io, x, x_per_slot, ids, T, top_k, y, ws, s);                                  \
  }

}  // namespace vqmi
