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
  // dense grid: blocks [0, n_full) each own a whole tile; the blocks after them
  // each own one of rem_split K slices of a remaining tile and add into y
  // (zeroed beforehand) atomically.
  int n_full, rem_split;
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

template <int D, int B, int G, class SH, bool MOE, bool WIDE>
__global__ __launch_bounds__(SH::kThreads, 1) void vq_gemm_kernel(GemmArgs a) {
  using L = CodebookLayout<D, B>;
  constexpr int CG = gemm_cg(D, WIDE);    // columns per lane half per super-step
  constexpr int S = CG / 8;               // k-steps of 16 (8 per half) per super-step
  constexpr int NCL = CG / D;             // codes per lane per super-step
  constexpr int SS = 2 * CG;              // columns per super-step
  constexpr int MB = SH::kMB;
  constexpr int NB = SH::kNB;
  constexpr int WN = SH::kTokens;
  constexpr int XROW = SS * 2 + 16;       // LDS bytes per token row (padded)
  constexpr int SEGS = SS / 8;            // 16-byte segments per token row
  constexpr int NT = SH::kThreads;
  constexpr int XLD = (WN * SEGS + NT - 1) / NT;  // x segments per thread per super-step
  constexpr int CPA = 8 / D;              // codebook entries per A fragment (8 columns)

  // Static LDS: codebook, then the two x tiles [2][WN][XROW].
  __shared__ __align__(16) uint8_t cb_lds[L::kBytes];
  __shared__ __align__(16) uint8_t xbuf[2 * WN * XROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // ---- which tile ----
  int rt, expert = 0, first = 0, count;
  int tok_base = 0;
  int kslice = 0, nslices = 1;  // this block's share of the tile's K range
  if constexpr (MOE) {
    const int tix = blockIdx.x;
    if (tix >= *a.n_tiles) return;
    expert = a.tiles[3 * tix + 0];
    first = a.tiles[3 * tix + 1];
    count = a.tiles[3 * tix + 2];
    rt = blockIdx.y;
  } else {
    const int bid = blockIdx.x;
    int tile;
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
    int tt;
    gemm_tile_coords(tile, a.n_row_tiles, a.n_tok_tiles, rt, tt);
    tok_base = tt * WN;
    count = min(WN, a.T - tok_base);
  }

  const uint32_t* codes = a.codes + (int64_t)expert * a.code_estride;
  const uint16_t* scales = a.scales + (int64_t)expert * a.scale_estride;
  const uint16_t* cb = a.codebook + (int64_t)expert * a.cb_estride;
  // codebook entries: staged in LDS, or read from device memory (large codebooks)
  const uint8_t* cbp;
  if constexpr (L::kGlobal) cbp = reinterpret_cast<const uint8_t*>(cb);
  else cbp = cb_lds;

  // K range (super-steps) of this block.
  const int nks_all = (a.cols + SS - 1) / SS;
  int ks_begin = 0, ks_end = nks_all;
  if constexpr (!MOE) {
    ks_begin = (int)((int64_t)nks_all * kslice / nslices);
    ks_end = (int)((int64_t)nks_all * (kslice + 1) / nslices);
  }

  // All streaming loads are branch-free buffer loads with 32-bit offsets:
  // tokens past the tile's count, rows past the end and super-steps past
  // ks_end get an out-of-range offset and read zeros.

  // ---- x: XLD segments of 16 bytes per thread per super-step ----
  rsrc_t rx;
  if constexpr (MOE) {
    rx = make_rsrc(a.x, (uint64_t)a.x_rows * a.cols * 2);
  } else {
    rx = make_rsrc(a.x + (int64_t)tok_base * a.cols, (uint64_t)count * a.cols * 2);
  }
  uint32_t xoff[XLD];
  int xdst[XLD];
#pragma unroll
  for (int i = 0; i < XLD; ++i) {
    const int gs = tid + i * NT;
    const int tok = gs / SEGS;
    const int seg = gs % SEGS;
    xdst[i] = gs < WN * SEGS ? tok * XROW + seg * 16 : -1;
    uint32_t row;
    if constexpr (MOE) {
      const int pair = tok < count ? a.pairs[first + tok] : 0;
      row = (uint32_t)(a.x_per_slot ? pair : pair / a.top_k);
    } else {
      row = (uint32_t)tok;
    }
    xoff[i] = (gs < WN * SEGS && tok < count) ? row * (uint32_t)a.cols * 2u + (uint32_t)seg * 16u : kOutOfRange;
  }

  // ---- A: this wave's 32*MB rows, lane row l32 of each m-block ----
  const int row_base = rt * SH::kRows + wave * 32 * MB;
  const rsrc_t rc = make_rsrc(codes, (uint64_t)a.rows * a.wr * 4);
  const rsrc_t rs = make_rsrc(scales, (uint64_t)a.rows * a.spr * 2);
  uint32_t coff[MB], soff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint32_t r = (uint32_t)(row_base + mb * 32 + l32);  // past the end: reads zeros
    coff[mb] = r * (uint32_t)a.wr * 4u;
    soff[mb] = r * (uint32_t)a.spr * 2u;
  }

  auto load_x = [&](int ks, u32x4 (&xr)[XLD]) {
    const bool live = ks < ks_end;
#pragma unroll
    for (int i = 0; i < XLD; ++i) xr[i] = buf_load_b128(rx, live ? xoff[i] + (uint32_t)ks * SS * 2u : kOutOfRange);
  };
  const bool x_bf16 = a.x_bf16 != 0;  // bf16 x: converted to fp16 on its way into LDS
  auto store_x = [&](int buf, const u32x4 (&xr)[XLD]) {
#pragma unroll
    for (int i = 0; i < XLD; ++i)
      if (xdst[i] >= 0)
        *reinterpret_cast<u32x4*>(xbuf + buf * (WN * XROW) + xdst[i]) = x_bf16 ? bf16x8_to_f16x8(xr[i]) : xr[i];
  };
  // Scales come in 16-byte windows of 8 groups per row (one load per lane
  // per 8 groups instead of one per super-step; a row's scales are used a
  // few bytes per super-step, so per-step loads would fetch a cache line per
  // row for 2 bytes).  The window of the next group range is fetched one
  // super-step before it is needed.  Rows whose scale runs are not 16-byte
  // aligned fill the window with 2-byte loads.  Every group of a super-step
  // lies in one window for both lane halves (8 groups span >= 512 columns).
  const bool sw_aligned = (a.spr & 7) == 0;
  u32x4 swc[MB], swp[MB];
  auto load_window = [&](int w, u32x4 (&dst)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint32_t off = soff[mb] + (uint32_t)w * 16u;
      if (sw_aligned) {
        dst[mb] = buf_load_b128(rs, off);
      } else {
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = (uint32_t)buf_load_b16(rs, off + 4u * q) | ((uint32_t)buf_load_b16(rs, off + 4u * q + 2u) << 16);
        dst[mb] = u32x4{v[0], v[1], v[2], v[3]};
      }
    }
  };
  auto window_of = [&](int ks) { return (ks * SS / G) >> 3; };
  auto load_codes = [&](int ks, LaneCodes<NCL, B> (&cc)[MB], uint16_t (&sc)[MB]) {
    const bool ok = ks < ks_end;
    const uint32_t bit = (uint32_t)(ks * 2 * NCL + h * NCL) * B;  // the lane's first code, in bits of the row
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) load_lane_codes<NCL, B>(cc[mb], rc, ok ? coff[mb] : kOutOfRange, bit);
    const int w = window_of(ks);
    if (ks == ks_begin) {
      load_window(w, swc);
    } else if (w != window_of(ks - 1)) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) swc[mb] = swp[mb];
    }
    if (window_of(ks + 1) != w) load_window(w + 1, swp);
    const int pos = ((ks * SS + h * CG) / G) & 7;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sc[mb] = (uint16_t)pick16(swc[mb], pos);
  };

  const uint32_t lane_off = lane_copy_offset<D, B>(lane);
  float16_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  // One super-step: dequantize the A fragments of each m-block straight into
  // registers and run the MFMAs against the x tile in LDS buffer `buf`.  The
  // codebook gathers of k-step s + 1 are issued before the arithmetic of
  // k-step s, so their LDS latency overlaps the MFMAs.  Every super-step is
  // whole: the API requires cols % (32 d) == 0 and SS divides 32 d (the wide
  // d = 2 variant runs only when cols % 128 == 0).
  auto compute = [&](int buf, const LaneCodes<NCL, B> (&cc_in)[MB], const uint16_t (&sc)[MB]) {
    LaneCodes<NCL, B> cc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      cc[mb] = cc_in[mb];
      align_lane_codes<NCL, B>(cc[mb]);  // widths whose runs are not word aligned
    }
    const uint8_t* xb = xbuf + buf * (WN * XROW);
    half2_t s2[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s2[mb] = as_half2((uint32_t)sc[mb] * 0x10001u);
    Entry<D> e[2][MB][CPA];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c = 0; c < CPA; ++c) e[0][mb][c] = lane_gather<D, B, NCL>(cbp, cc[mb], c, lane_off);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s + 1 < S) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int c = 0; c < CPA; ++c)
            e[(s + 1) & 1][mb][c] = lane_gather<D, B, NCL>(cbp, cc[mb], (s + 1) * CPA + c, lane_off);
      }
      half8_t bf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bf[nb] = *reinterpret_cast<const half8_t*>(xb + (nb * 32 + l32) * XROW + (h * CG + 8 * s) * 2);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        half2_t w[4];
#pragma unroll
        for (int c = 0; c < CPA; ++c)
#pragma unroll
          for (int j = 0; j < D / 2; ++j) w[c * (D / 2) + j] = e[s & 1][mb][c].v[j] * s2[mb];
        const half8_t af = half8_t{w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(bf[nb], af, acc[mb][nb]);
      }
    }
  };

  // Ping-pong over two register sets (A, B) and two LDS x buffers (0, 1):
  // the loads for super-step ks + 1 are issued before super-step ks is
  // computed.  No register copies and no exit in the middle of the loop body
  // (the second half is skipped by a uniform branch on an odd count), so the
  // accumulators stay in place and the prefetch stays in flight.
  u32x4 xr[XLD];
  LaneCodes<NCL, B> ccA[MB], ccB[MB];
  uint16_t scA[MB], scB[MB];

  load_x(ks_begin, xr);
  load_codes(ks_begin, ccA, scA);
  stage_codebook<D, B>(cb_lds, cb, tid, NT);
  store_x(0, xr);
  __syncthreads();

  if constexpr (kGemmPhaseOffset && NB >= 4 && (D == 2 || (D == 4 && B == 8) || D == 8) && LaneCodes<NCL, B>::kAligned &&
                !L::kGlobal) {
    // Phase-offset schedule for the 128-token tiles.  A super-step runs as
    // clusters of KC k-steps, each split into a dequant phase (codebook
    // gathers and fp16 multiplies for the cluster's W fragments, kept in
    // registers) and an MFMA phase (x fragments from LDS, KC * MB * NB
    // MFMAs), separated by block barriers.  The upper half of the waves
    // enters one phase late, so on every SIMD (waves w and w + 4 share one)
    // one wave runs its MFMAs while the other dequantizes.  Every wave passes
    // the same number of barriers: the late half one extra at the start, the
    // early half one at the end.  The MFMA phase runs at raised wave
    // priority, so the SIMD's issue slots go to the MFMAs first.  Not used
    // for d = 4 with 12-bit codes, where a cluster's fragments spill
    // registers.
    constexpr int KC = kGemmCluster < S ? kGemmCluster : S;
    static_assert(S % KC == 0, "clusters tile the super-step");
    const bool late = wave >= SH::kWaves / 2;
    auto phase_sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // x of the next super-step is stored at the end of this super-step's
    // last MFMA phase, behind a barrier that waits for it: the last reads of
    // that buffer (the super-step before) end at least two barriers earlier,
    // and the first reads of the new x (the next super-step's first MFMA
    // phase) come at least one barrier later for both halves.
    // The next super-step's x stage travels in NCLU parts, one per cluster:
    // part p is loaded at the start of cluster p's dequant phase and written
    // to LDS at the end of its MFMA phase (the buffer's last reads end before
    // the first part is written, and the barrier ending the super-step waits
    // for every part's stores), so only one part occupies registers.
    constexpr int NCLU = S / KC;
    static_assert(XLD % NCLU == 0, "x segments split evenly over the clusters");
    constexpr int XP = XLD / NCLU;
    auto load_xp = [&](int ks, int p, u32x4 (&q)[XP]) {
      const bool live = ks < ks_end;
#pragma unroll
      for (int i = 0; i < XP; ++i)
        q[i] = buf_load_b128(rx, live ? xoff[p * XP + i] + (uint32_t)ks * SS * 2u : kOutOfRange);
    };
    auto store_xp = [&](int buf, int p, const u32x4 (&q)[XP]) {
#pragma unroll
      for (int i = 0; i < XP; ++i)
        if (xdst[p * XP + i] >= 0)
          *reinterpret_cast<u32x4*>(xbuf + buf * (WN * XROW) + xdst[p * XP + i]) =
              x_bf16 ? bf16x8_to_f16x8(q[i]) : q[i];
    };
    auto super_step = [&](int ks, int buf, const LaneCodes<NCL, B> (&cc)[MB], const uint16_t (&sc)[MB],
                          LaneCodes<NCL, B> (&ccn)[MB], uint16_t (&scn)[MB]) {
      u32x4 xq[XP];
      load_xp(ks + 1, 0, xq);
      load_codes(ks + 1, ccn, scn);
      const uint8_t* xb = xbuf + buf * (WN * XROW);
      half2_t s2[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) s2[mb] = as_half2((uint32_t)sc[mb] * 0x10001u);
#pragma unroll
      for (int s0 = 0; s0 < S; s0 += KC) {
        if (s0 > 0) load_xp(ks + 1, s0 / KC, xq);
        half8_t af[KC][MB];
        Entry<D> e[KC][MB][CPA];
#pragma unroll
        for (int k = 0; k < KC; ++k)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int c = 0; c < CPA; ++c)
              e[k][mb][c] = lane_gather<D, B, NCL>(cbp, cc[mb], (s0 + k) * CPA + c, lane_off);
#pragma unroll
        for (int k = 0; k < KC; ++k)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            half2_t w[4];
#pragma unroll
            for (int c = 0; c < CPA; ++c)
#pragma unroll
              for (int j = 0; j < D / 2; ++j) w[c * (D / 2) + j] = e[k][mb][c].v[j] * s2[mb];
            af[k][mb] = half8_t{w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
          }
        phase_sync();
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          half8_t bf[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            bf[nb] = *reinterpret_cast<const half8_t*>(xb + (nb * 32 + l32) * XROW + (h * CG + 8 * (s0 + k)) * 2);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(bf[nb], af[k][mb], acc[mb][nb]);
        }
        __builtin_amdgcn_s_setprio(0);
        store_xp(buf ^ 1, s0 / KC, xq);
        if (s0 + KC == S) {
          __builtin_amdgcn_sched_barrier(0);
          lds_barrier();
          __builtin_amdgcn_sched_barrier(0);
        } else {
          phase_sync();
        }
      }
    };
    if (late) phase_sync();
    for (int ks = ks_begin; ks < ks_end; ks += 2) {
      super_step(ks, 0, ccA, scA, ccB, scB);
      if (ks + 1 < ks_end) super_step(ks + 1, 1, ccB, scB, ccA, scA);
    }
    if (!late) phase_sync();
  } else
  for (int ks = ks_begin; ks < ks_end; ks += 2) {
    load_x(ks + 1, xr);
    load_codes(ks + 1, ccB, scB);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    compute(0, ccA, scA);
    store_x(1, xr);
    __syncthreads();
    load_x(ks + 2, xr);
    load_codes(ks + 2, ccA, scA);
    __builtin_amdgcn_sched_barrier(0);
    if (ks + 1 < ks_end) compute(1, ccB, scB);
    store_x(0, xr);
    __syncthreads();
  }

  // ---- epilogue: x is the MFMA's A operand and W its B operand, so lane
  // (l32, h) holds W row row_base + 32*mb + l32 for tokens 32*nb + 8*(i/4) +
  // 4*h + (i%4): for each i a half-wave covers 32 consecutive y elements of
  // one token (128 contiguous bytes), for stores and atomics alike.
  // Output step.  Lane (l32, h) holds W row row_base + 32*mb + l32 for tokens
  // 32*nb + 8*(i/4) + 4*h + (i%4).  Each output kind has a loop nest of its
  // own (block-uniform branch outside the loops), so every nest unrolls and
  // the accumulators stay in registers.
  const int row = row_base + l32;  // + 32 * mb
  auto out_row = [&](int tok) {
    if constexpr (MOE) return a.pairs[first + tok];
    else return tok_base + tok;
  };
  if (a.epi == kEpiNone && a.y_kind == kOutF32) {
    // plain fp32: for each i a half-wave covers 32 consecutive y elements of
    // one token (128 contiguous bytes), for stores and atomics alike
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = nb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        if (tok >= count) continue;
        float* yrow = reinterpret_cast<float*>(a.y) + (int64_t)out_row(tok) * a.rows;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = row + 32 * mb;
          if (r < a.rows) {
            if (nslices > 1) atomicAdd(yrow + r, acc[mb][nb][i]);  // block-uniform branch
            else yrow[r] = acc[mb][nb][i];
          }
        }
      }
    }
  } else if (a.epi == kEpiSwiglu) {
    // rows 2i (gate, even lane) and 2i + 1 (up, the odd neighbour, fetched by
    // a DPP swap; both lanes of a pair hold the same tokens) -> y[.][i]
    const int y_kind = a.y_kind, half_rows = a.rows >> 1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = nb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        if (tok >= count) continue;
        const int64_t ybase = (int64_t)out_row(tok) * half_rows;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = row + 32 * mb;
          const float up = dpp_mov<0xB1>(acc[mb][nb][i]);  // quad_perm [1,0,3,2]
          if ((l32 & 1) == 0 && r < a.rows) store_out(a.y, ybase + (r >> 1), swiglu(acc[mb][nb][i], up), y_kind);
        }
      }
    }
  } else if (a.epi == kEpiCombine) {
    // routed only: y[token] += router weight x row
    if constexpr (MOE) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = nb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
          if (tok >= count) continue;
          const int pair = out_row(tok);
          const float wgt = a.route_w[pair];
          float* yrow = reinterpret_cast<float*>(a.y) + (int64_t)(pair / a.top_k) * a.rows;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int r = row + 32 * mb;
            if (r < a.rows) atomicAdd(yrow + r, wgt * acc[mb][nb][i]);
          }
        }
      }
    }
  } else {
    // fp16 / bf16 y (such tiles are never split along K)
    const int y_kind = a.y_kind;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = nb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
        if (tok >= count) continue;
        const int64_t ybase = (int64_t)out_row(tok) * a.rows;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int r = row + 32 * mb;
          if (r < a.rows) store_out(a.y, ybase + r, acc[mb][nb][i], y_kind);
        }
      }
    }
  }
}

// Zero the y region of tiles [first, first + gridDim.x), gridDim.y blocks per
// tile, 16-byte stores where the rows allow (a kernel rather than
// hipMemsetAsync, so it can sit in a graph).
static __global__ __launch_bounds__(256) void vq_zero_tiles_kernel(float* y, int rows, int T, int first, int n_row_tiles,
                                                            int n_tok_tiles, int tile_rows, int tile_tokens) {
  int rt, tt;
  gemm_tile_coords(first + (int)blockIdx.x, n_row_tiles, n_tok_tiles, rt, tt);
  const int r0 = rt * tile_rows, nr = min(tile_rows, rows - r0);
  const int t0 = tt * tile_tokens, nt = min(tile_tokens, T - t0);
  const bool vec = (rows & 3) == 0;  // r0 is a multiple of tile_rows (of 32)
  const int per_row = vec ? (nr + 3) / 4 : nr;
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < nt * per_row; i += gridDim.y * blockDim.x) {
    const int t = i / per_row, k = i - t * per_row;
    float* yr = y + (int64_t)(t0 + t) * rows + r0;
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
static_assert(GemmMoe::kTokens == kMoeTileTokens, "routing tiles match the grouped GEMM's token tile");

// d = 2 thin tiles (32 tokens) take 128-column super-steps when the columns
// allow: half the barriers and x stages per column, 6-10 % faster there; the
// 128-token tiles gain about 1 % and keep 64.
template <int D, class SH>
bool gemm_wide(int cols) { return D == 2 && SH::kTokens <= 32 && cols % 128 == 0; }

template <int D, int B, int G, class SH, bool MOE>
hipError_t gemm_launch(const GemmArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (D == 2 && SH::kTokens <= 32) {
    if (gemm_wide<D, SH>(a.cols)) {
      hipLaunchKernelGGL((vq_gemm_kernel<D, B, G, SH, MOE, true>), grid, dim3(SH::kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((vq_gemm_kernel<D, B, G, SH, MOE, false>), grid, dim3(SH::kThreads), 0, s, a);
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
  return a;
}

template <int D, int B, int G, class SH>
hipError_t gemm_dense(GemmArgs a, hipStream_t s) {
  a.n_row_tiles = (a.rows + SH::kRows - 1) / SH::kRows;
  a.n_tok_tiles = (a.T + SH::kTokens - 1) / SH::kTokens;
  const int tiles = a.n_row_tiles * a.n_tok_tiles;
  // each K slice keeps at least 512 columns (1024 for d = 8), whatever the
  // super-step length
  const int max_split = std::max(1, a.cols / (D == 8 ? 1024 : 512));
  const int cus = num_cus();
  // Whole rounds of tiles run as whole tiles; the tiles of a last, partial
  // round are split along K over the CUs and added atomically into a zeroed
  // y (their fp32 addition order then varies between runs).
  // The split minimises the partial round's time in tile rounds,
  // ceil(rem * split / cus) / split, plus a small charge per extra slice for
  // the atomic traffic.
  int full = (tiles / cus) * cus, rem = tiles - full, split = 1;
  if (rem > 0) {
    double best = 1e30;
    // the charge per slice scales with the tokens of a tile: the atomic adds
    // are T x rows per slice, negligible next to the weight stream at small T
    const double charge = 0.03 * std::min(1.0, (double)a.T / SH::kTokens);
    for (int sp = 1; sp <= std::min(32, max_split); ++sp) {
      const double c = (double)((rem * sp + cus - 1) / cus) / sp + charge * (sp - 1);
      if (c < best - 1e-9) {
        best = c;
        split = sp;
      }
    }
  }
  // K slices add fp32 partial sums: only a plain fp32 output can take them
  if (a.epi != kEpiNone || a.y_kind != kOutF32) split = 1;
  if (split == 1) {
    full = tiles;
    rem = 0;
  }
  a.n_full = full;
  a.rem_split = split;
  if (rem > 0) {
    hipLaunchKernelGGL(vq_zero_tiles_kernel, dim3(rem, std::max(1, 2 * cus / rem)), dim3(256), 0, s,
                       static_cast<float*>(a.y), a.rows,
                       a.T, full, a.n_row_tiles, a.n_tok_tiles, SH::kRows, SH::kTokens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return gemm_launch<D, B, G, SH, false>(a, dim3((unsigned)(full + rem * split)), s);
}

template <int D, int B, int G>
hipError_t gemm_geom(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) {
  GemmArgs a = base_args(w, io, x, y, G, D, B);
  a.T = T;
  if (T <= 32) return gemm_dense<D, B, G, GemmSmallT>(a, s);
  return gemm_dense<D, B, G, GemmLargeT>(a, s);
}

// The grouped GEMM over the tile list the routing kernel left in the
// workspace.
template <int D, int B, int G>
hipError_t moe_gemm_geom(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot, int T, int top_k,
                         void* y, int32_t* ws, hipStream_t s) {
  const int npairs = T * top_k;
  const int E = w.num_experts;
  GemmArgs a = base_args(w, io, x, y, G, D, B);
  a.tiles = moe_ws_tiles(ws, E, npairs);
  a.n_tiles = moe_ws_n_tiles(ws, E);
  a.pairs = moe_ws_pairs(ws, E);
  a.top_k = top_k;
  a.x_per_slot = x_per_slot;
  a.x_rows = x_per_slot ? npairs : T;
  a.n_row_tiles = (a.rows + GemmMoe::kRows - 1) / GemmMoe::kRows;
  dim3 grid(moe_max_tiles(npairs, E), a.n_row_tiles);
  return gemm_launch<D, B, G, GemmMoe, true>(a, grid, s);
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
hipError_t moe_gemm_bits(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot, int T, int top_k,
                         void* y, int32_t* ws, hipStream_t s) {
#define X(D, G) \
  if (w.d == D && w.group == G) return moe_gemm_geom<D, B, G>(w, io, x, x_per_slot, T, top_k, y, ws, s);
  X(2, 64) X(2, 128) X(4, 64) X(4, 128) X(8, 64) X(8, 128)
#undef X
  return hipErrorInvalidValue;
}

// The entry points of one code width's translation unit (vq_gemm_bNN.hip).
#define VQMI_GEMM_UNIT(B)                                                                                    \
  hipError_t gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) { \
    return gemm_bits<B>(w, io, x, T, y, s);                                                                  \
  }                                                                                                          \
  hipError_t moe_gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot, int T,     \
                           int top_k, void* y, int32_t* ws, hipStream_t s) {                                \
    return moe_gemm_bits<B>(w, io, x, x_per_slot, T, top_k, y, ws, s);                                       \
  }

}  // namespace vqmi
