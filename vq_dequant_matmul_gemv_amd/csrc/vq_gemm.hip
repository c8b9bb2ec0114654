// vq_gemm.hip -- prefill-shaped VQ matmul on fp16 MFMA (dense and grouped
// routed-expert), plus the on-device routing that groups (token, slot) pairs
// by expert.
//
// What is computed: y[t][r] = sum_c W[r][c] * x[t][c] with
// W[r][c] = fp16(codebook[code][c % d] * scale[r][c / g]) exactly as the
// dequant defines it (paper "Data-Free Vector Quantization Beats Affine
// Quantization at Matched Bytes Below 5 Bits", §2.2 and §3.4: prefill runs a
// prefill-shaped path over the same codes; model card
// "Qwen3.5-397B-A17B-VQ-2.4bpw", Methodology, for the format), fp32
// accumulation in v_mfma_f32_16x16x32_f16.
//
// Design for gfx950:
//  * A = dequantized W (16 rows x 32 k per MFMA), B = x (32 k x 16 tokens).
//    A wave owns 64 rows (4 m-blocks) and all WN tokens of the block tile;
//    the block's 4 waves cover 256 rows, so every weight is dequantized
//    exactly once per token tile, straight into the A-operand registers
//    (no LDS round trip for W).
//  * The contraction order over k is free, so each lane group (lanes 16g ..
//    16g+15) takes a contiguous run of CG columns per "super-step" (CG = 32,
//    or 64 for d = 8): a lane's codes for one super-step are one small
//    contiguous load (16, 8 or 12 bytes) and its x slices are contiguous.
//  * x tiles (WN tokens x 4*CG columns) go through LDS, double-buffered, one
//    barrier per super-step; rows are padded by 16 bytes so the 16-byte
//    fragment reads of 16 tokens hit distinct banks.
//  * Codebook in LDS (replicated for K = 256, as in the GEMV).
//  * Routed experts: the routing kernel counts pairs per expert, scans,
//    scatters pair ids by expert and emits a flat list of (expert, first,
//    count) token tiles; the GEMM walks that list with gathered x rows and
//    writes y[pair] rows directly.  All on the stream, no host sync.

#include "vq_device.h"
#include "vq_kernels.h"

#include <algorithm>

namespace vqmi {

namespace {

// Codes of one lane for one super-step: NCL codes of B bits, word aligned.
template <int NCL, int B>
struct LaneCodes {
  static constexpr int kWords = NCL * B / 32;
  uint32_t w[kWords];
};

template <int NCL, int B>
__device__ __forceinline__ void load_lane_codes(LaneCodes<NCL, B>& c, rsrc_t r, uint32_t off) {
  constexpr int W = LaneCodes<NCL, B>::kWords;
  if constexpr (W == 4) {
    u32x4 v = buf_load_b128(r, off);
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
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

template <int D, int B, int NCL>
__device__ __forceinline__ Entry<D> lane_gather(const uint8_t* lds, const LaneCodes<NCL, B>& c,
                                                int i, uint32_t lane_off) {
  using L = CodebookLayout<D, B>;
  uint32_t off;
  if constexpr (L::kReplicated) {
    off = entry_offset_byte<D, B>(c.w[i >> 2], i & 3, lane_off);
  } else {
    off = lane_code<NCL, B>(c, i) * (uint32_t)L::kEntryBytes;
  }
  return lds_entry<D>(lds, off);
}

}  // namespace

struct GemmArgs {
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  const uint16_t* x;
  float* y;
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
};

template <int D, int B, int G, int NBT, bool MOE>
__global__ __launch_bounds__(256) void vq_gemm_kernel(GemmArgs a) {
  using L = CodebookLayout<D, B>;
  constexpr int CG = (D == 8) ? 64 : 32;  // columns per lane group per super-step
  constexpr int S = CG / 8;               // MFMA k-steps (32 columns each) per super-step
  constexpr int NCL = CG / D;             // codes per lane per super-step
  constexpr int SS = 4 * CG;              // columns per super-step
  constexpr int MB = 4;                   // 16-row m-blocks per wave
  constexpr int WN = 16 * NBT;            // tokens per block tile
  constexpr int XROW = SS * 2 + 16;       // LDS bytes per token row (padded)
  constexpr int SEGS = SS / 8;            // 16-byte segments per token row
  constexpr int XLD = WN * SEGS / 256;    // x segments loaded per thread per super-step
  static_assert(XLD >= 1 && (WN * SEGS) % 256 == 0, "x tile must split evenly");
  constexpr int CPA = 8 / D;              // codes per A fragment (8 columns)

  // Static LDS: codebook, then the two x tiles [2][WN][XROW].
  __shared__ __align__(16) uint8_t cb_lds[L::kBytes];
  __shared__ __align__(16) uint8_t xbuf[2 * WN * XROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // ---- which tile ----
  int rt, expert = 0, first = 0, count;
  int tok_base = 0;
  if constexpr (MOE) {
    const int tix = blockIdx.x;
    if (tix >= *a.n_tiles) return;
    expert = a.tiles[3 * tix + 0];
    first = a.tiles[3 * tix + 1];
    count = a.tiles[3 * tix + 2];
    rt = blockIdx.y;
  } else {
    // XCD-aware order: blocks land on XCD (bid % 8) round-robin; give each XCD
    // a contiguous range of tiles, grouped 4 row tiles x all token tiles so
    // concurrently running blocks share x and W slices in that XCD's L2.
    const int N = a.n_row_tiles * a.n_tok_tiles;
    const int bid = blockIdx.x;
    const int q = N / 8, r8 = N % 8, xcd = bid % 8, j = bid / 8;
    const int tile = xcd * q + min(xcd, r8) + j;
    const int GR = 4;
    const int grp = tile / (GR * a.n_tok_tiles);
    const int in = tile - grp * GR * a.n_tok_tiles;
    const int rows_in_grp = min(GR, a.n_row_tiles - grp * GR);
    rt = grp * GR + in % rows_in_grp;
    const int tt = in / rows_in_grp;
    tok_base = tt * WN;
    count = min(WN, a.T - tok_base);
  }

  const uint32_t* codes = a.codes + (int64_t)expert * a.code_estride;
  const uint16_t* scales = a.scales + (int64_t)expert * a.scale_estride;
  const uint16_t* cb = a.codebook + (int64_t)expert * a.cb_estride;

  // All streaming loads are branch-free buffer loads with 32-bit offsets:
  // tokens past the tile's count, rows past the end and columns past `cols`
  // (the half super-step d = 2 can leave) get an out-of-range offset or fall
  // outside the buffer and read zeros, so every load of a super-step is in
  // flight at once and no lane needs a 64-bit address.

  // ---- x loading assignment: XLD segments of 16 bytes per thread ----
  const int seg = tid % SEGS;
  rsrc_t rx;
  uint32_t xoff[XLD];
  int xdst[XLD];
  if constexpr (MOE) {
    rx = make_rsrc(a.x, (uint64_t)a.x_rows * a.cols * 2);
  } else {
    rx = make_rsrc(a.x + (int64_t)tok_base * a.cols, (uint64_t)count * a.cols * 2);
  }
#pragma unroll
  for (int i = 0; i < XLD; ++i) {
    const int tok = tid / SEGS + i * (256 / SEGS);
    xdst[i] = tok * XROW + seg * 16;
    uint32_t row;
    if constexpr (MOE) {
      const int pair = tok < count ? a.pairs[first + tok] : 0;
      row = (uint32_t)(a.x_per_slot ? pair : pair / a.top_k);
    } else {
      row = (uint32_t)tok;
    }
    xoff[i] = tok < count ? row * (uint32_t)a.cols * 2u + (uint32_t)seg * 16u : kOutOfRange;
  }

  // ---- A assignment: wave owns rows rt*256 + wave*64 + [0, 64) ----
  const int row_base = rt * 256 + wave * 64;
  const rsrc_t rc = make_rsrc(codes, (uint64_t)a.rows * a.wr * 4);
  const rsrc_t rs = make_rsrc(scales, (uint64_t)a.rows * a.spr * 2);
  uint32_t coff[MB], soff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint32_t r = (uint32_t)(row_base + mb * 16 + l16);   // past the end: reads zeros
    coff[mb] = r * (uint32_t)a.wr * 4u;
    soff[mb] = r * (uint32_t)a.spr * 2u;
  }

  const int nks = (a.cols + SS - 1) / SS;
  constexpr int CW_SS = SS / D * B / 32;   // code words per row per super-step
  constexpr int NCLW = NCL * B / 32;       // code words per lane per super-step

  auto load_x = [&](int ks, u32x4 (&xr)[XLD]) {
    const bool ok = ks * SS + seg * 8 < a.cols;
    const uint32_t colb = (uint32_t)ks * SS * 2u;
#pragma unroll
    for (int i = 0; i < XLD; ++i) xr[i] = buf_load_b128(rx, ok ? xoff[i] + colb : kOutOfRange);
  };
  auto store_x = [&](int buf, const u32x4 (&xr)[XLD]) {
#pragma unroll
    for (int i = 0; i < XLD; ++i)
      *reinterpret_cast<u32x4*>(xbuf + buf * (WN * XROW) + xdst[i]) = xr[i];
  };
  auto load_codes = [&](int ks, LaneCodes<NCL, B> (&cc)[MB], uint16_t (&sc)[MB]) {
    const uint32_t wb = (uint32_t)(ks * CW_SS + g * NCLW) * 4u;
    const uint32_t sb = (uint32_t)((ks * SS + g * CG) / G) * 2u;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      load_lane_codes<NCL, B>(cc[mb], rc, coff[mb] + wb);
      sc[mb] = buf_load_b16(rs, soff[mb] + sb);
    }
  };

  const uint32_t lane_off = lane_copy_offset<D, B>(lane);
  float4_t acc[MB][NBT];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBT; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // One super-step: dequantize the A fragments of each m-block straight into
  // registers and run the MFMAs against the x tile in LDS buffer `buf`.
  auto compute = [&](int ks, int buf, const LaneCodes<NCL, B> (&cc)[MB], const uint16_t (&sc)[MB]) {
    const bool gcur = ks * SS + g * CG < a.cols;
    const uint8_t* xb = xbuf + buf * (WN * XROW);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      half8_t bf[NBT];
#pragma unroll
      for (int nb = 0; nb < NBT; ++nb)
        bf[nb] = *reinterpret_cast<const half8_t*>(xb + (nb * 16 + l16) * XROW + (g * CG + 8 * s) * 2);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const half2_t s2 = as_half2((uint32_t)sc[mb] | ((uint32_t)sc[mb] << 16));
        half2_t w[4];
#pragma unroll
        for (int c = 0; c < CPA; ++c) {
          const Entry<D> e = lane_gather<D, B, NCL>(cb_lds, cc[mb], s * CPA + c, lane_off);
#pragma unroll
          for (int j = 0; j < D / 2; ++j) w[c * (D / 2) + j] = e.v[j] * s2;
        }
        half8_t af = half8_t{w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
        if (!gcur) af = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int nb = 0; nb < NBT; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  };

  // Ping-pong over two register sets (A, B) and two LDS x buffers (0, 1):
  // the loads for super-step ks + 1 are issued before super-step ks is
  // computed; no register copies, so the prefetch stays in flight.
  u32x4 xr[XLD];
  LaneCodes<NCL, B> ccA[MB], ccB[MB];
  uint16_t scA[MB], scB[MB];

  load_x(0, xr);
  load_codes(0, ccA, scA);
  stage_codebook<D, B>(cb_lds, cb, tid, 256);
  store_x(0, xr);
  __syncthreads();

  for (int ks = 0; ks < nks; ks += 2) {
    const bool has1 = ks + 1 < nks;
    if (has1) {
      load_x(ks + 1, xr);
      load_codes(ks + 1, ccB, scB);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    compute(ks, 0, ccA, scA);
    if (has1) store_x(1, xr);
    __syncthreads();
    if (!has1) break;
    const bool has2 = ks + 2 < nks;
    if (has2) {
      load_x(ks + 2, xr);
      load_codes(ks + 2, ccA, scA);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(ks + 1, 1, ccB, scB);
    if (has2) store_x(0, xr);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*g + i of each m-block for token l16 ----
  const bool vec_ok = (a.rows & 3) == 0;
#pragma unroll
  for (int nb = 0; nb < NBT; ++nb) {
    const int tok = nb * 16 + l16;
    if (tok >= count) continue;
    int yr;
    if constexpr (MOE) yr = a.pairs[first + tok];
    else yr = tok_base + tok;
    float* yrow = a.y + (int64_t)yr * a.rows;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = row_base + mb * 16 + 4 * g;
      const float4_t v = acc[mb][nb];
      if (vec_ok && r + 3 < a.rows) {
        *reinterpret_cast<float4_t*>(yrow + r) = v;
      } else {
        if (r + 0 < a.rows) yrow[r + 0] = v.x;
        if (r + 1 < a.rows) yrow[r + 1] = v.y;
        if (r + 2 < a.rows) yrow[r + 2] = v.z;
        if (r + 3 < a.rows) yrow[r + 3] = v.w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// routing: group (token, slot) pairs by expert and emit the token-tile list.
// One block; pairs and experts are walked in strides of the block size.
// Workspace layout (int32): counts[E] | offsets[E] | fill[E] | tile_base[E] |
// n_tiles[1] | pad to 4 | pairs[npairs] | tiles[max_tiles][3]
// ---------------------------------------------------------------------------

struct RouteArgs {
  const int32_t* ids;
  int32_t* ws;
  float* y;
  int npairs, num_experts, rows, tile_tokens, max_tiles;
};

__global__ __launch_bounds__(1024) void vq_route_kernel(RouteArgs a) {
  const int E = a.num_experts;
  int32_t* counts = a.ws;
  int32_t* offsets = counts + E;
  int32_t* fill = offsets + E;
  int32_t* tbase = fill + E;
  int32_t* n_tiles = tbase + E;
  int32_t* pairs = a.ws + ((4 * E + 1 + 3) & ~3);
  int32_t* tiles = pairs + ((a.npairs + 3) & ~3);
  const int tid = threadIdx.x, nt = blockDim.x;
  __shared__ int32_t part[1024];

  for (int e = tid; e < E; e += nt) { counts[e] = 0; fill[e] = 0; }
  __syncthreads();
  for (int p = tid; p < a.npairs; p += nt) {
    const int e = a.ids[p];
    if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  }
  __syncthreads();
  // exclusive scans of counts and of tiles-per-expert: each thread owns a
  // contiguous run of experts
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sc = 0, st = 0;
  for (int e = e0; e < e1; ++e) { sc += counts[e]; st += (counts[e] + a.tile_tokens - 1) / a.tile_tokens; }
  // block scan over threads (two values packed: counts < 2^20 per block? use two passes)
  part[tid] = sc;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run_c = part[tid] - sc;
  __syncthreads();
  part[tid] = st;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run_t = part[tid] - st;
  if (tid == nt - 1) *n_tiles = part[tid];
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run_c;
    tbase[e] = run_t;
    const int c = counts[e];
    const int nt_e = (c + a.tile_tokens - 1) / a.tile_tokens;
    for (int k = 0; k < nt_e; ++k) {
      int32_t* t = tiles + 3 * (run_t + k);
      t[0] = e;
      t[1] = run_c + k * a.tile_tokens;
      t[2] = min(a.tile_tokens, c - k * a.tile_tokens);
    }
    run_c += c;
    run_t += nt_e;
  }
  __syncthreads();
  for (int p = tid; p < a.npairs; p += nt) {
    const int e = a.ids[p];
    if (e >= 0 && e < E) {
      const int pos = offsets[e] + atomicAdd(&fill[e], 1);
      pairs[pos] = p;
    } else {
      float* yr = a.y + (int64_t)p * a.rows;  // skipped slot: zero row
      for (int r = 0; r < a.rows; ++r) yr[r] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

namespace {

constexpr int kMoeTileTokens = 64;

int max_tiles_for(int npairs, int E) { return (npairs + kMoeTileTokens - 1) / kMoeTileTokens + E; }

template <int D, int B, int G, int NBT, bool MOE>
hipError_t gemm_launch(const GemmArgs& a, dim3 grid, hipStream_t s) {
  auto k = vq_gemm_kernel<D, B, G, NBT, MOE>;
  hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

GemmArgs base_args(const TensorView& w, const uint16_t* x, float* y, int G, int D, int B) {
  GemmArgs a{};
  a.codes = w.codes;
  a.codebook = w.codebook;
  a.scales = w.scales;
  a.x = x;
  a.y = y;
  a.code_estride = (int64_t)w.rows * w.wr;
  a.scale_estride = (int64_t)w.rows * (w.cols / G);
  a.cb_estride = w.cb_per_expert ? (int64_t)(1 << B) * D : 0;
  a.rows = w.rows;
  a.cols = w.cols;
  a.wr = w.wr;
  a.spr = w.cols / G;
  a.n_row_tiles = (w.rows + 255) / 256;
  return a;
}

template <int D, int B, int G>
hipError_t gemm_geom(const TensorView& w, const uint16_t* x, int T, float* y, hipStream_t s) {
  GemmArgs a = base_args(w, x, y, G, D, B);
  a.T = T;
  // token tile: 128 for long prompts, smaller when there are few tokens
  // (d = 8 is held to 64 by LDS: 64 KiB codebook + x tiles)
  int nbt = std::min((T + 15) / 16, 4);
  if (nbt > 2) nbt = 4;
  a.n_tok_tiles = (T + 16 * nbt - 1) / (16 * nbt);
  dim3 grid(a.n_row_tiles * a.n_tok_tiles);
  switch (nbt) {
    case 1: return gemm_launch<D, B, G, 1, false>(a, grid, s);
    case 2: return gemm_launch<D, B, G, 2, false>(a, grid, s);
    case 4: return gemm_launch<D, B, G, 4, false>(a, grid, s);
    default: return gemm_launch<D, B, G, 4, false>(a, grid, s);
  }
}

template <int D, int B, int G>
hipError_t moe_gemm_geom(const TensorView& w, const uint16_t* x, int x_per_slot,
                         const int32_t* ids, int T, int top_k, float* y, void* ws, hipStream_t s) {
  const int npairs = T * top_k;
  const int E = w.num_experts;
  const int mt = max_tiles_for(npairs, E);
  int32_t* wsi = static_cast<int32_t*>(ws);
  RouteArgs r{};
  r.ids = ids;
  r.ws = wsi;
  r.y = y;
  r.npairs = npairs;
  r.num_experts = E;
  r.rows = w.rows;
  r.tile_tokens = kMoeTileTokens;
  r.max_tiles = mt;
  hipLaunchKernelGGL(vq_route_kernel, dim3(1), dim3(1024), 0, s, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemmArgs a = base_args(w, x, y, G, D, B);
  int32_t* n_tiles = wsi + 4 * E;
  int32_t* pairs = wsi + ((4 * E + 1 + 3) & ~3);
  int32_t* tiles = pairs + ((npairs + 3) & ~3);
  a.tiles = tiles;
  a.n_tiles = n_tiles;
  a.pairs = pairs;
  a.top_k = top_k;
  a.x_per_slot = x_per_slot;
  a.x_rows = x_per_slot ? npairs : T;
  dim3 grid(mt, a.n_row_tiles);
  return gemm_launch<D, B, G, kMoeTileTokens / 16, true>(a, grid, s);
}

}  // namespace

size_t moe_workspace_bytes(int T, int top_k, int num_experts) {
  const int64_t npairs = (int64_t)T * top_k;
  if (npairs <= 0) return 0;
  const int64_t mt = (npairs + kMoeTileTokens - 1) / kMoeTileTokens + num_experts;
  const int64_t words = ((4 * (int64_t)num_experts + 1 + 3) & ~3) + ((npairs + 3) & ~3) + 3 * mt;
  return (size_t)(words * 4);
}

#define VQMI_GEOMS(X) \
  X(2, 8, 64) X(2, 8, 128) X(2, 12, 64) X(2, 12, 128) \
  X(4, 8, 64) X(4, 8, 128) X(4, 12, 64) X(4, 12, 128) \
  X(8, 8, 64) X(8, 8, 128) X(8, 12, 64) X(8, 12, 128)

hipError_t launch_gemm(const TensorView& w, const uint16_t* x, int T, float* y, hipStream_t s) {
#define X(D, B, G) \
  if (w.d == D && w.log2_k == B && w.group == G) return gemm_geom<D, B, G>(w, x, T, y, s);
  VQMI_GEOMS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_moe_gemm(const TensorView& w, const uint16_t* x, int x_per_slot,
                           const int32_t* ids, int T, int top_k, float* y, void* ws,
                           hipStream_t s) {
#define X(D, B, G)                                   \
  if (w.d == D && w.log2_k == B && w.group == G)     \
    return moe_gemm_geom<D, B, G>(w, x, x_per_slot, ids, T, top_k, y, ws, s);
  VQMI_GEOMS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace vqmi
