// vq_gemv.hip -- decode-shaped VQ matmul (dense and routed-expert), and the
// stand-alone dequant kernel.
//
// What is computed (paper "Data-Free Vector Quantization Beats Affine
// Quantization at Matched Bytes Below 5 Bits", §3.4: a fused decode-and-matmul
// that reads codes and codebook directly; model card
// "Qwen3.5-397B-A17B-VQ-2.4bpw", Methodology, for the format):
//   y[t][r] = sum_g scale[r][g] * sum_{c in group g} codebook[code(r, c/d)][c % d] * x[t][c]
// with fp32 accumulation.  Each product of two fp16 values is exact in fp32.
//
// Design for gfx950 (batch-1 decode is bound by the bytes of codes + scales):
//  * A row's code stream is cut into passes of 64 sixteen-code chunks (one
//    chunk, 16 or 24 bytes, per lane).  Each wave of a block owns one pass
//    position and a contiguous range of the block's rows: its lanes keep the
//    x columns of that pass in VGPRs for the whole kernel ("x-stationary"),
//    and every load instruction covers a contiguous 1 KiB (1.5 KiB) run of a
//    row.  Waves never wait on each other until the block's final combine.
//  * Each lane keeps a ring of PD rows' chunks in flight: the load for row
//    u + PD is issued as soon as row u is consumed.  Loads are buffer loads
//    with the row offset in an SGPR, so a load costs no address VALU.
//  * The codebook sits in LDS; for K = 256 it is replicated so that a lane's
//    gather bank depends only on its lane id (conflict-free).
//  * Inner loop per code: one v_perm_b32 (LDS offset), one LDS read, d/2
//    v_dot2_f32_f16 per token; the group scale multiplies the group's sum
//    once (an fma per group).  A row piece is summed across the wave by DPP;
//    with one pass per row it is stored directly, otherwise the pieces go to
//    a small LDS table and are added in pass order after one barrier.
//  * Routed experts (top-k MoE): blockIdx.y is the (token, slot) pair; the
//    block reads its expert id and points at that expert's codes and scales.
//    An id outside [0, E) writes a zero row.

#include "vq_device.h"
#include "vq_kernels.h"

#include <algorithm>

namespace vqmi {

struct GemvArgs {
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  const uint16_t* x;
  float* y;
  const int32_t* ids;     // routed: [pairs]; dense: nullptr
  int64_t code_estride;   // words between experts
  int64_t scale_estride;  // fp16 between experts
  int64_t cb_estride;     // fp16 between per-expert codebooks (0: shared)
  int rows, cols, wr, spr;
  int P;                  // 16-code chunks per row in this column slice
  int p0;                 // first chunk of the slice
  int passes;             // ceil(P / 64)
  int waves_per_pass;     // waves of a block sharing one pass position
  int accumulate;         // add into y (column slices after the first)
  int T;                  // dense: tokens; routed: pairs
  int top_k;
  int num_experts;
  int x_per_slot;
};

constexpr int gemv_max_tt(int D) { return D == 8 ? 1 : 2; }
// Waves per block: 16 where x (8*d VGPRs per token) and the ring fit in 128
// VGPRs, else 8.
constexpr int gemv_max_waves(int D, int TT) { return (D == 2 || (D == 4 && TT == 1)) ? 16 : 8; }
// Rows in flight per lane.  Measured on MI355X (17408x5120, d=2): a ring of
// 3-4 rows with 15-16 waves per CU beats deeper rings (6: +8 %, 12: +30 %);
// more outstanding requests per CU only queue up.
template <int D, int B, int TT>
struct GemvCfg {
  static constexpr int kPD = gemv_max_waves(D, TT) == 16 ? 4 : 6;
};
constexpr int kGemvRowPieces = 4096;  // LDS table entries for split rows (floats)

// Total of v over the 64 lanes of the wave, valid in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v = row16_sum(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

template <int D, int B, int G, int TT, bool MOE>
__global__ __launch_bounds__(64 * gemv_max_waves(D, TT)) void vq_gemv_kernel(GemvArgs a) {
  using L = CodebookLayout<D, B>;
  constexpr int PD = GemvCfg<D, B, TT>::kPD;
  constexpr int NSC = (16 * D > G) ? (16 * D / G) : 1;  // scales per chunk
  constexpr int CPS = 16 / NSC;                          // codes per scale in a chunk
  constexpr int HX = 8 * D;                              // half2 of x per chunk per token
  constexpr int CB = Chunk<B>::kWords * 4;               // code bytes per chunk
  static_assert(TT <= gemv_max_tt(D), "token tile too large for this d");

  __shared__ __align__(16) uint8_t cb_lds[L::kBytes];
  __shared__ __align__(16) u32x4 raw[256];               // replicated layout: entries before expansion
  __shared__ float pieces[kGemvRowPieces];               // [brows][passes][TT] when passes > 1

  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int passes = a.passes;
  const int k = a.waves_per_pass;
  const int c = wave % passes;                           // this wave's pass
  const int jw = wave / passes;                          // its slot among the pass's waves
  const bool wave_on = jw < k;

  // ---- this block's rows, this wave's rows ----
  const int nblk = gridDim.x;
  const int brow0 = (int)((int64_t)a.rows * blockIdx.x / nblk);
  const int brows = (int)((int64_t)a.rows * (blockIdx.x + 1) / nblk) - brow0;
  const int wr0 = wave_on ? brows * jw / k : 0;
  const int wr1 = wave_on ? brows * (jw + 1) / k : 0;
  const int nrows = wr1 - wr0;

  const uint32_t* codes = a.codes;
  const uint16_t* scales = a.scales;
  const uint16_t* cb = a.codebook;
  const uint16_t* xb;
  float* yb;
  int ntok;
  if constexpr (MOE) {
    const int pair = blockIdx.y;
    const int e = a.ids[pair];
    yb = a.y + (int64_t)pair * a.rows;
    if (e < 0 || e >= a.num_experts) {  // skipped slot: zero rows (block-uniform exit)
      if (a.p0 == 0)
        for (int r = tid; r < brows; r += nt) yb[brow0 + r] = 0.f;
      return;
    }
    codes += (int64_t)e * a.code_estride;
    scales += (int64_t)e * a.scale_estride;
    cb += (int64_t)e * a.cb_estride;
    const int t = pair / a.top_k;
    xb = a.x + (int64_t)(a.x_per_slot ? pair : t) * a.cols;
    ntok = 1;
  } else {
    const int tok0 = blockIdx.y * TT;
    xb = a.x + (int64_t)tok0 * a.cols;
    yb = a.y + (int64_t)tok0 * a.rows;
    ntok = min(TT, a.T - tok0);
  }

  const int p = c * 64 + lane;            // chunk within the slice
  const int gp = a.p0 + p;                // chunk within the full row
  const bool in_row = p < a.P;            // lanes past the row end add nothing

  // ---- x of this lane's chunk into VGPRs; codebook entries ----
  const rsrc_t rx = make_rsrc(xb, (uint64_t)ntok * a.cols * 2);
  u32x4 xr[TT][HX / 4];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < HX / 4; ++q)
      xr[tt][q] = buf_load_b128(rx, in_row ? (uint32_t)(tt * a.cols + gp * 16 * D) * 2u + 16u * q : kOutOfRange);
  u32x4 ce = u32x4{0u, 0u, 0u, 0u};
  if constexpr (L::kReplicated) {
    if (tid < 256) {
      if constexpr (D == 2) ce.x = reinterpret_cast<const uint32_t*>(cb)[tid];
      else if constexpr (D == 4) { const u32x2 t = reinterpret_cast<const u32x2*>(cb)[tid]; ce.x = t.x; ce.y = t.y; }
      else ce = reinterpret_cast<const u32x4*>(cb)[tid];
    }
  }

  // ---- the prefetch ring: row offsets in SGPRs, lane offsets constant ----
  const rsrc_t rc = make_rsrc(codes, (uint64_t)a.rows * a.wr * 4);
  const rsrc_t rs = make_rsrc(scales, (uint64_t)a.rows * a.spr * 2);
  const uint32_t row_cb = (uint32_t)a.wr * 4u;
  const uint32_t row_sb = (uint32_t)a.spr * 2u;
  const uint32_t c_lane = in_row ? (uint32_t)gp * CB : kOutOfRange;
  const uint32_t s_lane = in_row ? (uint32_t)((gp * 16 * D) / G) * 2u : kOutOfRange;

  Chunk<B> ring[PD];
  uint16_t rsc[PD][NSC];
  int l_row = 0;  // next row (of this wave's range) to load
  // Loads are unconditional: a row past the wave's range gets an
  // out-of-range lane offset and reads zeros, so every ring slot issues the
  // same loads and the in-order vmcnt waits stay exact.
  auto load_row = [&](Chunk<B>& ch, uint16_t (&sc)[NSC]) {
    const bool live = l_row < nrows;
    const uint32_t so = live ? (uint32_t)(brow0 + wr0 + l_row) * row_cb : 0u;
    const uint32_t ss = live ? (uint32_t)(brow0 + wr0 + l_row) * row_sb : 0u;
    const uint32_t vc = live ? c_lane : kOutOfRange;
    const uint32_t vs = live ? s_lane : kOutOfRange;
    if constexpr (B == 8) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, vc, so, 0));
      ch.w[0] = v.x; ch.w[1] = v.y; ch.w[2] = v.z; ch.w[3] = v.w;
    } else {
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, vc + 8u * h, so, 0));
        ch.w[2 * h] = v.x; ch.w[2 * h + 1] = v.y;
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < NSC; ++s2) sc[s2] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs + 2u * s2, ss, 0);
    ++l_row;
  };
#pragma unroll
  for (int j = 0; j < PD; ++j) load_row(ring[j], rsc[j]);

  if constexpr (L::kReplicated) {
    if (tid < 256) raw[tid] = ce;
  } else {
    stage_codebook<D, B>(cb_lds, cb, tid, nt);
  }
  __syncthreads();
  if constexpr (L::kReplicated) {
    for (int q = tid; q < 4096; q += nt) {  // slot q holds copies of entry q / 16
      const u32x4 e = raw[q >> 4];
      u32x4 v;
      if constexpr (D == 2) v = u32x4{e.x, e.x, e.x, e.x};
      else if constexpr (D == 4) v = u32x4{e.x, e.y, e.x, e.y};
      else v = e;
      reinterpret_cast<u32x4*>(cb_lds)[q] = v;
    }
    __syncthreads();
  }

  half2_t xv[TT][HX];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int q = 0; q < HX / 4; ++q) {
      xv[tt][4 * q + 0] = as_half2(xr[tt][q].x);
      xv[tt][4 * q + 1] = as_half2(xr[tt][q].y);
      xv[tt][4 * q + 2] = as_half2(xr[tt][q].z);
      xv[tt][4 * q + 3] = as_half2(xr[tt][q].w);
    }

  const uint32_t lane_off = lane_copy_offset<D, B>(lane);
  // one pass and no accumulation: a row's wave sum is final; otherwise the
  // pieces meet in LDS and are stored (or added) after the loop
  const bool direct = passes == 1 && !a.accumulate;
  int c_row = 0;  // next row to compute
  auto compute_row = [&](const Chunk<B>& ch, const uint16_t (&sc)[NSC]) {
    float acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NSC; ++s2) {
      float g[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) g[tt] = 0.f;
#pragma unroll
      for (int i = s2 * CPS; i < (s2 + 1) * CPS; ++i) {
        const Entry<D> e = gather<D, B>(cb_lds, ch, i, lane_off);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int j = 0; j < D / 2; ++j) g[tt] = dot2(e.v[j], xv[tt][i * (D / 2) + j], g[tt]);
      }
      const float scale = half_bits_to_float(sc[s2]);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[tt] = __builtin_fmaf(g[tt], scale, acc[tt]);
    }
    const int r = wr0 + c_row;  // block-relative row
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float v = wave_sum_to_lane63(in_row ? acc[tt] : 0.f);
      if (lane == 63) {
        if (direct) {
          if (tt < ntok) yb[(int64_t)tt * a.rows + brow0 + r] = v;
        } else {
          pieces[(r * passes + c) * TT + tt] = v;
        }
      }
    }
    ++c_row;
  };

  for (int u0 = 0; u0 < nrows; u0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      if (u0 + j < nrows) compute_row(ring[j], rsc[j]);  // wave-uniform branch
      load_row(ring[j], rsc[j]);
    }
  }

  if (!direct) {  // add each row's pass pieces in pass order (deterministic)
    __syncthreads();
    for (int r = tid; r < brows; r += nt) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        float v = 0.f;
        for (int cc = 0; cc < passes; ++cc) v += pieces[(r * passes + cc) * TT + tt];
        if (tt < ntok) {
          float* dst = yb + (int64_t)tt * a.rows + brow0 + r;
          *dst = a.accumulate ? *dst + v : v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dequant: W[r][c] = fp16(codebook[code][c % d] * scale[r][c / g]) -- the same
// gather as the GEMV, one v_pk_mul_f16 (IEEE fp16 multiply, round to nearest
// even, subnormals kept) per pair of weights.
// ---------------------------------------------------------------------------

struct DequantArgs {
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  uint16_t* out;
  int rows, cols, wr, spr, P;
};

template <int D, int B, int G>
__global__ __launch_bounds__(256) void vq_dequant_kernel(DequantArgs a) {
  using L = CodebookLayout<D, B>;
  constexpr int NSC = (16 * D > G) ? (16 * D / G) : 1;
  constexpr int CPS = 16 / NSC;
  __shared__ __align__(16) uint8_t smem[L::kBytes];
  stage_codebook<D, B>(smem, a.codebook, threadIdx.x, blockDim.x);
  __syncthreads();
  const uint32_t lane_off = lane_copy_offset<D, B>(threadIdx.x & 63);
  const int64_t total = (int64_t)a.rows * a.P;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(q / a.P);
    const int p = (int)(q - (int64_t)r * a.P);
    Chunk<B> ch;
    load_chunk<B>(ch, a.codes + (int64_t)r * a.wr + (int64_t)p * Chunk<B>::kWords);
    uint32_t outw[8 * D];
#pragma unroll
    for (int s = 0; s < NSC; ++s) {
      const uint16_t sb = a.scales[(int64_t)r * a.spr + (p * 16 * D) / G + s];
      const half2_t s2 = as_half2((uint32_t)sb | ((uint32_t)sb << 16));
#pragma unroll
      for (int i = s * CPS; i < (s + 1) * CPS; ++i) {
        const Entry<D> e = gather<D, B>(smem, ch, i, lane_off);
#pragma unroll
        for (int j = 0; j < D / 2; ++j) outw[i * (D / 2) + j] = as_u32(e.v[j] * s2);
      }
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.out + (int64_t)r * a.cols + (int64_t)p * 16 * D);
#pragma unroll
    for (int q4 = 0; q4 < 2 * D; ++q4)
      dst[q4] = u32x4{outw[4 * q4], outw[4 * q4 + 1], outw[4 * q4 + 2], outw[4 * q4 + 3]};
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

namespace {

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

template <int D, int B, int G, int TT, bool MOE>
hipError_t gemv_launch(const GemvArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((vq_gemv_kernel<D, B, G, TT, MOE>), grid, dim3(64 * a.passes * a.waves_per_pass),
                     0, s, a);
  return hipGetLastError();
}

// Rows are split over blocks so that one block per CU covers the grid; each
// pass of a slice gets `waves_per_pass` waves; slices of at most
// `max_waves` passes run one after another, accumulating into y.
template <int D, int B, int G, int TT, bool MOE>
hipError_t gemv_slices(GemvArgs a, int P_total, int ycount, hipStream_t s) {
  constexpr int maxw = gemv_max_waves(D, TT);
  const int passes_total = (P_total + 63) / 64;
  const int n_slices = (passes_total + maxw - 1) / maxw;
  const int passes_per = (passes_total + n_slices - 1) / n_slices;
  const int blocks_fill = std::max(1, num_cus() / std::max(1, ycount));
  for (int sl = 0; sl < n_slices; ++sl) {
    a.p0 = sl * passes_per * 64;
    a.P = std::min(passes_per * 64, P_total - a.p0);
    a.passes = (a.P + 63) / 64;
    a.waves_per_pass = maxw / a.passes;
    a.accumulate = sl > 0;
    // enough blocks that each block's row-piece table fits in LDS
    const int64_t min_blocks = ((int64_t)a.rows * a.passes * TT + kGemvRowPieces - 1) / kGemvRowPieces;
    const int blocks = (int)std::min<int64_t>(a.rows, std::max<int64_t>(blocks_fill, min_blocks));
    hipError_t e = gemv_launch<D, B, G, TT, MOE>(a, dim3(blocks, ycount), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, int B, int G>
hipError_t gemv_geom(const TensorView& w, const uint16_t* x, int T, float* y, const int32_t* ids,
                     int top_k, int x_per_slot, hipStream_t s) {
  GemvArgs a{};
  a.codes = w.codes;
  a.codebook = w.codebook;
  a.scales = w.scales;
  a.x = x;
  a.y = y;
  a.ids = ids;
  a.code_estride = (int64_t)w.rows * w.wr;
  a.scale_estride = (int64_t)w.rows * (w.cols / G);
  a.cb_estride = w.cb_per_expert ? (int64_t)(1 << B) * D : 0;
  a.rows = w.rows;
  a.cols = w.cols;
  a.wr = w.wr;
  a.spr = w.cols / G;
  const int P_total = w.cols / (16 * D);
  a.top_k = top_k;
  a.num_experts = w.num_experts;
  a.x_per_slot = x_per_slot;
  const int tt = std::min(T >= 2 ? 2 : 1, gemv_max_tt(D));
  if (ids) {
    a.T = T * top_k;
    return gemv_slices<D, B, G, 1, true>(a, P_total, T * top_k, s);
  }
  a.T = T;
  const int ycount = (T + tt - 1) / tt;
  if constexpr (gemv_max_tt(D) >= 2) {
    if (tt == 2) return gemv_slices<D, B, G, 2, false>(a, P_total, ycount, s);
  }
  return gemv_slices<D, B, G, 1, false>(a, P_total, ycount, s);
}

template <int D, int B, int G>
hipError_t dequant_geom(const TensorView& w, int expert, uint16_t* out, hipStream_t s) {
  using L = CodebookLayout<D, B>;
  DequantArgs a{};
  a.codes = w.codes + (int64_t)expert * w.rows * w.wr;
  a.codebook = w.codebook + (w.cb_per_expert ? (int64_t)expert * (1 << B) * D : 0);
  a.scales = w.scales + (int64_t)expert * w.rows * (w.cols / G);
  a.out = out;
  a.rows = w.rows;
  a.cols = w.cols;
  a.wr = w.wr;
  a.spr = w.cols / G;
  a.P = w.cols / (16 * D);
  const int64_t chunks = (int64_t)a.rows * a.P;
  const int blocks = (int)std::min<int64_t>((chunks + 255) / 256, (int64_t)num_cus() * 4);
  auto k = vq_dequant_kernel<D, B, G>;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

#define VQMI_GEOMS(X) \
  X(2, 8, 64) X(2, 8, 128) X(2, 12, 64) X(2, 12, 128) \
  X(4, 8, 64) X(4, 8, 128) X(4, 12, 64) X(4, 12, 128) \
  X(8, 8, 64) X(8, 8, 128) X(8, 12, 64) X(8, 12, 128)

hipError_t launch_gemv(const TensorView& w, const uint16_t* x, int T, float* y,
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s) {
#define X(D, B, G)                                                   \
  if (w.d == D && w.log2_k == B && w.group == G)                     \
    return gemv_geom<D, B, G>(w, x, T, y, ids, top_k, x_per_slot, s);
  VQMI_GEOMS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_dequant(const TensorView& w, int expert, uint16_t* out, hipStream_t s) {
#define X(D, B, G) \
  if (w.d == D && w.log2_k == B && w.group == G) return dequant_geom<D, B, G>(w, expert, out, s);
  VQMI_GEOMS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace vqmi
