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
//  * Each wave owns whole output rows and streams them on its own: no block
//    barrier after set-up and no cross-wave reduction.  A row's code stream
//    is walked in passes of 64 sixteen-code chunks, one chunk (16 or 24
//    bytes) per lane per pass, so every load instruction of a wave covers a
//    contiguous 1 KiB (or 1.5 KiB) run of the row.
//  * A ring of PD chunks per lane is kept in flight: the load for unit u + PD
//    (unit = one pass over one row) is issued as soon as unit u is consumed,
//    so a CU holds ~100-150 KiB of outstanding reads with one or two waves per
//    SIMD.  Loads are buffer loads (one SGPR descriptor, 32-bit lane offsets).
//  * x is staged once per block into LDS, zero-padded to whole passes and
//    swizzled so that the 16-byte x reads of eight consecutive chunks hit
//    eight different bank groups.
//  * The codebook sits in LDS; for K = 256 it is replicated so that a lane's
//    gather bank depends only on its lane id (conflict-free).
//  * Inner loop per code: one v_perm_b32 (LDS offset), one LDS read, d/2
//    v_dot2_f32_f16 per token; the group scale multiplies the group's sum
//    once (an fma per group).  The row total is a DPP reduction across the
//    wave; lane 63 stores it.
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
  int accumulate;         // add into y (column slices after the first)
  int T;                  // dense: tokens; routed: pairs
  int top_k;
  int num_experts;
  int x_per_slot;
};

// Prefetch depth (units in flight per lane) and largest token tile.
template <int D, int B>
struct GemvCfg {
  static constexpr int kPD = B == 8 ? 12 : 8;
};
constexpr int gemv_max_tt(int D) { return D == 8 ? 1 : 2; }

// Total of v over the 64 lanes of the wave, valid in lane 63.
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v = row16_sum(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

// x for up to TT tokens -> LDS.  Chunk p's S = 2d segments of 16 bytes sit
// at segment (p*(S+1) + q): one segment of padding per chunk, so the reads of
// segment q by eight consecutive chunks fall in eight different bank groups
// while q stays a compile-time offset.  Zero past the row end.  The codebook:
// the plain layout is copied directly; the replicated layout's 256 entries
// are copied raw to the area after x and expanded after a barrier.  Every
// load of a round is issued before the first is waited on.
template <int D, int B, int TT>
__device__ __forceinline__ void stage_x_and_codebook_impl(u32x4* xl, uint8_t* cb_lds,
                                                          const uint16_t* xb, const uint16_t* cb,
                                                          int cols, int ntok, int P, int xchunks,
                                                          int tid, int nt) {
  using L = CodebookLayout<D, B>;
  constexpr int S = 2 * D;
  constexpr int XR = 12;  // x segments in flight per thread per round
  const int xsegs = xchunks * (S + 1);       // per token, padded
  u32x4* raw = xl + TT * xsegs;
  u32x4 e = u32x4{0u, 0u, 0u, 0u};
  if constexpr (L::kReplicated) {
    if (tid < 256) {
      if constexpr (D == 2) e.x = reinterpret_cast<const uint32_t*>(cb)[tid];
      else if constexpr (D == 4) { const u32x2 t = reinterpret_cast<const u32x2*>(cb)[tid]; e.x = t.x; e.y = t.y; }
      else e = reinterpret_cast<const u32x4*>(cb)[tid];
    }
  }
  const int nseg = xchunks * S;               // segments per token (S is a power of two)
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const u32x4* src = reinterpret_cast<const u32x4*>(xb + (int64_t)tt * cols);
    const bool tok_ok = tt < ntok;
    for (int base = tid; base < nseg; base += XR * nt) {
      u32x4 v[XR];
#pragma unroll
      for (int u = 0; u < XR; ++u) {
        const int ls = base + u * nt;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (ls < nseg && (ls / S) < P && tok_ok) v[u] = src[ls];
      }
#pragma unroll
      for (int u = 0; u < XR; ++u) {
        const int ls = base + u * nt;
        if (ls < nseg) xl[tt * xsegs + (ls / S) * (S + 1) + (ls % S)] = v[u];
      }
    }
  }
  if constexpr (L::kReplicated) {
    if (tid < 256) raw[tid] = e;
  } else {
    stage_codebook<D, B>(cb_lds, cb, tid, nt);
  }
}

// Replicated layout: slot q (16 bytes) holds copies of entry q / 16, read
// from the raw copy in LDS (16 lanes share one address: a broadcast).
template <int D, int B>
__device__ __forceinline__ void expand_codebook_impl(uint8_t* cb_lds, const u32x4* raw, int tid, int nt) {
  using L = CodebookLayout<D, B>;
  if constexpr (L::kReplicated) {
    for (int q = tid; q < 4096; q += nt) {
      const u32x4 e = raw[q >> 4];
      u32x4 v;
      if constexpr (D == 2) v = u32x4{e.x, e.x, e.x, e.x};
      else if constexpr (D == 4) v = u32x4{e.x, e.y, e.x, e.y};
      else v = e;
      reinterpret_cast<u32x4*>(cb_lds)[q] = v;
    }
  }
}

template <int D, int B, int G, int TT, bool MOE>
__global__ __launch_bounds__(1024) void vq_gemv_kernel(GemvArgs a) {
  using L = CodebookLayout<D, B>;
  constexpr int PD = GemvCfg<D, B>::kPD;
  constexpr int NSC = (16 * D > G) ? (16 * D / G) : 1;  // scales per chunk
  constexpr int CPS = 16 / NSC;                          // codes per scale in a chunk
  constexpr int S = 2 * D;                               // 16-byte x segments per chunk
  constexpr int CB = Chunk<B>::kWords * 4;               // code bytes per chunk
  constexpr int MAXW = 16;                               // waves per block (max)
  static_assert(TT <= gemv_max_tt(D), "token tile too large for this d");

  __shared__ __align__(16) uint8_t cb_lds[L::kBytes];
  __shared__ float split_val[MAXW][2][TT];
  __shared__ int split_row[MAXW][2];
  extern __shared__ __align__(16) u32x4 xl[];           // [TT][chunks*(S+1)] segments + raw cb

  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int nw = nt >> 6;
  const int P = a.P;
  const int passes = a.passes;
  const int xchunks = passes * 64;
  const int xsegs = xchunks * (S + 1);                   // per token

  // ---- this block's rows, this wave's units (unit = one pass over a row) ----
  const int nblk = gridDim.x;
  const int brow0 = (int)((int64_t)a.rows * blockIdx.x / nblk);
  const int brows = (int)((int64_t)a.rows * (blockIdx.x + 1) / nblk) - brow0;
  const int units = brows * passes;
  const int ub = units * wave / nw;
  const int ue = units * (wave + 1) / nw;

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

  // ---- stage x and the codebook into LDS ----
  // These loads come ahead of the first ring loads so that their wait does
  // not include the HBM latency of the codes.
  stage_x_and_codebook_impl<D, B, TT>(xl, cb_lds, xb + (int64_t)a.p0 * 16 * D, cb, a.cols, ntok, P,
                                      xchunks, tid, nt);

  // ---- the prefetch ring ----
  const rsrc_t rc = make_rsrc(codes, (uint64_t)a.rows * a.wr * 4);
  const rsrc_t rs = make_rsrc(scales, (uint64_t)a.rows * a.spr * 2);
  const uint32_t row_cb = (uint32_t)a.wr * 4u;
  const uint32_t row_sb = (uint32_t)a.spr * 2u;
  const uint32_t lane_cb = (uint32_t)lane * CB;

  Chunk<B> ring[PD];
  uint16_t rsc[PD][NSC];
  int l_row = ub / passes, l_pass = ub - (ub / passes) * passes;  // next unit to load
  int l_left = ue - ub;
  // Loads are unconditional: a unit past the wave's last one gets an
  // out-of-range offset and reads zeros, so every unit slot issues the same
  // loads and the in-order vmcnt waits stay exact.
  auto load_unit = [&](Chunk<B>& c, uint16_t (&sc)[NSC]) {
    const bool live = l_left > 0;
    const uint32_t r = (uint32_t)(brow0 + l_row);
    const uint32_t cbase = r * row_cb + (uint32_t)((a.p0 + l_pass * 64) * CB);
    // chunks past the row end read in-bounds neighbours; masked out at use
    load_chunk<B>(c, rc, live ? cbase + lane_cb : kOutOfRange);
    const int gp = a.p0 + l_pass * 64 + lane;  // chunk within the full row
#pragma unroll
    for (int s = 0; s < NSC; ++s)
      sc[s] = buf_load_b16(rs, live ? r * row_sb + (uint32_t)(((gp * 16 * D) / G + s) * 2) : kOutOfRange);
    if (++l_pass == passes) { l_pass = 0; ++l_row; }
    --l_left;
  };
#pragma unroll
  for (int j = 0; j < PD; ++j) load_unit(ring[j], rsc[j]);
  __syncthreads();
  expand_codebook_impl<D, B>(cb_lds, xl + TT * xsegs, tid, nt);
  if (lane == 0) {
    split_row[wave][0] = -1;
    split_row[wave][1] = -1;
  }
  __syncthreads();

  const uint32_t lane_off = lane_copy_offset<D, B>(lane);
  float part[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) part[tt] = 0.f;
  int c_row = ub / passes, c_pass = ub - (ub / passes) * passes;  // next unit to compute
  const bool first_partial = c_pass != 0;  // the first row began in an earlier wave
  const int first_row = c_row;

  auto compute_unit = [&](const Chunk<B>& c, const uint16_t (&sc)[NSC]) {
    const int p = c_pass * 64 + lane;
    const u32x4* xs = xl + p * (S + 1);
    float g[TT], acc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[tt] = 0.f;
#pragma unroll
    for (int s = 0; s < NSC; ++s) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) g[tt] = 0.f;
#pragma unroll
      for (int i = s * CPS; i < (s + 1) * CPS; ++i) {
        const Entry<D> e = gather<D, B>(cb_lds, c, i, lane_off);
        const int q = (i * D) / 8;  // x segment holding code i's D columns
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const u32x4 xv = xs[tt * xsegs + q];
#pragma unroll
          for (int j = 0; j < D / 2; ++j) {
            const int w = ((i * D) / 2 + j) & 3;  // dword within the segment
            g[tt] = dot2(e.v[j], as_half2(w == 0 ? xv.x : w == 1 ? xv.y : w == 2 ? xv.z : xv.w), g[tt]);
          }
        }
      }
      const float scale = half_bits_to_float(sc[s]);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[tt] = __builtin_fmaf(g[tt], scale, acc[tt]);
    }
    const bool in_row = p < P;  // lanes past the row end (last pass) add nothing
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) part[tt] += in_row ? acc[tt] : 0.f;
    if (++c_pass == passes) {  // row complete: reduce across the wave
      const bool split = first_partial && c_row == first_row;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float v = wave_sum_to_lane63(part[tt]);
        if (lane == 63) {
          if (split) {
            split_val[wave][0][tt] = v;
          } else if (tt < ntok) {
            float* dst = yb + (int64_t)tt * a.rows + brow0 + c_row;
            *dst = a.accumulate ? *dst + v : v;
          }
        }
        part[tt] = 0.f;
      }
      if (split && lane == 63) split_row[wave][0] = c_row;
      c_pass = 0;
      ++c_row;
    }
  };

  const int u_total = ue - ub;
  for (int u0 = 0; u0 < u_total; u0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      if (u0 + j < u_total) compute_unit(ring[j], rsc[j]);  // wave-uniform branch
      load_unit(ring[j], rsc[j]);
    }
  }
  // an unfinished last row continues in the next wave(s)
  if (c_pass != 0) {
    const int slot = (first_partial && c_row == first_row) ? 0 : 1;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float v = wave_sum_to_lane63(part[tt]);
      if (lane == 63) split_val[wave][slot][tt] = v;
    }
    if (lane == 63) split_row[wave][slot] = c_row;
  }
  __syncthreads();
  // rows cut by a wave boundary: add the pieces in wave order (deterministic)
  for (int r = tid; r < brows; r += nt) {
    float v[TT];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) v[tt] = 0.f;
    for (int w = 0; w < nw; ++w) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (split_row[w][sl] == r) {
          any = true;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) v[tt] += split_val[w][sl][tt];
        }
      }
    }
    if (any) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt < ntok) {
          float* dst = yb + (int64_t)tt * a.rows + brow0 + r;
          *dst = a.accumulate ? *dst + v[tt] : v[tt];
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

// Raise the kernel's dynamic-LDS limit (set once per kernel and device;
// gfx950 has 160 KiB of LDS per CU).
template <typename K>
hipError_t allow_lds(K kernel) {
  static thread_local int done_dev = -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (done_dev == dev) return hipSuccess;
  hipFuncAttributes fa;
  e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)(160 * 1024 - fa.sharedSizeBytes));
  if (e == hipSuccess) done_dev = dev;
  return e;
}

constexpr int kGemvWaves = 16;  // waves per block

template <int D, int B, int G, int TT, bool MOE>
hipError_t gemv_launch(const GemvArgs& a, dim3 grid, hipStream_t s) {
  using L = CodebookLayout<D, B>;
  const size_t lds = ((size_t)TT * a.passes * 64 * (2 * D + 1) + 256) * 16;  // dynamic: x + raw codebook
  auto k = vq_gemv_kernel<D, B, G, TT, MOE>;
  hipError_t e = allow_lds(k);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, grid, dim3(64 * kGemvWaves), lds, s, a);
  return hipGetLastError();
}

// Column-slice size (in 16-code chunks) whose x, padded, fits in the LDS the
// codebook leaves free.
template <int D, int B, int TT>
int gemv_max_slice_chunks() {
  using L = CodebookLayout<D, B>;
  const int budget = 160 * 1024 - L::kBytes - 256 * 16 - 2048;  // minus raw codebook, split slots
  const int per_pass = 64 * (2 * D + 1) * 16 * TT;
  return std::max(1, budget / per_pass) * 64;
}

template <int D, int B, int G, int TT, bool MOE>
hipError_t gemv_slices(GemvArgs a, int P_total, dim3 grid, hipStream_t s) {
  const int maxc = gemv_max_slice_chunks<D, B, TT>();
  const int n_slices = (P_total + maxc - 1) / maxc;
  const int per = (P_total + n_slices - 1) / n_slices;
  for (int sl = 0; sl < n_slices; ++sl) {
    a.p0 = sl * per;
    a.P = std::min(per, P_total - a.p0);
    a.passes = (a.P + 63) / 64;
    a.accumulate = sl > 0;
    hipError_t e = gemv_launch<D, B, G, TT, MOE>(a, grid, s);
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
  // one block of kGemvWaves waves per CU across the whole grid (all token
  // tiles / pairs); rows are split evenly over blocks and units evenly over
  // the waves of a block
  const int tt = std::min(T >= 2 ? 2 : 1, gemv_max_tt(D));
  const int ycount = ids ? T * top_k : (T + tt - 1) / tt;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(w.rows, num_cus() / std::max(1, ycount)));
  dim3 grid(blocks, ycount);
  if (ids) {
    a.T = T * top_k;
    return gemv_slices<D, B, G, 1, true>(a, P_total, grid, s);
  }
  a.T = T;
  if constexpr (gemv_max_tt(D) >= 2) {
    if (tt == 2) return gemv_slices<D, B, G, 2, false>(a, P_total, grid, s);
  }
  return gemv_slices<D, B, G, 1, false>(a, P_total, grid, s);
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
