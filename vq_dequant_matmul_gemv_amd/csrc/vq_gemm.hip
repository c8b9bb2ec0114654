// vq_gemm.hip -- the on-device routing that groups (token, slot) pairs by
// expert for the grouped GEMM, the fill kernels, the static scratch of
// vq_moe_gemm_no_alloc, and the dispatch of the prefill-shaped kernels by
// code width (vq_gemm_bNN.hip; the kernels are in vq_gemm_impl.h).
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

// Zero n 32-bit words (16-byte stores where aligned), grid-stride.
__global__ __launch_bounds__(256) void vq_zero_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = ((reinterpret_cast<uintptr_t>(p) & 15) == 0) ? n / 4 : 0;
  for (int64_t i = i0; i < n4; i += stride) reinterpret_cast<u32x4*>(p)[i] = u32x4{0u, 0u, 0u, 0u};
  for (int64_t i = 4 * n4 + i0; i < n; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// routing: group (token, slot) pairs by expert and emit the token-tile list.
// One block; pairs and experts are walked in strides of the block size.
// Workspace layout (int32): counts[E] | offsets[E] | fill[E] | tile_base[E] |
// n_tiles[1] | n_wide[1] | pad to 4 | pairs[npairs] | tiles[max_tiles][3]
// ---------------------------------------------------------------------------

struct RouteArgs {
  const int32_t* ids;
  int32_t* ws;
  void* y;            // skipped slots' output rows are zeroed (nullptr: none to zero)
  int y_row_halves;   // 16-bit words per output row
  int npairs, num_experts;
  int wide;           // list 128-pair tiles for hot experts
};

// An expert's tiles: with wide tiles, one per whole kMoeWideTokens pairs and
// one for a remainder above kMoeWideMin; a smaller remainder (or every pair,
// without wide tiles) in tiles of kMoeTileTokens.
__device__ __forceinline__ void expert_tiles(int c, bool wide, int& nw, int& nt) {
  const int r = wide ? c % kMoeWideTokens : c;
  nw = wide ? c / kMoeWideTokens + (r > kMoeWideMin ? 1 : 0) : 0;
  nt = (wide && r > kMoeWideMin) ? 0 : (r + kMoeTileTokens - 1) / kMoeTileTokens;
}

// Experts whose counters fit in LDS (two int32 per expert); more experts use
// the workspace copies.  Counters in LDS matter: with skewed routing hundreds
// of pairs add to one hot expert's counter, and global atomics on one address
// serialize at L2 (tens of microseconds per call), LDS atomics do not.
constexpr int kRouteLdsExperts = 8192;

// Pairs a thread of the routing block keeps in registers (id and rank within
// its expert) between counting and scattering: up to 16 x 1024 pairs the ids
// are read once and every pair's place comes from its counting atomic, with
// no second pass of atomics; larger calls take the two-pass path.
constexpr int kRouteRegPairs = 16;

template <bool kLds>
__device__ __forceinline__ void route_pairs(const RouteArgs& a, int32_t* counts, int32_t* fill, int32_t* part) {
  const int E = a.num_experts;
  int32_t* tbase = a.ws + 3 * E;
  int32_t* n_tiles = moe_ws_n_tiles(a.ws, E);
  int32_t* n_wide = moe_ws_n_wide(a.ws, E);
  const bool wide = a.wide != 0;
  int32_t* pairs = moe_ws_pairs(a.ws, E);
  int32_t* tiles = moe_ws_tiles(a.ws, E, a.npairs);
  const int tid = threadIdx.x, nt = blockDim.x;
  // one pass (LDS counters, pairs held in registers) or two (counters and
  // their second use in the workspace, or too many pairs)
  const bool one_pass = kLds && a.npairs <= kRouteRegPairs * nt;
  // expert offsets: in LDS (the fill counters are not needed) on the one-pass
  // path, in the workspace otherwise
  int32_t* offsets = one_pass ? fill : a.ws + E;
  int32_t my_e[kRouteRegPairs], my_rank[kRouteRegPairs];

  for (int e = tid; e < E; e += nt) { counts[e] = 0; fill[e] = 0; }
  __syncthreads();
  if (one_pass) {
    // every id load in flight at once (an index past the end reads pair 0,
    // then is dropped), then the counting atomics
#pragma unroll
    for (int k = 0; k < kRouteRegPairs; ++k) {
      const int p = tid + k * nt;
      my_e[k] = a.ids[p < a.npairs ? p : 0];
    }
#pragma unroll
    for (int k = 0; k < kRouteRegPairs; ++k) {
      const int p = tid + k * nt;
      const int e = my_e[k];
      const bool ok = p < a.npairs && e >= 0 && e < E;
      my_e[k] = ok ? e : -1;
      my_rank[k] = ok ? atomicAdd(&counts[e], 1) : -1;
    }
  } else {
    for (int p = tid; p < a.npairs; p += nt) {
      const int e = a.ids[p];
      if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
    }
  }
  __syncthreads();
  // exclusive scans of the pair counts, the wide tiles and the 32-pair tiles
  // per expert: each thread owns a contiguous run of experts
  const int per = (E + nt - 1) / nt;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int sc = 0, sw = 0, st = 0;
  for (int e = e0; e < e1; ++e) {
    int nw_e, nt_e;
    expert_tiles(counts[e], wide, nw_e, nt_e);
    sc += counts[e];
    sw += nw_e;
    st += nt_e;
  }
  // The three scans at once: inclusive within each wave by shuffles, then
  // over the (at most 16) wave totals by the first wave; two barriers in all.
  const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
  int ic = sc, iw = sw, it = st;
  for (int off = 1; off < 64; off <<= 1) {
    const int c = __shfl_up(ic, off, 64), w = __shfl_up(iw, off, 64), t = __shfl_up(it, off, 64);
    if (lane >= off) { ic += c; iw += w; it += t; }
  }
  if (lane == 63) { part[wid] = ic; part[32 + wid] = iw; part[64 + wid] = it; }
  __syncthreads();
  if (wid == 0) {
    const int wc = lane < nw ? part[lane] : 0, ww = lane < nw ? part[32 + lane] : 0;
    const int wt = lane < nw ? part[64 + lane] : 0;
    int jc = wc, jw = ww, jt = wt;
    for (int off = 1; off < 32; off <<= 1) {
      const int c = __shfl_up(jc, off, 64), w = __shfl_up(jw, off, 64), t = __shfl_up(jt, off, 64);
      if (lane >= off) { jc += c; jw += w; jt += t; }
    }
    if (lane < nw) { part[96 + lane] = jc - wc; part[128 + lane] = jw - ww; part[160 + lane] = jt - wt; }
    if (lane == nw - 1) {
      part[192] = jw;  // wide tiles in all: the 32-pair tiles follow them
      *n_tiles = jw + jt;
      *n_wide = jw;
    }
  }
  __syncthreads();
  const int total_w = part[192];
  int run_c = part[96 + wid] + ic - sc;
  int run_w = part[128 + wid] + iw - sw;
  int run_t = total_w + part[160 + wid] + it - st;
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run_c;
    const int c = counts[e];
    int nw_e, nt_e;
    expert_tiles(c, wide, nw_e, nt_e);
    tbase[e] = nw_e > 0 ? run_w : run_t;
    for (int k = 0; k < nw_e; ++k) {
      int32_t* t = tiles + 3 * (run_w + k);
      t[0] = e;
      t[1] = run_c + k * kMoeWideTokens;
      t[2] = min(kMoeWideTokens, c - k * kMoeWideTokens);
    }
    const int c0 = nw_e * kMoeWideTokens;  // pairs the wide tiles took
    for (int k = 0; k < nt_e; ++k) {
      int32_t* t = tiles + 3 * (run_t + k);
      t[0] = e;
      t[1] = run_c + c0 + k * kMoeTileTokens;
      t[2] = min(kMoeTileTokens, c - c0 - k * kMoeTileTokens);
    }
    run_c += c;
    run_w += nw_e;
    run_t += nt_e;
  }
  __syncthreads();
  auto skipped = [&](int p) {  // skipped slot: zero its output row
    if (a.y) {
      uint16_t* yr = static_cast<uint16_t*>(a.y) + (int64_t)p * a.y_row_halves;
      for (int r = 0; r < a.y_row_halves; ++r) yr[r] = 0;
    }
  };
  if (one_pass) {
#pragma unroll
    for (int k = 0; k < kRouteRegPairs; ++k) {
      const int p = tid + k * nt;
      if (my_e[k] >= 0) pairs[offsets[my_e[k]] + my_rank[k]] = p;
      else if (p < a.npairs) skipped(p);
    }
  } else {
    for (int p = tid; p < a.npairs; p += nt) {
      const int e = a.ids[p];
      if (e >= 0 && e < E) {
        const int pos = offsets[e] + atomicAdd(&fill[e], 1);
        pairs[pos] = p;
      } else {
        skipped(p);
      }
    }
  }
}

__global__ __launch_bounds__(1024) void vq_route_kernel(RouteArgs a) {
  __shared__ int32_t part[1024];
  __shared__ int32_t lds_counts[kRouteLdsExperts], lds_fill[kRouteLdsExperts];
  if (a.num_experts <= kRouteLdsExperts) {
    route_pairs<true>(a, lds_counts, lds_fill, part);
  } else {
    route_pairs<false>(a, a.ws, a.ws + 2 * a.num_experts, part);
  }
}

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

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (vq_moe_gemm_no_alloc): the
// routing workspace lives in this file-scope device array, one copy per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the device symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
// ---------------------------------------------------------------------------

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n / 4 + 255) / 256 + 1, (int64_t)num_cus() * 4);
  hipLaunchKernelGGL(vq_zero_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

size_t moe_workspace_bytes(int T, int top_k, int num_experts) {
  const int64_t npairs = (int64_t)T * top_k;
  if (npairs <= 0) return 0;
  const int64_t mt = (npairs + kMoeTileTokens - 1) / kMoeTileTokens + num_experts;
  const int64_t words = ((4 * (int64_t)num_experts + 1 + 3) & ~3) + ((npairs + 3) & ~3) + 3 * mt;
  return (size_t)(words * 4);
}
hipError_t launch_gemm(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s) {
  switch (w.log2_k) {
#define X(B) \
  case B: return gemm_b##B(w, io, x, T, y, s);
    VQMI_BITS(X)
#undef X
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_route(const int32_t* ids, int npairs, int num_experts, int32_t* ws, void* y_skip, int y_row_halves,
                        bool wide, hipStream_t s) {
  RouteArgs r{};
  r.ids = ids;
  r.ws = ws;
  r.y = y_skip;
  r.y_row_halves = y_row_halves;
  r.npairs = npairs;
  r.num_experts = num_experts;
  r.wide = wide ? 1 : 0;
  hipLaunchKernelGGL(vq_route_kernel, dim3(1), dim3(1024), 0, s, r);
  return hipGetLastError();
}

// Zero y for the combine step, then (in the code width's unit) route and run
// the grouped GEMM.
hipError_t launch_moe_gemm(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot,
                           const int32_t* ids, int T, int top_k, void* y, void* ws, hipStream_t s) {
  int32_t* wsi = static_cast<int32_t*>(ws);
  if (io.epi == kEpiCombine) {  // the slots add into y: zero it first
    hipError_t e = launch_zero(y, (size_t)T * w.rows * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  switch (w.log2_k) {
#define X(B) \
  case B: return moe_gemm_b##B(w, io, x, x_per_slot, ids, T, top_k, y, wsi, s);
    VQMI_BITS(X)
#undef X
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace vqmi
