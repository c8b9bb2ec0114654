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
//  * A block owns a contiguous range of rows.  Its waves walk the range in
//    row groups: a group is 64 / L rows, each row served by L lanes, each lane
//    holding C sixteen-code chunks of the row (chunks li, li + L, ... of the
//    pass), so one load instruction reads a contiguous run of every row of the
//    group and all 64 lanes are busy.  A row longer than L*C chunks is covered
//    in several passes of equal width whose partial sums meet in LDS; a pass
//    count dividing the waves lets every wave keep one pass (and its x).
//  * Everything small is staged once per block, before any compute: the x
//    columns of the launch, the block's scales and the codebook (replicated
//    for K = 256 so that a lane's gather bank depends only on its lane id).
//    The per-row stream then carries only code loads, one 16-byte (or 24-byte)
//    load per chunk and lane: the number of memory instructions in flight
//    per CU, not their bytes, is what limits a streaming kernel here, so no
//    instruction is spent on a 2-byte scale.
//  * x sits in VGPRs for a whole pass (x-stationary); the inner loop per code
//    is one v_perm_b32 (LDS offset), one LDS gather and d/2 v_dot2_f32_f16;
//    the group scale multiplies each group sum once.
//  * Several tokens run as one grid slice each (blockIdx.y), re-reading the
//    codes per token: above a few tokens the MFMA GEMM is the faster kernel
//    and the C ABI's vq_gemv hands such calls to it.
//  * Each wave keeps P row groups' loads in flight (P items of C chunks per
//    lane, about six chunks in all): wide items (d = 2, five chunks per lane)
//    keep one, since a deeper ring only holds the wave at the issue of loads
//    that cannot enter the CU's full memory queue; narrow ones (d = 4 and 8)
//    keep up to four.  A slot's next item is loaded chunk by chunk, each
//    chunk as soon as its codebook gathers are issued, so the loads leave
//    during the compute without adding to the loads in flight.
//  * Routed experts (top-k MoE): blockIdx.y is the (token, slot) pair; the
//    block reads its expert id and points at that expert's codes and scales.
//    An id outside [0, E) writes a zero row.  Dense projections sharing x
//    (gate and up) run the same way as a two-expert stack in one launch.

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
  int rows_base, rows_extra;  // block b owns rows_base (+1 if b < rows_extra) rows
  int q0, nq;             // column slice of this launch, in 16-code chunks
  int lanes_log2;         // L = 1 << lanes_log2 lanes per row (2..5)
  int passes;             // ceil(nq / (L * C))
  int accumulate;         // add into y (column slices after the first)
  int T;                  // dense: tokens; routed: pairs
  int tok0;               // dense: first token of this launch
  int top_k;
  int num_experts;
  int x_per_slot;
};

constexpr int kGemvWaves = 8;                  // two waves per SIMD
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvXMaxBytes = 40 * 1024;      // largest x slice in LDS
constexpr int kGemvScaleBytes = 24 * 1024;     // the block's scale rows (136 rows of 80 groups fit)
constexpr int kGemvPieces = 4096;              // per-(row, pass) partial sums

// Chunks per lane a pass can hold in VGPRs: x costs 8*d VGPRs per chunk.
__host__ __device__ constexpr int gemv_max_c(int D) { return D == 2 ? 5 : (D == 4 ? 3 : 1); }

// Items a wave keeps in flight: about six 16-code chunks per lane in all, so
// narrow items (few chunks per lane) still put enough bytes on the wire per
// memory round trip.
__host__ __device__ constexpr int gemv_ring(int C) { return C >= 4 ? 1 : (C == 3 ? 2 : (C == 2 ? 3 : 4)); }

// Sum of v over aligned groups of L = 1 << lg lanes; valid in the group's last lane.
__device__ __forceinline__ float lane_group_sum(float v, int lg) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: every lane holds its quad's sum
  if (lg >= 3) v += dpp_mov<0x141>(v);  // row_half_mirror: 8-lane sums
  if (lg >= 4) v += dpp_mov<0x140>(v);  // row_mirror: 16-lane sums
  if (lg >= 5)                          // row_bcast15: rows 1 and 3 add rows 0 and 2
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  return v;
}

// XS: the x slice takes XS * 8 KiB of LDS (2 or 5); fewer staging loads for
// short rows.
template <int D, int B, int G, int C, int XS, bool MOE>
//
// The arguments a block needs before its first loads come first, as scalars:
// with kernel-argument preloading (the build passes
// -amdgpu-kernarg-preload-count) they arrive in SGPRs at wave launch instead
// of after a scalar load from the argument buffer.  The rest (output,
// routing, accumulation) is only needed later and stays in the struct.
//   xs: x of token tok0 (dense) or x (routed); shape = nq | lanes_log2 << 12 |
//   passes << 15 | pass width << 23 (chunks per pass, at most L * C); cols =
//   spr * G.
__global__ __launch_bounds__(kGemvThreads) void vq_gemv_kernel(
    const uint32_t* __restrict__ codes_in, const uint16_t* __restrict__ cb_in,
    const uint16_t* __restrict__ scales_in, const uint16_t* __restrict__ xs, int rows, int rows_base,
    int rows_extra, int q0, int spr, uint32_t shape, GemvArgs a) {
  using LY = CodebookLayout<D, B>;
  constexpr int NSC = (16 * D > G) ? (16 * D / G) : 1;  // scales per chunk
  constexpr int CPS = 16 / NSC;                          // codes per scale in a chunk
  constexpr int HX = 8 * D;                              // half2 of x per chunk
  constexpr int CB = Chunk<B>::kWords * 4;               // code bytes per chunk
  constexpr int NW = kGemvWaves;
  constexpr int NT = kGemvThreads;
  static_assert(C <= gemv_max_c(D), "tile does not fit the VGPR budget");

  __shared__ __align__(16) uint8_t cb_lds[LY::kBytes];
  constexpr int XBYTES = XS * 8192;
  __shared__ __align__(16) uint8_t x_lds[XBYTES];                   // [nq * 16 * D] fp16
  __shared__ __align__(16) uint8_t s_lds[kGemvScaleBytes];          // the block's scale rows
  __shared__ float pieces[kGemvPieces];                             // [rows][passes]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nq = (int)(shape & 0xfffu);
  const int lg = (int)((shape >> 12) & 0x7u);
  const int passes = (int)((shape >> 15) & 0xffu);
  const int PW = (int)(shape >> 23);       // chunks per pass; the last pass may hold fewer
  const int cols = spr * G;
  const int wr = cols / (32 * D) * B;     // code words per row
  const int L = 1 << lg;
  const int R = 64 >> lg;                 // rows per group
  const int rsub = lane >> lg;            // this lane's row within the group
  const int li = lane & (L - 1);          // this lane's position within the row

  // ---- this block's rows ----
  const int bid = blockIdx.x;
  const int brow0 = bid * rows_base + min(bid, rows_extra);
  const int brows = rows_base + (bid < rows_extra ? 1 : 0);
  const int ngroups = (brows + R - 1) / R;

  const uint32_t* codes = codes_in;
  const uint16_t* scales = scales_in;
  const uint16_t* cb = cb_in;
  const uint16_t* xb;
  float* yb;
  if constexpr (MOE) {
    const int pair = blockIdx.y;
    const int e = a.ids[pair];
    yb = a.y + (int64_t)pair * rows;
    if (e < 0 || e >= a.num_experts) {  // skipped slot: zero rows (block-uniform exit)
      if (!a.accumulate)
        for (int r = tid; r < brows; r += NT) yb[brow0 + r] = 0.f;
      return;
    }
    codes += (int64_t)e * a.code_estride;
    scales += (int64_t)e * a.scale_estride;
    cb += (int64_t)e * a.cb_estride;
    xb = xs + (int64_t)(a.x_per_slot ? pair : pair / a.top_k) * cols;
  } else {
    xb = xs + (int64_t)blockIdx.y * cols;  // one token per grid slice
    yb = a.y + (int64_t)(a.tok0 + blockIdx.y) * rows;
  }

  // ---- small loads first: x slice, codebook entries, the block's scales ----
  const int xcols = nq * 16 * D;                        // columns of the slice
  const uint32_t xbytes = (uint32_t)xcols * 2u;
  constexpr int XL = (XBYTES + NT * 16 - 1) / (NT * 16);
  u32x4 xg[XL];
  const rsrc_t rx = make_rsrc(xb, (uint64_t)cols * 2);
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const uint32_t o = (uint32_t)(tid + q * NT) * 16u;  // byte in the x slice
    xg[q] = buf_load_b128(rx, o < xbytes ? (uint32_t)q0 * 32u * D + o : kOutOfRange);
  }
  // codebook (replicated layout): lane l < 32 of wave w holds entry 32 w + l
  u32x4 ce = u32x4{0u, 0u, 0u, 0u};
  if constexpr (LY::kReplicated) {
    static_assert(NW * 32 == 256, "one codebook entry per lane of the first half-waves");
    if (lane < 32) {
      const int ent = wave * 32 + lane;
      if constexpr (D == 2) ce.x = reinterpret_cast<const uint32_t*>(cb)[ent];
      else if constexpr (D == 4) { const u32x2 t = reinterpret_cast<const u32x2*>(cb)[ent]; ce.x = t.x; ce.y = t.y; }
      else ce = reinterpret_cast<const u32x4*>(cb)[ent];
    }
  }
  // scale rows [brow0, brow0 + brows), read as 16-byte pieces from a 16-byte
  // boundary at or below the first scale
  const uint64_t s_first = (uint64_t)brow0 * spr * 2u;
  const uint32_t s_skew = (uint32_t)(s_first & 15u);
  const uint32_t s_span = (uint32_t)brows * (uint32_t)spr * 2u + s_skew;
  const uint32_t s_avail = (uint32_t)((uint64_t)rows * spr * 2u - (s_first - s_skew));  // to the tensor's end
  const rsrc_t rsb = make_rsrc(reinterpret_cast<const uint8_t*>(scales) + (s_first - s_skew), s_avail);
  constexpr int SL = (kGemvScaleBytes + NT * 16 - 1) / (NT * 16);
  u32x4 sg[SL];
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const uint32_t o = (uint32_t)(tid + q * NT) * 16u;
    sg[q] = buf_load_b128(rsb, (o < s_span && o + 16u <= s_avail) ? o : kOutOfRange);
    if (o < s_span && o + 16u > s_avail) {  // the tensor ends inside this piece: 2-byte loads
      uint32_t h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) h[k] = buf_load_b16(rsb, o + 2u * k < s_avail ? o + 2u * k : kOutOfRange);
      sg[q] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }

  // Every wave's small loads enter the CU's in-order memory queue ahead of
  // any wave's code loads (a plain s_barrier: it waits for no load).
  __builtin_amdgcn_s_barrier();

  // ---- the code stream: work item u = (pass, group) in pass-major order ----
  const rsrc_t rc = make_rsrc(codes, (uint64_t)rows * wr * 4);
  const uint32_t row_cb = (uint32_t)wr * 4u;
  // items f = group * passes + pass, dealt round-robin over the waves: when
  // the wave count is a multiple of the pass count a wave keeps one pass (no
  // x reloads), and the block's waves always read neighbouring row groups.
  const int total_items = ngroups * passes;
  const int step_g = NW / passes, step_p = NW - step_g * passes;  // f += NW
  const int n_items = total_items > wave ? (total_items - wave + NW - 1) / NW : 0;
  constexpr int P = gemv_ring(C);
  Chunk<B> ring[P][C];                                  // codes of the items in flight
  int l_item = 0;                                       // next item to load
  int l_pass = wave % passes, l_g = wave / passes;  // its pass and group
  uint32_t lane_vo[C];                                  // per-lane code offsets of l_pass
  auto set_pass_offsets = [&](int pass) {
    const int lim = min(PW, nq - pass * PW);            // chunks of this pass
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int qp = j * L + li;                        // chunk within the pass
      const uint32_t vo = (uint32_t)rsub * row_cb + (uint32_t)(q0 + pass * PW + qp) * CB;
      lane_vo[j] = qp < lim ? vo : kOutOfRange;
    }
  };
  set_pass_offsets(l_pass);
  // Loads are unconditional: a chunk past the slice, a row past the block or
  // an item past the wave's list gets an out-of-range offset and reads zeros,
  // so every item issues the same loads and the in-order vmcnt waits stay exact.
  // An item's loads are issued chunk by chunk (load_chunk) between
  // load_begin, which fixes the item's rows, and load_end, which moves on.
  struct NextLoad {
    uint32_t so;   // byte offset of the group's first row
    bool rowok;    // this lane's row exists and the item is on the wave's list
  };
  auto load_begin = [&]() {
    const bool live = l_item < n_items;
    const int r = brow0 + l_g * R;                      // first row of the group
    // the row offset is wave-uniform; saying so keeps it in an SGPR (the
    // buffer load's soffset) across the item loop
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane((int)(live ? (uint32_t)r * row_cb : 0u));
    return NextLoad{so, live && l_g * R + rsub < brows};
  };
  auto load_chunk = [&](Chunk<B>& dst, int j, const NextLoad& nl) {
    const uint32_t vo = nl.rowok ? lane_vo[j] : kOutOfRange;
    if constexpr (B == 8) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, vo, nl.so, 0));
      dst.w[0] = v.x; dst.w[1] = v.y; dst.w[2] = v.z; dst.w[3] = v.w;
    } else {
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, vo + 8u * h, nl.so, 0));
        dst.w[2 * h] = v.x; dst.w[2 * h + 1] = v.y;
      }
    }
  };
  auto load_end = [&]() {
    ++l_item;
    l_g += step_g;
    l_pass += step_p;
    if (l_pass >= passes) { l_pass -= passes; ++l_g; }
    if (step_p != 0) set_pass_offsets(l_pass);
  };
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const NextLoad nl = load_begin();
#pragma unroll
    for (int j = 0; j < C; ++j) load_chunk(ring[k][j], j, nl);
    load_end();
  }

  // ---- stage the small data in LDS ----
  if constexpr (LY::kReplicated) {
    // Wave w fills slots [512 w, 512 w + 512) of the 4096 16-byte slots (slot
    // q holds copies of entry q / 16): lane l writes slots 512 w + 64 k + l,
    // copies of entry 32 w + 4 k + l / 16, which lane 4 k + l / 16 of the same
    // wave holds -- a cross-lane permute, no LDS round trip or extra barrier.
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int src = (4 * k + (lane >> 4)) * 4;
      u32x4 e;
      e.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)ce.x);
      e.y = D >= 4 ? (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)ce.y) : 0u;
      e.z = D == 8 ? (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)ce.z) : 0u;
      e.w = D == 8 ? (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)ce.w) : 0u;
      u32x4 v;
      if constexpr (D == 2) v = u32x4{e.x, e.x, e.x, e.x};
      else if constexpr (D == 4) v = u32x4{e.x, e.y, e.x, e.y};
      else v = e;
      reinterpret_cast<u32x4*>(cb_lds)[wave * 512 + 64 * k + lane] = v;
    }
  }
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const uint32_t o = (uint32_t)(tid + q * NT) * 16u;
    if (o < (uint32_t)XBYTES) *reinterpret_cast<u32x4*>(x_lds + o) = xg[q];
  }
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const uint32_t o = (uint32_t)(tid + q * NT) * 16u;
    if (o < (uint32_t)kGemvScaleBytes) *reinterpret_cast<u32x4*>(s_lds + o) = sg[q];
  }
  if constexpr (!LY::kReplicated) stage_codebook<D, B>(cb_lds, cb, tid, NT);
  lds_barrier();

  const uint32_t lane_off = lane_copy_offset<D, B>(lane);
  half2_t xv[C][HX];
  uint32_t lane_sq[C], lane_ok[C];  // per pass: scale byte offset in the row, chunk-valid mask
  int cur_pass = -1;
  int pass = wave % passes, g = wave / passes;
  auto item = [&](Chunk<B> (&rs)[C]) {
    if (pass != cur_pass) {  // x of this pass into VGPRs (zeros past the slice)
      cur_pass = pass;
      const int lim = min(PW, nq - pass * PW);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const int qp = j * L + li;
        const int q = pass * PW + qp;
        const bool ok = qp < lim;
        lane_sq[j] = ((uint32_t)(q0 + q) * 16u * D) / G * 2u;
        lane_ok[j] = ok ? 0xffffffffu : 0u;
#pragma unroll
        for (int k = 0; k < HX / 4; ++k) {
          u32x4 v = u32x4{0u, 0u, 0u, 0u};
          if (ok) v = *reinterpret_cast<const u32x4*>(x_lds + (uint32_t)q * 32u * D + 16u * k);
          xv[j][4 * k + 0] = as_half2(v.x);
          xv[j][4 * k + 1] = as_half2(v.y);
          xv[j][4 * k + 2] = as_half2(v.z);
          xv[j][4 * k + 3] = as_half2(v.w);
        }
      }
    }

    const int rb = g * R + rsub;                        // row within the block
    const uint32_t srow = s_skew + (uint32_t)rb * (uint32_t)spr * 2u;  // the row's scales in s_lds
    const uint32_t rowok = rb < brows ? 0xffffffffu : 0u;
    float acc = 0.f;
    // The gathers of step t + 1 are issued before the dot products of step
    // t; a step is SB codes of one chunk (16 for d = 2, 8 for d = 4, 4 for
    // d = 8), so the gathered entries in flight take 2 * SB * d / 2 = 32 VGPRs
    // whatever d, and wide x-stationary tiles (5 chunks per lane) fit for d = 4
    // too.  Everything is computed unconditionally; a chunk past the slice or
    // a row past the block is dropped with a bit mask (a select would let the
    // compiler branch around the gathers).
    constexpr int S = (D == 2) ? 1 : (D == 4 ? 2 : 4);  // steps per chunk
    constexpr int SB = 16 / S;                          // codes per step
    static_assert(CPS % SB == 0, "a step lies inside one scale group");
    //
    // This slot's next item (u + P) is loaded chunk by chunk: once the last
    // gather of chunk j is issued, the chunk's code registers are free and its
    // load for the next item goes out at once.  The wave so keeps C chunk
    // loads in flight, no more than loading whole items after the compute,
    // but they leave during the compute rather than after it.
    const NextLoad nl = load_begin();
    Entry<D> e[2][SB];
    auto issue = [&](int t, Entry<D> (&dst)[SB]) {
#pragma unroll
      for (int i = 0; i < SB; ++i) dst[i] = gather<D, B>(cb_lds, rs[t / S], (t % S) * SB + i, lane_off);
      if (t % S == S - 1) {  // kept in place: the scheduler would sink it below later waits
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(rs[t / S], t / S, nl);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    issue(0, e[0]);
    float gs[2] = {0.f, 0.f};  // two chains for ILP, restarted per scale group
#pragma unroll
    for (int t = 0; t < C * S; ++t) {
      if (t + 1 < C * S) issue(t + 1, e[(t + 1) & 1]);
      const int j = t / S, b = t % S;
#pragma unroll
      for (int ii = 0; ii < SB; ++ii) {
        const int i = b * SB + ii;
#pragma unroll
        for (int k = 0; k < D / 2; ++k)
          gs[(i * (D / 2) + k) & 1] = dot2(e[t & 1][ii].v[k], xv[j][i * (D / 2) + k], gs[(i * (D / 2) + k) & 1]);
      }
      if (((b + 1) * SB) % CPS == 0) {  // the step ends scale group s2 of chunk j
        const int s2 = (b + 1) * SB / CPS - 1;
        const uint32_t keep = lane_ok[j] & rowok;
        const uint16_t sbits = *reinterpret_cast<const uint16_t*>(s_lds + ((srow + lane_sq[j] + 2u * s2) & keep));
        const float scale = half_bits_to_float(sbits);
        const float gsum = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, gs[0] + gs[1]) & keep);
        acc = __builtin_fmaf(gsum, __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, scale) & keep), acc);
        gs[0] = gs[1] = 0.f;
      }
    }
    const float v = lane_group_sum(acc, lg);
    if (li == L - 1 && rb < brows) pieces[rb * passes + pass] = v;
    load_end();
    g += step_g;
    pass += step_p;
    if (pass >= passes) { pass -= passes; ++g; }
  };
  // Slot k of the ring holds items k, k + P, k + 2P, ...: unrolled by P so
  // every slot is a fixed set of registers.  The wave runs its item count
  // rounded up to P; the extra items read zeros (their loads are out of
  // range) and store nothing (their rows lie past the block).  With no
  // branch and no global store in the loop, every wait for a slot's codes
  // leaves the other slots' loads in flight.
  for (int u0 = 0; u0 < n_items; u0 += P) {
#pragma unroll
    for (int k = 0; k < P; ++k) item(ring[k]);
  }

  {  // y: each row's pass pieces added in pass order (deterministic)
    __syncthreads();
    for (int r = tid; r < brows; r += NT) {
      float v = 0.f;
      for (int c = 0; c < passes; ++c) v += pieces[r * passes + c];
      float* dst = yb + brow0 + r;
      *dst = a.accumulate ? *dst + v : v;
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

// Lane tiling of a slice of nq chunks: L = 1 << lg lanes per row, C chunks
// per lane, `passes` passes of ceil(nq / passes) chunks each (the kernel
// derives the same pass width).  The bytes per row group (L * C chunks per
// row) set how much every memory round trip of a wave delivers, so the
// widest pass wins, among tilings that leave at most a quarter of the
// lane-chunk slots idle (idle slots cost issue slots, not bytes) -- with one
// exception: when the pass count does not divide the wave count, a wave's
// items change pass and reload x from LDS each time (8*d VGPRs per chunk,
// as many LDS bytes as the item's gathers), so a tiling whose pass count
// divides the waves -- the smallest such count the pass width allows -- is
// taken at up to 3/8 idle slots.
// For d >= 4 the kernel is bound by its gathers and dot products, not by HBM,
// and idle slots still gather and multiply: among the tilings whose pass
// count divides the waves it takes the most useful chunks per item (C times
// the pass width over L*C), then the fewest idle slots, then the fewest
// passes -- e.g. 64 chunks run on 32 lanes x 2 rather than 32 x 3 (a third
// of the slots idle), the same bytes per item.
struct LaneTiling {
  int lg, C, passes;
};

LaneTiling plan_tiling(int nq, int max_c, int waves, bool cu_bound) {
  LaneTiling best{2, 1, (nq + 3) / 4};
  int best_lc = 0;
  double best_useful = -1.0, best_idle = 2.0;
  for (int pass_rule = 0; pass_rule < 2 && best_lc == 0; ++pass_rule)
    for (int C = 1; C <= max_c; ++C)
      for (int lg = 2; lg <= 5; ++lg) {
        const int LC = C << lg;
        int passes = (nq + LC - 1) / LC;
        if (pass_rule == 0) {  // passes dividing the waves, up to 3/8 idle
          while (passes <= waves && waves % passes != 0) ++passes;
          if (passes > waves) continue;
        }
        const long slots = (long)passes * LC;
        if (pass_rule == 0) {
          if (8 * (slots - nq) > 3 * slots) continue;
        } else if (4 * (slots - nq) > slots) {
          continue;
        }
        if (pass_rule == 0 && cu_bound) {
          const int pw = (nq + passes - 1) / passes;
          const double useful = (double)C * pw / LC;     // useful chunks per lane per item
          const double idle = (double)(slots - nq) / slots;
          const bool better = useful > best_useful + 1e-9 ||
                              (useful > best_useful - 1e-9 &&
                               (idle < best_idle - 1e-9 ||
                                (idle < best_idle + 1e-9 &&
                                 (passes < best.passes || (passes == best.passes && lg > best.lg)))));
          if (best_lc == 0 || better) {
            best = LaneTiling{lg, C, passes};
            best_lc = LC;
            best_useful = useful;
            best_idle = idle;
          }
        } else if (LC > best_lc || (LC == best_lc && lg > best.lg)) {
          best = LaneTiling{lg, C, passes};
          best_lc = LC;
        }
      }
  if (best_lc == 0) {  // tiny rows: fewest slots
    long best_slots = -1;
    for (int C = 1; C <= max_c; ++C)
      for (int lg = 2; lg <= 5; ++lg) {
        const int LC = C << lg;
        const int passes = (nq + LC - 1) / LC;
        const long slots = (long)passes * LC;
        if (best_slots < 0 || slots < best_slots) {
          best = LaneTiling{lg, C, passes};
          best_slots = slots;
        }
      }
  }
  return best;
}

template <int D, int B, int G, int C, int XS, bool MOE>
hipError_t gemv_launch_c(const GemvArgs& a, dim3 grid, hipStream_t s) {
  const uint16_t* xs = MOE ? a.x : a.x + (int64_t)a.tok0 * a.cols;
  const int pw = (a.nq + a.passes - 1) / a.passes;
  if (a.nq > 0xfff || a.lanes_log2 > 7 || a.passes > 0xff || pw > 0x1ff || pw > C << a.lanes_log2)
    return hipErrorInvalidValue;
  const uint32_t shape = (uint32_t)a.nq | ((uint32_t)a.lanes_log2 << 12) | ((uint32_t)a.passes << 15) |
                         ((uint32_t)pw << 23);
  hipLaunchKernelGGL((vq_gemv_kernel<D, B, G, C, XS, MOE>), grid, dim3(kGemvThreads), 0, s, a.codes, a.codebook,
                     a.scales, xs, a.rows, a.rows_base, a.rows_extra, a.q0, a.spr, shape, a);
  return hipGetLastError();
}

template <int D, int B, int G, int XS, bool MOE>
hipError_t gemv_launch(const GemvArgs& a, int C, dim3 grid, hipStream_t s) {
  constexpr int MC = gemv_max_c(D);
  switch (C) {
    case 1: return gemv_launch_c<D, B, G, 1, XS, MOE>(a, grid, s);
    case 2: if constexpr (MC >= 2) return gemv_launch_c<D, B, G, 2, XS, MOE>(a, grid, s); break;
    case 3: if constexpr (MC >= 3) return gemv_launch_c<D, B, G, 3, XS, MOE>(a, grid, s); break;
    case 4: if constexpr (MC >= 4) return gemv_launch_c<D, B, G, 4, XS, MOE>(a, grid, s); break;
    case 5: if constexpr (MC >= 5) return gemv_launch_c<D, B, G, 5, XS, MOE>(a, grid, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// Column slices that fit the x slice in LDS run one after another, adding
// into y; rows are split over about one block per CU (per token slice), or
// more where a block's scales or row pieces would not fit in LDS.  Dense
// calls run one grid slice per token (blockIdx.y), routed calls one per
// (token, slot) pair.
template <int D, int B, int G, bool MOE>
hipError_t gemv_run(GemvArgs a, int P, int ycount, hipStream_t s) {
  const int slice_max = kGemvXMaxBytes / (32 * D);
  const int n_slices = (P + slice_max - 1) / slice_max;
  const int per_slice = (P + n_slices - 1) / n_slices;
  const int blocks_fill = std::max(1, num_cus() / std::max(1, ycount));
  for (int sl = 0; sl < n_slices; ++sl) {
    a.q0 = sl * per_slice;
    a.nq = std::min(per_slice, P - a.q0);
    a.accumulate = sl > 0;
    const LaneTiling t = plan_tiling(a.nq, gemv_max_c(D), kGemvWaves, D >= 4);
    a.lanes_log2 = t.lg;
    a.passes = t.passes;
    const int64_t by_scales = std::max<int64_t>(1, (kGemvScaleBytes - 16) / (2 * (int64_t)a.spr));
    const int64_t by_pieces = std::max<int64_t>(1, kGemvPieces / (int64_t)t.passes);
    const int64_t rows_max = std::min(by_scales, by_pieces);
    const int64_t blocks = std::min<int64_t>(a.rows, std::max<int64_t>(blocks_fill, (a.rows + rows_max - 1) / rows_max));
    a.rows_base = (int)(a.rows / blocks);
    a.rows_extra = (int)(a.rows - (int64_t)a.rows_base * blocks);
    const int XS = (int64_t)a.nq * 32 * D <= 2 * 8192 ? 2 : 5;
    // dense: at most 65535 token slices per launch
    for (int y0 = 0; y0 < ycount; y0 += 65535) {
      const int yc = std::min(65535, ycount - y0);
      if (!MOE) a.tok0 = y0;
      hipError_t e = XS == 2 ? gemv_launch<D, B, G, 2, MOE>(a, t.C, dim3((unsigned)blocks, (unsigned)yc), s)
                             : gemv_launch<D, B, G, 5, MOE>(a, t.C, dim3((unsigned)blocks, (unsigned)yc), s);
      if (e != hipSuccess) return e;
      if (MOE) break;
    }
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
  const int P = w.cols / (16 * D);
  a.top_k = top_k;
  a.num_experts = w.num_experts;
  a.x_per_slot = x_per_slot;
  if (ids) {
    a.T = T * top_k;
    return gemv_run<D, B, G, true>(a, P, T * top_k, s);
  }
  a.T = T;
  return gemv_run<D, B, G, false>(a, P, T, s);
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
