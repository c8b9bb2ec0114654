// vq_kernels.h -- host-side launch interface of the HIP kernels (internal to
// libvqmi.so; the public C ABI is include/vq.h).  Every launcher enqueues on
// the given stream and returns the launch status; arguments are already
// validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqmi {

struct TensorView {
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  int rows, cols, d, log2_k, group, num_experts, cb_per_expert;
  int wr;  // words per row
};

// Input/output types and the fused output step of a call.
enum OutKind { kOutF32 = 0, kOutF16 = 1, kOutBF16 = 2 };
enum Epilogue { kEpiNone = 0, kEpiSwiglu = 1, kEpiCombine = 2 };
struct IoSpec {
  int x_bf16 = 0;               // x holds bf16 bit patterns (else fp16)
  int y_kind = kOutF32;         // OutKind of y
  int epi = kEpiNone;           // Epilogue
  const float* route_w = nullptr;  // kEpiCombine: [pairs] router weights
};

// Code widths the kernels are built for: B = log2 K = 4 ... 14 (K = 16 ...
// 16384), each in its own translation units (vq_gemv_bNN.hip, vq_gemm_bNN.hip).
#define VQMI_BITS(X) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14)
constexpr int kMinBits = 4;
constexpr int kMaxBits = 14;

#define VQMI_DECLARE_WIDTH(B)                                                                                \
  hipError_t gemv_b##B(const TensorView& w, const IoSpec& io, const void* x, int T, void* y,                \
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s);                        \
  hipError_t dequant_b##B(const TensorView& w, int expert, uint16_t* out, hipStream_t s);                   \
  hipError_t gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s); \
  hipError_t moe_gemm_b##B(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot,           \
                           const int32_t* ids, int T, int top_k, void* y, int32_t* ws, hipStream_t s);
VQMI_BITS(VQMI_DECLARE_WIDTH)
#undef VQMI_DECLARE_WIDTH

hipError_t launch_dequant(const TensorView& w, int expert, uint16_t* out, hipStream_t s);

// Dense (ids == nullptr, T tokens) or routed (ids != nullptr, T*top_k pairs).
hipError_t launch_gemv(const TensorView& w, const IoSpec& io, const void* x, int T, void* y,
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s);

hipError_t launch_gemm(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s);

// The matrix-core GEMV (vq_gemv_impl.h, MF) takes dense calls of two or more
// tokens whose rows give every CU at least one 16-row group: up to four
// tokens on rows that fit one block's passes (d = 2: 5120 columns, d = 4:
// 6144, d = 8: 4096), and, for a plain fp32 output (fp32 y, no fused output
// step), longer rows in column slices added into y and up to 16 tokens in its
// 16-token mode.  That mode's column slices are one pass wide (d = 2: 640
// columns, d = 4: 768, d = 8: 512) and every slice adds each output once
// more, atomically; the tokens it takes are capped at 160 / slices (measured:
// 5120x17408, 23 slices at d = 4: 16.3 against 18.2 us for the GEMM at T = 5,
// 26.6 against 22.3 at T = 16; 17408x5120, 7 slices: 20.9 against 22.1 at T =
// 16).
__host__ __device__ inline int gemv_mf_max_cols(int d) { return d == 2 ? 5120 : (d == 4 ? 6144 : 4096); }
__host__ __device__ constexpr int gemv_mf_slice_cols(int d) { return d == 2 ? 640 : (d == 4 ? 768 : 512); }
inline int gemv_mf_max_tokens(int rows, int cols, int d, int cus, bool plain_out) {
  if (rows < 16 * cus) return 0;
  if (!plain_out) return cols <= gemv_mf_max_cols(d) ? 4 : 0;
  const int n_sl = (cols + gemv_mf_slice_cols(d) - 1) / gemv_mf_slice_cols(d);
  const int wide = 160 / n_sl;
  return wide > 16 ? 16 : (wide < 4 ? 4 : wide);
}
inline bool gemv_mf_takes(int rows, int cols, int d, int T, int cus, bool plain_out) {
  return T >= 2 && T <= gemv_mf_max_tokens(rows, cols, d, cus, plain_out);
}
// Compute units of the current device (cached on first use).
int device_cus();

// Zero `bytes` (a multiple of 4) at p, on the stream, with a kernel (so it can
// sit in a captured graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

size_t moe_workspace_bytes(int T, int top_k, int num_experts);

// Routed GEMM: (token, slot) pairs go in tiles of this many per expert; with
// wide tiles on, also in tiles of kMoeWideTokens: one per whole 128 pairs of
// an expert and one for a remainder above kMoeWideMin (a smaller remainder
// takes 32-pair tiles).
constexpr int kMoeTileTokens = 32;
constexpr int kMoeWideTokens = 128;
constexpr int kMoeWideMin = 64;

// Routing workspace (int32): counts[E] | offsets[E] | fill[E] | tile_base[E] |
// n_tiles | n_wide | pad to 4 | pairs[npairs] | tiles[max_tiles][3] (expert,
// first pair, count; the n_wide wide tiles first).  At most ceil(npairs /
// 32) + E tiles (an expert's wide tiles never outnumber its 32-pair tiles).
__host__ __device__ inline int moe_max_tiles(int npairs, int E) {
  return (npairs + kMoeTileTokens - 1) / kMoeTileTokens + E;
}
__host__ __device__ inline int32_t* moe_ws_n_tiles(int32_t* ws, int E) { return ws + 4 * E; }
__host__ __device__ inline int32_t* moe_ws_n_wide(int32_t* ws, int E) { return ws + 4 * E + 1; }
__host__ __device__ inline int32_t* moe_ws_pairs(int32_t* ws, int E) { return ws + ((4 * E + 1 + 3) & ~3); }
__host__ __device__ inline int32_t* moe_ws_tiles(int32_t* ws, int E, int npairs) {
  return moe_ws_pairs(ws, E) + ((npairs + 3) & ~3);
}

// Bytes of the library's static device scratch array (one per GPU), and its
// address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
hipError_t static_scratch(void** out);
// The routing pass (vq_gemm.hip): group the pairs of `ids` by expert into
// the workspace and write the tile list (wide: 128-pair tiles for hot
// experts); skipped slots' output rows (y_row_halves 16-bit words each) are
// zeroed unless y_skip is null.
hipError_t launch_route(const int32_t* ids, int npairs, int num_experts, int32_t* ws, void* y_skip, int y_row_halves,
                        bool wide, hipStream_t s);
hipError_t launch_moe_gemm(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot,
                           const int32_t* ids, int T, int top_k, void* y, void* ws, hipStream_t s);

// The fit of one tensor (vq_encode.hip).
size_t encode_workspace_bytes(int rows, int cols, int d, int log2_k, int n_sample);
hipError_t launch_encode(const float* w, int rows, int cols, int d, int log2_k, int group, const int32_t* sample_idx,
                         int n_sample, const double* uniforms, int iters, uint32_t* codes, uint16_t* codebook,
                         uint16_t* scales, double* relerr, void* workspace, hipStream_t s);

}  // namespace vqmi
