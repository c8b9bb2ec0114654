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

hipError_t launch_dequant(const TensorView& w, int expert, uint16_t* out, hipStream_t s);

// Dense (ids == nullptr, T tokens) or routed (ids != nullptr, T*top_k pairs).
hipError_t launch_gemv(const TensorView& w, const IoSpec& io, const void* x, int T, void* y,
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s);

hipError_t launch_gemm(const TensorView& w, const IoSpec& io, const void* x, int T, void* y, hipStream_t s);

// Zero `bytes` (a multiple of 4) at p, on the stream, with a kernel (so it can
// sit in a captured graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

size_t moe_workspace_bytes(int T, int top_k, int num_experts);

// Bytes of the library's static device scratch array (one per GPU), and its
// address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
hipError_t static_scratch(void** out);
hipError_t launch_moe_gemm(const TensorView& w, const IoSpec& io, const void* x, int x_per_slot,
                           const int32_t* ids, int T, int top_k, void* y, void* ws, hipStream_t s);

}  // namespace vqmi
