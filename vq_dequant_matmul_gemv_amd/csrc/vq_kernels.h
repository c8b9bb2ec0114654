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

hipError_t launch_dequant(const TensorView& w, int expert, uint16_t* out, hipStream_t s);

// Dense (ids == nullptr, T tokens) or routed (ids != nullptr, T*top_k pairs).
hipError_t launch_gemv(const TensorView& w, const uint16_t* x, int T, float* y,
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s);

hipError_t launch_gemm(const TensorView& w, const uint16_t* x, int T, float* y, hipStream_t s);

size_t moe_workspace_bytes(int T, int top_k, int num_experts);

// Bytes of the library's static device scratch array (one per GPU), and its
// address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
hipError_t static_scratch(void** out);
hipError_t launch_moe_gemm(const TensorView& w, const uint16_t* x, int x_per_slot,
                           const int32_t* ids, int T, int top_k, float* y, void* ws,
                           hipStream_t s);

}  // namespace vqmi
