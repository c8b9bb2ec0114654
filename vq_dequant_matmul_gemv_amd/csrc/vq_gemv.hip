// vq_gemv.hip -- the decode-shaped kernels (GEMV, routed GEMV, dequant),
// dispatched by code width to the translation units that instantiate them
// (vq_gemv_bNN.hip; the kernels themselves are in vq_gemv_impl.h).
#include "vq_kernels.h"

namespace vqmi {

hipError_t launch_gemv(const TensorView& w, const IoSpec& io, const void* x, int T, void* y,
                       const int32_t* ids, int top_k, int x_per_slot, hipStream_t s) {
  if (io.epi == kEpiCombine) {  // the slots add into y: zero it first
    hipError_t e = launch_zero(y, (size_t)T * w.rows * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  switch (w.log2_k) {
#define X(B) \
  case B: return gemv_b##B(w, io, x, T, y, ids, top_k, x_per_slot, s);
    VQMI_BITS(X)
#undef X
    default: break;
  }
  return hipErrorInvalidValue;
}

int device_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

hipError_t launch_dequant(const TensorView& w, int expert, uint16_t* out, hipStream_t s) {
  switch (w.log2_k) {
#define X(B) \
  case B: return dequant_b##B(w, expert, out, s);
    VQMI_BITS(X)
#undef X
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace vqmi
