// vq_gemv_b07.hip -- GEMV and dequant kernels for 7-bit codes (K = 128); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(7)
}  // namespace vqmi
