// vq_gemv_b06.hip -- GEMV and dequant kernels for 6-bit codes (K = 64); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(6)
}  // namespace vqmi
