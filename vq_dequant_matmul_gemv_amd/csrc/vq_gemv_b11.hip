// vq_gemv_b11.hip -- GEMV and dequant kernels for 11-bit codes (K = 2048); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(11)
}  // namespace vqmi
