// vq_gemv_b04.hip -- GEMV and dequant kernels for 4-bit codes (K = 16); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(4)
}  // namespace vqmi
