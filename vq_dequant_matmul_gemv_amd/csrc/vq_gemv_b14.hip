// vq_gemv_b14.hip -- GEMV and dequant kernels for 14-bit codes (K = 16384); see vq_gemv_impl.h.
#include "vq_gemv_impl.h"

namespace vqmi {
VQMI_GEMV_UNIT(14)
}  // namespace vqmi
