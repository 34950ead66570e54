// Q8_0 matvec kernel instances with 1-column lane rows (m_tile 1..8).
#include "q8_gemv_kernel.h"

namespace q8 {

GemvKernel gemv_kernel_v1(int m_tile) { return pick_m_tile<1>(m_tile); }

}  // namespace q8
