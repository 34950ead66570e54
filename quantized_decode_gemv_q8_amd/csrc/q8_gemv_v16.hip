// Q8_0 matvec kernel instances with 16-column lane rows (m_tile 1..2).
#include "q8_gemv_kernel.h"

namespace q8 {

GemvKernel gemv_kernel_v16(int m_tile) { return pick_m_tile<16>(m_tile); }

}  // namespace q8
