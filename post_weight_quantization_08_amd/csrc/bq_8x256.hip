// Block quantizer kernels of one workgroup shape (see block_quant.h).
#include "block_quant.h"

namespace gq {

void launch_bq_8x256(const QArgs& a, int g, int64_t batch, hipStream_t st) { launch_bq_g<8, 256>(a, g, batch, st); }
void launch_bq_static(const QArgs& a, int64_t batch, hipStream_t st) { launch_bq<8, 256, 0, false>(a, batch, st); }

}  // namespace gq
