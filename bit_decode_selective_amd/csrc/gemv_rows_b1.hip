// Row-tile GEMV kernels (split and fused, batch 1-2 per launch) for 1-bit resident
// codes; see gemv_rows.h and gemv.hip.
#include "gemv_rows.h"

namespace sfg {
sf_status gemv_rows_b1(GemvArgs& a, int R, int nb, int kind, hipStream_t s) {
  return dispatch_r<CodecPow2<1>, 1>(a, R, nb, kind, s);
}
}  // namespace sfg
