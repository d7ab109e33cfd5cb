// MXFP4 W4A4 GEMM on the gfx950 scaled matrix instruction (placeholder until
// the operand layout is established).
#include "q4_internal.h"

namespace q4 {

hipError_t launch_mx_gemm(const GemmArgs& g, int64_t max_mtiles, hipStream_t stream) {
  (void)g;
  (void)max_mtiles;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace q4
