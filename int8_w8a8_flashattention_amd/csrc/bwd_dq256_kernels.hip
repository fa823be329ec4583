// bwd_dq256_kernels.hip - the backward's dQ kernel at D = 256 (bwd_dq.h), compiled
// with the matrix products' results in accumulation registers: at this head dim the
// Q and dO operands and the dQ accumulators alone fill the vector registers.
#include "bwd_dq.h"

namespace i8a {

using namespace bwd;

hipError_t launch_bwd_dq256(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream) {
  return a.causal ? dq_d<256, true>(a, p, ws, stream) : dq_d<256, false>(a, p, ws, stream);
}

}  // namespace i8a
