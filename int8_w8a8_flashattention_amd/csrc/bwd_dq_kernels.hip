// bwd_dq_kernels.hip - the backward's dQ kernel (launch 2 of attn_bwd; the other
// launches are in bwd_kernels.hip).  This file is compiled with the matrix products'
// results in ordinary vector registers (-amdgpu-mfma-vgpr-form): the kernel's softmax
// arithmetic reads every product result, and the accumulation registers would otherwise
// be copied out of them on every block.
#include "bwd_dq.h"

namespace i8a {

using namespace bwd;

hipError_t launch_bwd_dq(const BwdArgs& a, const BwdPlan& p, char* ws, hipStream_t stream) {
#define I8A_BWD_DQ(DD) \
  case DD:             \
    return a.causal ? dq_d<DD, true>(a, p, ws, stream) : dq_d<DD, false>(a, p, ws, stream);
  switch (a.D) {
    I8A_BWD_DQ(32) I8A_BWD_DQ(64) I8A_BWD_DQ(128)
    case 256:
      return launch_bwd_dq256(a, p, ws, stream);
    default:
      return hipErrorInvalidValue;
  }
#undef I8A_BWD_DQ
}

}  // namespace i8a
