// Large-batch forward ("gemm" path): placeholder until the fp16 MFMA kernels land.
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

GemmPlan gemm_plan(int m, int n, int r, int B) {
  GemmPlan p{};
  (void)m; (void)n; (void)r; (void)B;
  p.bytes = 0;
  return p;
}

hipError_t gemm_forward(const FwdArgs& a, const GemmPlan& p) {
  (void)a; (void)p;
  return hipErrorNotSupported;
}

}  // namespace nq
