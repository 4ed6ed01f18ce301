// Instances of the matrix-core backward for float16 tensors.
#include "kernels_bwd_mfma.hpp"

namespace aa {
namespace bw {

template <>
int run_backward_mfma<ElemF16>(const BwdParams& p, int KT, int DT, const Pass (&pp)[3],
                          hipStream_t st) {
  return run_backward_mfma_impl<ElemF16>(p, KT, DT, pp, st);
}

}  // namespace bw
}  // namespace aa
