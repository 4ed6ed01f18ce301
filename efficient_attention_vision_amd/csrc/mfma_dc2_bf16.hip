// Instances of the matrix-core kernel for head dims up to 64 (DC = 2),
// bfloat16 tensors.
#include "kernels_mfma.hpp"

namespace aa {

template <>
int launch_mfma_dc<2, ElemBF16>(const MfmaParams& mp, int ktc, int variant, long grid,
                              hipStream_t st) {
  return launch_mfma_switch<2, ElemBF16>(mp, ktc, variant, grid, st);
}

}  // namespace aa
