// Instances of the matrix-core kernel for head dims up to 128 (DC = 4).
#include "kernels_mfma.hpp"

namespace aa {

template <int KTC>
static int launch_one(const MfmaParams& mp, long grid, hipStream_t st) {
  agent_mfma_kernel<4, KTC>
      <<<dim3((unsigned)grid), dim3(kThreads), (unsigned)Cfg<4, KTC>::TOTAL, st>>>(mp);
  return (int)hipGetLastError();
}

template <>
int launch_mfma_dc<4>(const MfmaParams& mp, int ktc, long grid, hipStream_t st) {
  switch (ktc) {
    case 4: return launch_one<4>(mp, grid, st);
    case 8: return launch_one<8>(mp, grid, st);
    default: return launch_one<16>(mp, grid, st);
  }
}

}  // namespace aa
