// Instances of the matrix-core kernel for head dims up to 64 (DC = 2).
#include "kernels_mfma.hpp"

namespace aa {

template <int KTC, bool STRIDED>
static int launch_one(const MfmaParams& mp, long grid, hipStream_t st) {
  agent_mfma_kernel<2, KTC, STRIDED>
      <<<dim3((unsigned)grid), dim3(kThreads), (unsigned)Cfg<2, KTC>::TOTAL, st>>>(mp);
  return (int)hipGetLastError();
}

template <>
int launch_mfma_dc<2>(const MfmaParams& mp, int ktc, bool strided, long grid, hipStream_t st) {
  switch (ktc) {
    case 4: return strided ? launch_one<4, true>(mp, grid, st) : launch_one<4, false>(mp, grid, st);
    case 8: return strided ? launch_one<8, true>(mp, grid, st) : launch_one<8, false>(mp, grid, st);
    default:
      return strided ? launch_one<16, true>(mp, grid, st) : launch_one<16, false>(mp, grid, st);
  }
}

}  // namespace aa
