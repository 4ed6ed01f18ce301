// Instances of the module's projection kernels (float32, bfloat16, float16).
#include "agent_attn.h"
#include "kernels_proj.hpp"

namespace aa {
namespace pj {

namespace {
template <class T, class El>
int launch_t(const ProjParams& p, int mode, hipStream_t st) {
  const dim3 grid((unsigned)((p.M + kTok - 1) / kTok), (unsigned)((p.Nout + kFeat - 1) / kFeat));
  if (mode == 0) proj_kernel<T, El, 0><<<grid, dim3(kThr), 0, st>>>(p);
  else proj_kernel<T, El, 1><<<grid, dim3(kThr), 0, st>>>(p);
  return (int)hipGetLastError();
}
}  // namespace

int launch_proj(const ProjParams& p, int mode, int dtype, hipStream_t st) {
  switch (dtype) {
    case AGENT_ATTN_F32: return launch_t<float, ElemBF16>(p, mode, st);
    case AGENT_ATTN_F16: return launch_t<uint16_t, ElemF16>(p, mode, st);
    default: return launch_t<uint16_t, ElemBF16>(p, mode, st);
  }
}

int launch_heads_concat(const void* o, void* y, int M, int N, int H, int d, int dtype,
                        hipStream_t st) {
  const int items = M * (H * d / 8);
  const dim3 grid((unsigned)((items + 255) / 256));
  if (dtype == AGENT_ATTN_F32)
    heads_concat<float><<<grid, dim3(256), 0, st>>>((const float*)o, (float*)y, M, N, H, d);
  else
    heads_concat<uint16_t><<<grid, dim3(256), 0, st>>>((const uint16_t*)o, (uint16_t*)y, M, N,
                                                       H, d);
  return (int)hipGetLastError();
}

}  // namespace pj
}  // namespace aa
