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

template <class El, int FT>
int launch_16(const ProjParams& p, int mode, hipStream_t st) {
  const dim3 grid((unsigned)((p.Nout + 32 * FT - 1) / (32 * FT)), (unsigned)((p.M + 127) / 128));
  const unsigned lds = (unsigned)gemm16_lds_bytes<FT>(p.C > kKStep ? 2 : 1);
  if (mode == 0) proj_gemm16<El, 0, FT><<<grid, dim3(kThr), lds, st>>>(p);
  else proj_gemm16<El, 1, FT><<<grid, dim3(kThr), lds, st>>>(p);
  return (int)hipGetLastError();
}

// Feature tile: 128 outputs per workgroup from 256 outputs, else 64 (more
// workgroups in flight for the short products; measured faster than one
// 192-wide tile at 192 outputs).
template <class El>
int launch_16(const ProjParams& p, int mode, hipStream_t st) {
  return p.Nout >= 256 ? launch_16<El, 4>(p, mode, st) : launch_16<El, 2>(p, mode, st);
}
}  // namespace

int launch_proj(const ProjParams& p, int mode, int dtype, hipStream_t st) {
  switch (dtype) {
    case AGENT_ATTN_F32: return launch_t<float, ElemBF16>(p, mode, st);
    case AGENT_ATTN_F16: return launch_16<ElemF16>(p, mode, st);
    default: return launch_16<ElemBF16>(p, mode, st);
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
