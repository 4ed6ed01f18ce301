// Shared device helpers of the Agent Attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "agent_attn.h"

namespace aa {

typedef uint16_t bf16_t;  // bfloat16 storage

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxD = AGENT_ATTN_MAX_HEAD_DIM;
constexpr int kMaxAgents = AGENT_ATTN_MAX_AGENTS;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of the XCD (accelerator complex die) the calling wave runs on: the
// XCC_ID hardware register (id 20), bits [3:0].
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11));
}

// Element strides of q, k, v and out: batch b, head h and token n of the
// [B, H, N, d] view (channels contiguous).  Head index bh = b*H + h.
struct Strides {
  long b, h, n;
  int H;
};
__host__ __device__ __forceinline__ long head_offset(const Strides& st, long bh) {
  return (bh / st.H) * st.b + (bh % st.H) * st.h;
}

// Bits of the fault word that the fused kernel leaves in its workspace.
constexpr unsigned kFaultBarrier = 1u;   // a group barrier gave up waiting
constexpr unsigned kFaultXcd = 2u;       // a workgroup ran off its planned XCD

}  // namespace aa
