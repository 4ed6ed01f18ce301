// Batched matrix products of the backward pass on matrix cores, for the
// path that materialises the probability matrices (more than 64 agents).
//
// Same contract as bgemm_f32 (kernels_gemm.hpp): part[z][b][i][j] = alpha *
// sum over kk in split z of A(b; i, kk) B(b; kk, j), operands of any strides
// and of type float, bfloat16 or float16.  The products run as
// v_mfma_f32_16x16x32_bf16: a bfloat16 operand enters as it is, a float32 or
// float16 operand as a pair hi + lo of bfloat16 values (hi = x rounded, lo =
// x - hi rounded), and a product of pairs as hi*hi + hi*lo + lo*hi, which
// leaves about 2^-16 of each term (float16 values are exact as a pair).
// Accumulation is float32.
//
// Tile 64 (i) x 64 (j) per workgroup, contraction in steps of 32 through LDS
// rows of 32 + 8 elements (bank spread); the four waves form a 2 x 2 grid of
// 32 x 32 (four 16 x 16 MFMA tiles each).  MFMA rows are the output rows i,
// columns the output columns j, so a store instruction writes 16 consecutive
// columns of four rows.  Global loads run along each operand's unit-stride
// dimension; the next step's elements are loaded into registers while the
// current step's MFMAs run.
#pragma once

#include <type_traits>

#include "kernels_gemm.hpp"
#include "kernels_mfma.hpp"

namespace aa {

template <typename T>
struct GemmOperand {
  static constexpr bool kLo = !std::is_same<T, bf16_t>::value;   // needs a lo part
};

template <typename TA, typename TB>
__global__ void __launch_bounds__(256)
bgemm_mfma(MatRef A, MatRef B, float* __restrict__ part, int M, int N, int K, int kchunk,
           int splits, long batch, float alpha) {
  constexpr int BM = 64, BN = 64, BK = 32, RS = BK + 8;
  constexpr bool ALO = GemmOperand<TA>::kLo, BLO = GemmOperand<TB>::kLo;
  __shared__ __attribute__((aligned(16))) uint16_t sAh[BM * RS];
  __shared__ __attribute__((aligned(16))) uint16_t sAl[ALO ? BM * RS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sBh[BN * RS];
  __shared__ __attribute__((aligned(16))) uint16_t sBl[BLO ? BN * RS : 8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int wi = wave & 1, wj = wave >> 1;
  const long bz = blockIdx.z / splits;
  const int z = blockIdx.z - (int)(bz * splits);
  const int i0 = blockIdx.y * BM, j0 = blockIdx.x * BN;
  const int k0 = z * kchunk, k1 = min(K, k0 + kchunk);
  const TA* a = static_cast<const TA*>(A.base) + bz * A.bs;
  const TB* b = static_cast<const TB*>(B.base) + bz * B.bs;
  const bool a_kfast = A.cs == 1, b_kfast = B.rs == 1;
  // element e of this thread: A tile row ai[e], column ak[e]; B tile row bj[e]
  // (output column), column bk[e]; consecutive threads run along the unit
  // stride of each operand
  int ai[8], ak[8], bj[8], bk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int idx = tid + 256 * e;   // 0 .. 2047
    ai[e] = a_kfast ? idx >> 5 : idx & 63;
    ak[e] = a_kfast ? idx & 31 : idx >> 6;
    bj[e] = b_kfast ? idx >> 5 : idx & 63;
    bk[e] = b_kfast ? idx & 31 : idx >> 6;
  }
  float xa[8], xb[8];
  auto gload = [&](int kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int gi = i0 + ai[e], gk = kb + ak[e];
      xa[e] = (gi < M && gk < k1) ? to_f32(a[gi * A.rs + gk * A.cs]) : 0.f;
      const int gj = j0 + bj[e], gk2 = kb + bk[e];
      xb[e] = (gj < N && gk2 < k1) ? to_f32(b[gk2 * B.rs + gj * B.cs]) : 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t ha = ElemBF16::bits(xa[e]);
      sAh[ai[e] * RS + ak[e]] = ha;
      if (ALO) sAl[ai[e] * RS + ak[e]] = ElemBF16::bits(xa[e] - ElemBF16::value(ha));
      const uint16_t hb = ElemBF16::bits(xb[e]);
      sBh[bj[e] * RS + bk[e]] = hb;
      if (BLO) sBl[bj[e] * RS + bk[e]] = ElemBF16::bits(xb[e] - ElemBF16::value(hb));
    }
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (k0 < k1) gload(k0);
  for (int kb = k0; kb < k1; kb += BK) {
    lstore();
    __syncthreads();
    if (kb + BK < k1) gload(kb + BK);   // travels during the MFMAs
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ra = (wi * 32 + 16 * t + r) * RS + 8 * g, rb = (wj * 32 + 16 * t + r) * RS + 8 * g;
      ah[t] = *reinterpret_cast<const bf16x8*>(sAh + ra);
      bh[t] = *reinterpret_cast<const bf16x8*>(sBh + rb);
      if (ALO) al[t] = *reinterpret_cast<const bf16x8*>(sAl + ra);
      if (BLO) bl[t] = *reinterpret_cast<const bf16x8*>(sBl + rb);
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj) {
        acc[ti][tj] = ElemBF16::mma(ah[ti], bh[tj], acc[ti][tj]);
        if (BLO) acc[ti][tj] = ElemBF16::mma(ah[ti], bl[tj], acc[ti][tj]);
        if (ALO) acc[ti][tj] = ElemBF16::mma(al[ti], bh[tj], acc[ti][tj]);
      }
    __syncthreads();
  }
  float* out = part + ((long)z * batch + bz) * (long)M * N;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
      const int gj = j0 + wj * 32 + 16 * tj + r;
      if (gj >= N) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int gi = i0 + wi * 32 + 16 * ti + 4 * g + t;
        if (gi < M) out[(long)gi * N + gj] = alpha * acc[ti][tj][t];
      }
    }
}

}  // namespace aa
