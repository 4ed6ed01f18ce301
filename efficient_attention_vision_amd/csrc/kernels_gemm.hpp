// Batched, tiled float32 matrix products and the softmax-gradient
// elementwise steps of the Agent Attention backward pass.
//
// The backward of the two Softmax attentions ("Agent Attention: On the
// Integration of Softmax and Linear Attention", §4) is a chain of products
// of N x k, k x d and N x d matrices per head, with the probabilities P1
// (k x N) and P2 (N x k) recomputed and kept in the workspace:
//   S2 = Q A^T, P2 = softmax(scale S2)       S1 = A K^T, P1 = softmax(scale S1)
//   V_A = P1 V (the forward's aggregation, recomputed)
//   dV_A = P2^T dO    dP2 = dO V_A^T   dS2 = P2 (dP2 - rowsum(P2 dP2))
//   dQ = scale dS2 A  dA = scale dS2^T Q + scale dS1 K
//   dP1 = dV_A V^T    dS1 = P1 (dP1 - rowsum(P1 dP1))
//   dK = scale dS1^T A   dV = P1^T dV_A
// All arithmetic is float32.
#pragma once

#include "common.hpp"
#include "kernels_backward.hpp"   // half_t

namespace aa {

// One operand of a batched product: element (b; r, c) at
// base + b*bs + r*rs + c*cs, of type T.
struct MatRef {
  const void* base;
  long bs, rs, cs;
};

// part[z][b][i][j] = alpha * sum over kk in split z of A(b; i, kk) B(b; kk, j),
// i < M, j < N; split z covers kk in [z*kchunk, min(K, (z+1)*kchunk)).
// Grid: x over 64-column tiles, y over 64-row tiles, z = batch*splits + z.
// 256 threads, each computing a 4 x 4 block of the 64 x 64 tile.
template <typename TA, typename TB>
__global__ void __launch_bounds__(256)
bgemm_f32(MatRef A, MatRef B, float* __restrict__ part, int M, int N, int K, int kchunk,
          int splits, long batch, float alpha) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const long bz = blockIdx.z / splits;
  const int z = blockIdx.z - (int)(bz * splits);
  const int i0 = blockIdx.y * BM, j0 = blockIdx.x * BN;
  const int k0 = z * kchunk, k1 = min(K, k0 + kchunk);
  const TA* a = static_cast<const TA*>(A.base) + bz * A.bs;
  const TB* b = static_cast<const TB*>(B.base) + bz * B.bs;
  const bool a_kfast = A.cs == 1, b_kfast = B.rs == 1;
  float acc[4][4] = {};
  for (int kb = k0; kb < k1; kb += BK) {
    __syncthreads();
    // consecutive threads take consecutive elements in memory (the unit
    // stride dimension of each operand), 1024 elements of each tile
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;       // 0 .. 1023
      const int ii = a_kfast ? idx >> 4 : idx & 63, ka = a_kfast ? idx & 15 : idx >> 6;
      const int gi = i0 + ii, gka = kb + ka;
      As[ka][ii] = (gi < M && gka < k1) ? to_f32(a[gi * A.rs + gka * A.cs]) : 0.f;
      const int jj = b_kfast ? idx >> 4 : idx & 63, kb2 = b_kfast ? idx & 15 : idx >> 6;
      const int gj = j0 + jj, gkb = kb + kb2;
      Bs[kb2][jj] = (gj < N && gkb < k1) ? to_f32(b[gkb * B.rs + gj * B.cs]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float4 av = *reinterpret_cast<const float4*>(&As[kk][4 * ty]);
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][4 * tx]);
      const float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(ar[r], br[c], acc[r][c]);
    }
  }
  float* out = part + ((long)z * batch + bz) * (long)M * N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gi = i0 + 4 * ty + r;
    if (gi >= M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int gj = j0 + 4 * tx + c;
      if (gj < N) out[(long)gi * N + gj] = alpha * acc[r][c];
    }
  }
}

// out[e] = (accumulate ? out[e] : 0) + factor * sum over z of part[z][e],
// e < n (n = batch * M * N).
__global__ void __launch_bounds__(256)
sum_splits(const float* __restrict__ part, float* __restrict__ out, long n, int splits,
           float factor, int accumulate) {
  for (long e = blockIdx.x * 256L + threadIdx.x; e < n; e += (long)gridDim.x * 256) {
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[(long)z * n + e];
    out[e] = (accumulate ? out[e] : 0.f) + factor * s;
  }
}

// In place, one block per row of length L: row = softmax(sl2 * row) in the
// log2 domain (the probabilities P2 from S2, and P1 from S1).
__global__ void __launch_bounds__(256)
row_softmax_log2(float* __restrict__ S, int L, float sl2) {
  float* row = S + (long)blockIdx.x * L;
  __shared__ float red[256];
  float m = -INFINITY;
  for (int i = threadIdx.x; i < L; i += 256) m = fmaxf(m, row[i] * sl2);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  m = red[0];
  __syncthreads();
  float l = 0.f;
  for (int i = threadIdx.x; i < L; i += 256) l += fast_exp2(row[i] * sl2 - m);
  red[threadIdx.x] = l;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  for (int i = threadIdx.x; i < L; i += 256) row[i] = fast_exp2(row[i] * sl2 - m) * inv;
}

// Wave-wide sum and max (64 lanes).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Short rows (L <= 256, the agents of a token): one wave per row, four rows
// per block.  softmax_short: row = softmax(sl2 * row) in place;
// softmax_grad_short: dP <- P * (dP - sum(P * dP)) in place.
__global__ void __launch_bounds__(256)
softmax_short(float* __restrict__ S, long rows, int L, float sl2) {
  const long r = blockIdx.x * 4L + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  float* row = S + r * L;
  float x[4];
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = lane + 64 * e;
    x[e] = i < L ? row[i] * sl2 : -INFINITY;
    m = fmaxf(m, x[e]);
  }
  m = wave_max(m);
  float l = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = lane + 64 * e < L ? fast_exp2(x[e] - m) : 0.f;
    l += x[e];
  }
  const float inv = 1.0f / wave_sum(l);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (lane + 64 * e < L) row[lane + 64 * e] = x[e] * inv;
}

__global__ void __launch_bounds__(256)
softmax_grad_short(const float* __restrict__ P, float* __restrict__ dP, long rows, int L) {
  const long r = blockIdx.x * 4L + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* p = P + r * L;
  float* g = dP + r * L;
  float pv[4], gv[4], s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = lane + 64 * e;
    pv[e] = i < L ? p[i] : 0.f;
    gv[e] = i < L ? g[i] : 0.f;
    s = fmaf(pv[e], gv[e], s);
  }
  const float D = wave_sum(s);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (lane + 64 * e < L) g[lane + 64 * e] = pv[e] * (gv[e] - D);
}

// In place, one block per row of length L: dP <- P * (dP - sum(P * dP)), the
// gradient of a row softmax with respect to its (scaled) logits.
__global__ void __launch_bounds__(256)
softmax_grad_rows(const float* __restrict__ P, float* __restrict__ dP, int L) {
  const float* p = P + (long)blockIdx.x * L;
  float* g = dP + (long)blockIdx.x * L;
  __shared__ float red[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < L; i += 256) s = fmaf(p[i], g[i], s);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float D = red[0];
  for (int i = threadIdx.x; i < L; i += 256) g[i] = p[i] * (g[i] - D);
}

// dQ (of type T) at token n of head bh = dQacc + the pooled agents'
// gradient dA spread over their windows (dA null: supplied agents).
// Thread per (token, channel).
template <typename T>
__global__ void __launch_bounds__(256)
finish_dq(const float* __restrict__ dQacc, const float* __restrict__ dA, T* __restrict__ dQ,
          long BH, int N, int d, int nag, int h, int w, int s) {
  const long n_el = BH * N * d;
  for (long e = blockIdx.x * 256L + threadIdx.x; e < n_el; e += (long)gridDim.x * 256) {
    float g = dQacc[e];
    if (dA) {
      const long bh = e / ((long)N * d);
      const int rem = (int)(e - bh * N * d), n = rem / d, c = rem - n * d;
      const int r = n / w, cc = n - r * w;
      const int i0 = max(0, (r * s) / h - 1), i1 = min(s - 1, (r * s) / h + 1);
      const int j0 = max(0, (cc * s) / w - 1), j1 = min(s - 1, (cc * s) / w + 1);
      for (int i = i0; i <= i1; ++i) {
        const int rs = (i * h) / s, re = ((i + 1) * h + s - 1) / s;
        if (r < rs || r >= re) continue;
        for (int j = j0; j <= j1; ++j) {
          const int cs = (j * w) / s, ce = ((j + 1) * w + s - 1) / s;
          if (cc < cs || cc >= ce) continue;
          g += dA[(bh * nag + i * s + j) * (long)d + c] / (float)((re - rs) * (ce - cs));
        }
      }
    }
    dQ[e] = from_f32<T>(g);
  }
}

// out (type T) = src (float32), n elements.
template <typename T>
__global__ void __launch_bounds__(256)
store_as(const float* __restrict__ src, T* __restrict__ out, long n) {
  for (long e = blockIdx.x * 256L + threadIdx.x; e < n; e += (long)gridDim.x * 256)
    out[e] = from_f32<T>(src[e]);
}

}  // namespace aa
