// Portable float32-arithmetic kernels of the Agent Attention forward.
//
// These serve float32 I/O (where the matrix-core bf16 path would not hold a
// 1e-5 tolerance) and any shape the matrix-core kernels do not take.  One
// thread owns one agent row (aggregation) or one query row (broadcast) and
// runs an exact online softmax in the log2 domain: every logit is
// pre-multiplied by scale*log2(e) so that exp() becomes the hardware exp2.
//
// Sources: "Agent Attention: On the Integration of Softmax and Linear
// Attention" (paperlayer.ai summary), §4 Agent Transformer (aggregation and
// broadcast as two Softmax attentions; pooling as the default agent source);
// "Agent Attention：Transformer计算量太大？…" (jsqmd.com), §1 pseudocode.
#pragma once

#include "common.hpp"

namespace aa {

// ---------------------------------------------------------------- pooling
// A[bh, i*s+j, :] = mean of q over grid rows [floor(i h/s), ceil((i+1) h/s))
// and columns [floor(j w/s), ceil((j+1) w/s)).  One block (256 threads) per
// (bh, agent): 64 lanes over channels x 4 groups over window rows.
// Module terms of the scalar broadcast (each pointer may be null): agent
// bias B2 [H, N, nag], and the depth-wise convolution of V (same layout as
// Q) with weights [H*d, 3, 3], bias [H*d], over a grid of width w.
struct ScalarMod {
  const float* bias2;
  const void* v;
  const float* dwc_w;
  const float* dwc_b;
  int w;
};

template <typename T>
__global__ void __launch_bounds__(256)
pool_kernel(const T* __restrict__ q, float* __restrict__ A, int h, int w, int d, int s,
            Strides sq) {
  const int k = s * s;
  const int agent = blockIdx.x % k;
  const long bh = blockIdx.x / k;
  const int i = agent / s, j = agent % s;
  const int r0 = (i * h) / s, r1 = ((i + 1) * h + s - 1) / s;
  const int c0 = (j * w) / s, c1 = ((j + 1) * w + s - 1) / s;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const T* qh = q + head_offset(sq, bh);
  __shared__ float red[4][kMaxD];
  for (int c = tx; c < d; c += 64) {
    float acc = 0.f;
    for (int r = r0 + ty; r < r1; r += 4)
      for (int cc = c0; cc < c1; ++cc) acc += to_f32(qh[((long)r * w + cc) * sq.n + c]);
    red[ty][c] = acc;
  }
  __syncthreads();
  if (ty == 0) {
    const float inv = 1.0f / (float)((r1 - r0) * (c1 - c0));
    for (int c = tx; c < d; c += 64)
      A[(bh * k + agent) * d + c] = ((red[0][c] + red[1][c]) + (red[2][c] + red[3][c])) * inv;
  }
}

// Caller-supplied agents (dtype) -> float32 workspace copy.
template <typename T>
__global__ void __launch_bounds__(256)
widen_kernel(const T* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    dst[i] = to_f32(src[i]);
}

// ------------------------------------------------------------ aggregation
// Split-N partial aggregation.  Block = (bh, chunk of tokens); thread t owns
// agent t.  Writes part[bh][chunk][t] = {m, l, acc[0..d)} where, over the
// chunk's tokens n, m = max_n x_n, l = sum_n 2^(x_n - m),
// acc = sum_n 2^(x_n - m) V[n], x_n = scale*log2(e) * <A_t, K_n>.
template <typename T, int MAXD>
__global__ void __launch_bounds__(256)
aggregate_partial_scalar(const float* __restrict__ A, const T* __restrict__ K,
                         const T* __restrict__ V, float* __restrict__ part, int N, int d,
                         int nag, float sl2, int chunk, int nchunks, Strides sk,
                         const float* __restrict__ bias1) {
  constexpr int TS = MAXD > 64 ? 16 : 32;
  const int ch = blockIdx.x % nchunks;
  const long bh = blockIdx.x / nchunks;
  const int t = threadIdx.x;
  const bool active = t < nag;
  __shared__ float Ks[TS][MAXD];
  __shared__ float Vs[TS][MAXD];
  float a[MAXD], acc[MAXD];
#pragma unroll
  for (int c = 0; c < MAXD; ++c) {
    a[c] = (active && c < d) ? A[(bh * nag + t) * d + c] : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int n0 = ch * chunk, n1 = min(N, n0 + chunk);
  const T* Kh = K + head_offset(sk, bh);
  const T* Vh = V + head_offset(sk, bh);
  // agent bias B1[h][t][n] of the head's parameters (null: none)
  const float* b1 = bias1 ? bias1 + ((bh % sk.H) * nag + (active ? t : 0)) * (long)N : nullptr;
  for (int nb = n0; nb < n1; nb += TS) {
    const int cnt = min(TS, n1 - nb);
    __syncthreads();
    for (int idx = t; idx < cnt * d; idx += 256) {
      const int tok = idx / d, c = idx - tok * d;
      Ks[tok][c] = to_f32(Kh[(long)(nb + tok) * sk.n + c]);
      Vs[tok][c] = to_f32(Vh[(long)(nb + tok) * sk.n + c]);
    }
    __syncthreads();
    if (active) {
      float sc[TS];
      float mx = m;
#pragma unroll
      for (int tok = 0; tok < TS; ++tok) {
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < MAXD; ++c)
          if (c < d) dot = fmaf(a[c], Ks[tok][c], dot);
        sc[tok] = dot * sl2;
        if (b1 && tok < cnt) sc[tok] = fmaf(b1[nb + tok], kLog2e, sc[tok]);
        if (tok < cnt) mx = fmaxf(mx, sc[tok]);
      }
      const float corr = fast_exp2(m - mx);
      l *= corr;
#pragma unroll
      for (int c = 0; c < MAXD; ++c) acc[c] *= corr;
#pragma unroll
      for (int tok = 0; tok < TS; ++tok) {
        if (tok < cnt) {
          const float p = fast_exp2(sc[tok] - mx);
          l += p;
#pragma unroll
          for (int c = 0; c < MAXD; ++c)
            if (c < d) acc[c] = fmaf(p, Vs[tok][c], acc[c]);
        }
      }
      m = mx;
    }
  }
  if (active) {
    float* o = part + ((bh * nchunks + ch) * (long)nag + t) * (d + 2);
    o[0] = m;
    o[1] = l;
#pragma unroll
    for (int c = 0; c < MAXD; ++c)
      if (c < d) o[2 + c] = acc[c];
  }
}

// Merge of the split-N partials: V_A = sum_j 2^(m_j-M) acc_j / sum_j 2^(m_j-M) l_j
// with M = max_j m_j.  Block = (bh, agent), threads over channels.
__global__ void __launch_bounds__(128)
merge_partials_kernel(const float* __restrict__ part, float* __restrict__ VA, int d, int nag,
                      int nchunks) {
  const int agent = blockIdx.x % nag;
  const long bh = blockIdx.x / nag;
  const long stride = (long)nag * (d + 2);
  const float* p0 = part + ((bh * nchunks) * (long)nag + agent) * (d + 2);
  float M = -INFINITY;
  for (int j = 0; j < nchunks; ++j) M = fmaxf(M, p0[j * stride]);
  float L = 0.f;
  for (int j = 0; j < nchunks; ++j) L += p0[j * stride + 1] * fast_exp2(p0[j * stride] - M);
  const float inv = 1.0f / L;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < nchunks; ++j)
      acc = fmaf(p0[j * stride + 2 + c], fast_exp2(p0[j * stride] - M), acc);
    VA[(bh * nag + agent) * d + c] = acc * inv;
  }
}

// -------------------------------------------------------------- broadcast
// Block = (bh, 256 queries); thread owns one query row.  Agents and agent
// values stream through LDS in chunks of AC.
template <typename T, int MAXD>
__global__ void __launch_bounds__(256)
broadcast_scalar(const T* __restrict__ Q, const float* __restrict__ A,
                 const float* __restrict__ VA, T* __restrict__ O, int N, int d, int nag,
                 float sl2, int nqblk, Strides sq, ScalarMod md) {
  constexpr int AC = MAXD > 64 ? 16 : 32;
  const int qb = blockIdx.x % nqblk;
  const long bh = blockIdx.x / nqblk;
  const int n = qb * 256 + threadIdx.x;
  const bool active = n < N;
  __shared__ float As[AC][MAXD];
  __shared__ float Vs[AC][MAXD];
  const T* qrow = Q + head_offset(sq, bh) + (long)(active ? n : 0) * sq.n;
  float qv[MAXD], o[MAXD];
#pragma unroll
  for (int c = 0; c < MAXD; ++c) {
    qv[c] = (active && c < d) ? to_f32(qrow[c]) : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* Ah = A + bh * (long)nag * d;
  const float* Vh = VA + bh * (long)nag * d;
  const long hh = bh % sq.H;   // head of the batch entry: index of the module parameters
  const float* b2 = md.bias2 ? md.bias2 + (hh * N + (active ? n : 0)) * (long)nag : nullptr;
  for (int a0 = 0; a0 < nag; a0 += AC) {
    const int cnt = min(AC, nag - a0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < cnt * d; idx += 256) {
      const int ag = idx / d, c = idx - ag * d;
      As[ag][c] = Ah[(long)(a0 + ag) * d + c];
      Vs[ag][c] = Vh[(long)(a0 + ag) * d + c];
    }
    __syncthreads();
    float sc[AC];
    float mx = m;
#pragma unroll
    for (int ag = 0; ag < AC; ++ag) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < MAXD; ++c)
        if (c < d) dot = fmaf(qv[c], As[ag][c], dot);
      sc[ag] = dot * sl2;
      if (b2 && ag < cnt) sc[ag] = fmaf(b2[a0 + ag], kLog2e, sc[ag]);
      if (ag < cnt) mx = fmaxf(mx, sc[ag]);
    }
    const float corr = fast_exp2(m - mx);
    l *= corr;
#pragma unroll
    for (int c = 0; c < MAXD; ++c) o[c] *= corr;
#pragma unroll
    for (int ag = 0; ag < AC; ++ag) {
      if (ag < cnt) {
        const float p = fast_exp2(sc[ag] - mx);
        l += p;
#pragma unroll
        for (int c = 0; c < MAXD; ++c)
          if (c < d) o[c] = fmaf(p, Vs[ag][c], o[c]);
      }
    }
    m = mx;
  }
  if (active) {
    T* orow = O + head_offset(sq, bh) + (long)n * sq.n;
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < MAXD; ++c) o[c] *= inv;
    if (md.dwc_w) {
      // + DWC(V): 3 x 3 neighbourhood of token n on the grid, zero outside
      const T* Vsrc = static_cast<const T*>(md.v) + head_offset(sq, bh);
      const int row = n / md.w, col = n - row * md.w, rows = N / md.w;
#pragma unroll
      for (int c = 0; c < MAXD; ++c) {
        if (c >= d) continue;
        const long ch = hh * d + c;
        float acc = md.dwc_b ? md.dwc_b[ch] : 0.f;
        for (int tap = 0; tap < 9; ++tap) {
          const int rr = row + tap / 3 - 1, cc = col + tap % 3 - 1;
          if (rr >= 0 && rr < rows && cc >= 0 && cc < md.w)
            acc = fmaf(md.dwc_w[ch * 9 + tap], to_f32(Vsrc[(long)(rr * md.w + cc) * sq.n + c]),
                       acc);
        }
        o[c] += acc;
      }
    }
#pragma unroll
    for (int c = 0; c < MAXD; ++c)
      if (c < d) orow[c] = from_f32<T>(o[c]);
  }
}

}  // namespace aa
