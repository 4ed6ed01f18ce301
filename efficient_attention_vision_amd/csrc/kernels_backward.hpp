// Float32-arithmetic kernels of the Agent Attention backward pass.
//
// Gradients of O = softmax(scale Q A^T) softmax(scale A K^T) V through the
// two Softmax attentions and the pooling ("Agent Attention: On the
// Integration of Softmax and Linear Attention", §4 Agent Transformer: the
// operator is two Softmax attentions; §6: A = f(Q)).  With P1 = softmax(S1),
// S1 = scale A K^T (agents x tokens), V_A = P1 V, P2 = softmax(S2),
// S2 = scale Q A^T (tokens x agents), O = P2 V_A and the output gradient dO:
//   dV_A = P2^T dO,   dS2 = P2 * (dO V_A^T - D2),  D2[n] = dO[n] . O[n]
//   dQ   = scale dS2 A,   dA = scale dS2^T Q + scale dS1 K
//   dV   = P1^T dV_A,  dS1 = P1 * (dV_A V^T - D1), D1[a] = dV_A[a] . V_A[a]
//   dK   = scale dS1^T A
// and, for pooled agents, dQ += the agents' gradient spread evenly over
// their windows.  (D2 and D1 are the row sums of P * dP of each softmax.)
// Probabilities are recomputed from the saved log-sum-exps (log2 domain):
// p = 2^(scale log2(e) <a, x> - lse).  One thread owns one agent row (agent
// passes, split over token chunks) or one token row (token passes).
#pragma once

#include "common.hpp"

namespace aa {

// float16 storage for the float32 kernels (bfloat16 has its own bf16_t)
struct half_t {
  uint16_t bits;
};
__device__ __forceinline__ float to_f32(half_t x) {
  return static_cast<float>(__builtin_bit_cast(_Float16, x.bits));
}
template <>
__device__ __forceinline__ half_t from_f32<half_t>(float x) {
  return half_t{__builtin_bit_cast(uint16_t, static_cast<_Float16>(x))};
}

// Per token n of head bh: lse2[n] = log2 sum_a 2^(x_a) with x_a = scale
// log2(e) <q_n, A_a>, and D2[n] = dO[n] . O[n], O recomputed in float32.
template <typename T, int MAXD>
__global__ void __launch_bounds__(256)
bwd_token_stats(const T* __restrict__ Q, const T* __restrict__ dO, const float* __restrict__ A,
                const float* __restrict__ VA, float* __restrict__ lse2, float* __restrict__ D2,
                int N, int d, int nag, float sl2, int nqblk, Strides sq) {
  constexpr int AC = MAXD > 64 ? 16 : 32;
  const int qb = blockIdx.x % nqblk;
  const long bh = blockIdx.x / nqblk;
  const int n = qb * 256 + threadIdx.x;
  const bool active = n < N;
  __shared__ float As[AC][MAXD];
  __shared__ float Vs[AC][MAXD];
  const long ro = head_offset(sq, bh) + (long)(active ? n : 0) * sq.n;
  float qv[MAXD], o[MAXD];
#pragma unroll
  for (int c = 0; c < MAXD; ++c) {
    qv[c] = (active && c < d) ? to_f32(Q[ro + c]) : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* Ah = A + bh * (long)nag * d;
  const float* Vh = VA + bh * (long)nag * d;
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
    const float inv = 1.0f / l;
    float dd = 0.f;
#pragma unroll
    for (int c = 0; c < MAXD; ++c)
      if (c < d) dd = fmaf(to_f32(dO[ro + c]), o[c] * inv, dd);
    lse2[bh * N + n] = m + __log2f(l);
    D2[bh * N + n] = dd;
  }
}

// Agent pass, one thread per agent a, block = (bh, chunk of tokens), rows
// X (keys of the softmax) and Y staged through LDS:
//   p  = 2^(sl2 <A_a, X_n> - L),   ds = p (<W_a, Y_n> - D)
//   acc2[a] += ds X_n,   acc1[a] += p Y_n (BCAST only)
// BCAST (broadcast softmax, over agents per token): X = Q, Y = dO, W = V_A,
//   L = lse2[n], D = D2[n]; acc1 -> dV_A, acc2 -> dA / scale.
// otherwise (aggregation softmax, over tokens per agent): X = K, Y = V,
//   W = dV_A, L = lse1[a], D = D1[a] = <dV_A[a], V_A[a]>; acc2 -> dA / scale.
// Writes per-chunk partials part[bh][chunk][a][d] (acc1 to part1).
template <typename T, int MAXD, bool BCAST>
__global__ void __launch_bounds__(256)
bwd_agent_pass(const T* __restrict__ X, const T* __restrict__ Y, const float* __restrict__ A,
               const float* __restrict__ W, const float* __restrict__ VA,
               const float* __restrict__ lse_tok, const float* __restrict__ D_tok,
               const float* __restrict__ lse_ag, float* __restrict__ D_ag,
               float* __restrict__ part1, float* __restrict__ part2, int N, int d, int nag,
               float sl2, int chunk, int nchunks, Strides sx) {
  constexpr int TS = MAXD > 64 ? 16 : 32;
  const int ch = blockIdx.x % nchunks;
  const long bh = blockIdx.x / nchunks;
  const int t = threadIdx.x;
  const bool active = t < nag;
  __shared__ float Xs[TS][MAXD];
  __shared__ float Ys[TS][MAXD];
  __shared__ float Ls[TS], Ds[TS];
  const long arow = (bh * nag + (active ? t : 0)) * (long)d;
  float a[MAXD], wv[MAXD], acc1[MAXD], acc2[MAXD];
  float Dag = 0.f;
#pragma unroll
  for (int c = 0; c < MAXD; ++c) {
    a[c] = (active && c < d) ? A[arow + c] : 0.f;
    wv[c] = (active && c < d) ? W[arow + c] : 0.f;
    if (!BCAST && active && c < d) Dag = fmaf(wv[c], VA[arow + c], Dag);
    acc1[c] = 0.f;
    acc2[c] = 0.f;
  }
  const float Lag = (!BCAST && active) ? lse_ag[bh * nag + t] : 0.f;
  if (!BCAST && active && ch == 0) D_ag[bh * nag + t] = Dag;
  const int n0 = ch * chunk, n1 = min(N, n0 + chunk);
  const T* Xh = X + head_offset(sx, bh);
  const T* Yh = Y + head_offset(sx, bh);
  for (int nb = n0; nb < n1; nb += TS) {
    const int cnt = min(TS, n1 - nb);
    __syncthreads();
    for (int idx = t; idx < cnt * d; idx += 256) {
      const int tok = idx / d, c = idx - tok * d;
      Xs[tok][c] = to_f32(Xh[(long)(nb + tok) * sx.n + c]);
      Ys[tok][c] = to_f32(Yh[(long)(nb + tok) * sx.n + c]);
    }
    if (BCAST && t < cnt) {
      Ls[t] = lse_tok[bh * N + nb + t];
      Ds[t] = D_tok[bh * N + nb + t];
    }
    __syncthreads();
    if (active) {
      for (int tok = 0; tok < cnt; ++tok) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < MAXD; ++c)
          if (c < d) {
            s = fmaf(a[c], Xs[tok][c], s);
            dp = fmaf(wv[c], Ys[tok][c], dp);
          }
        const float p = fast_exp2(s * sl2 - (BCAST ? Ls[tok] : Lag));
        const float ds = p * (dp - (BCAST ? Ds[tok] : Dag));
#pragma unroll
        for (int c = 0; c < MAXD; ++c)
          if (c < d) {
            acc2[c] = fmaf(ds, Xs[tok][c], acc2[c]);
            if (BCAST) acc1[c] = fmaf(p, Ys[tok][c], acc1[c]);
          }
      }
    }
  }
  if (active) {
    const long o = ((bh * nchunks + ch) * (long)nag + t) * d;
#pragma unroll
    for (int c = 0; c < MAXD; ++c)
      if (c < d) {
        part2[o + c] = acc2[c];
        if (BCAST) part1[o + c] = acc1[c];
      }
  }
}

// out[bh][a][c] (+)= factor * sum over chunks of part[bh][chunk][a][c].
__global__ void __launch_bounds__(256)
bwd_sum_chunks(const float* __restrict__ part, float* __restrict__ out, long BH, int nag, int d,
               int nchunks, float factor, int accumulate) {
  const long n = BH * nag * d;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const long bh = i / ((long)nag * d), r = i - bh * nag * d;
    float s = 0.f;
    for (int j = 0; j < nchunks; ++j) s += part[(bh * nchunks + j) * (long)nag * d + r];
    out[i] = (accumulate ? out[i] : 0.f) + factor * s;
  }
}

// Token pass, one thread per token n, agent rows A and W streamed through
// LDS:  p = 2^(sl2 <X_n, A_a> - L),  ds = p (<Y_n, W_a> - D),
//   g[n] += ds A_a,   h[n] += p W_a (KV only).
// not KV (broadcast softmax): X = Q, Y = dO, W = V_A, L = lse2[n], D = D2[n]
//   -> G = dQ = scale g (+ the pooled agents' gradient dA spread over their
//   windows when pool is set).
// KV (aggregation softmax): X = K, Y = V, W = dV_A, L = lse1[a], D = D1[a]
//   -> G = dK = scale g, Hout = dV = h.
template <typename T, int MAXD, bool KV>
__global__ void __launch_bounds__(256)
bwd_token_pass(const T* __restrict__ X, const T* __restrict__ Y, const float* __restrict__ A,
               const float* __restrict__ W, const float* __restrict__ lse_tok,
               const float* __restrict__ D_tok, const float* __restrict__ lse_ag,
               const float* __restrict__ D_ag, const float* __restrict__ dA_pool,
               T* __restrict__ G, T* __restrict__ Hout, int N, int d, int nag, float sl2,
               float scale, int nqblk, Strides sx, int h, int w, int s) {
  constexpr int AC = MAXD > 64 ? 16 : 32;
  const int qb = blockIdx.x % nqblk;
  const long bh = blockIdx.x / nqblk;
  const int n = qb * 256 + threadIdx.x;
  const bool active = n < N;
  __shared__ float As[AC][MAXD];
  __shared__ float Ws[AC][MAXD];
  __shared__ float La[AC], Da[AC];
  const long ro = head_offset(sx, bh) + (long)(active ? n : 0) * sx.n;
  float xv[MAXD], yv[MAXD], g[MAXD], hv[MAXD];
#pragma unroll
  for (int c = 0; c < MAXD; ++c) {
    xv[c] = (active && c < d) ? to_f32(X[ro + c]) : 0.f;
    yv[c] = (active && c < d) ? to_f32(Y[ro + c]) : 0.f;
    g[c] = 0.f;
    hv[c] = 0.f;
  }
  const float Ltok = (!KV && active) ? lse_tok[bh * N + n] : 0.f;
  const float Dtok = (!KV && active) ? D_tok[bh * N + n] : 0.f;
  const float* Ah = A + bh * (long)nag * d;
  const float* Wh = W + bh * (long)nag * d;
  for (int a0 = 0; a0 < nag; a0 += AC) {
    const int cnt = min(AC, nag - a0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < cnt * d; idx += 256) {
      const int ag = idx / d, c = idx - ag * d;
      As[ag][c] = Ah[(long)(a0 + ag) * d + c];
      Ws[ag][c] = Wh[(long)(a0 + ag) * d + c];
    }
    if (KV && (int)threadIdx.x < cnt) {
      La[threadIdx.x] = lse_ag[bh * nag + a0 + threadIdx.x];
      Da[threadIdx.x] = D_ag[bh * nag + a0 + threadIdx.x];
    }
    __syncthreads();
    for (int ag = 0; ag < cnt; ++ag) {
      float sdot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < MAXD; ++c)
        if (c < d) {
          sdot = fmaf(xv[c], As[ag][c], sdot);
          dp = fmaf(yv[c], Ws[ag][c], dp);
        }
      const float p = fast_exp2(sdot * sl2 - (KV ? La[ag] : Ltok));
      const float ds = p * (dp - (KV ? Da[ag] : Dtok));
#pragma unroll
      for (int c = 0; c < MAXD; ++c)
        if (c < d) {
          g[c] = fmaf(ds, As[ag][c], g[c]);
          if (KV) hv[c] = fmaf(p, Ws[ag][c], hv[c]);
        }
    }
  }
  if (!active) return;
#pragma unroll
  for (int c = 0; c < MAXD; ++c) g[c] *= scale;
  if (!KV && dA_pool) {
    // the pooled agents' gradient: agent (i, j) averages rows
    // [floor(i h/s), ceil((i+1) h/s)) x columns [floor(j w/s), ceil((j+1) w/s))
    const int r = n / w, cc = n - r * w;
    const float* dAh = dA_pool + bh * (long)nag * d;
    const int i0 = max(0, (r * s) / h - 1), i1 = min(s - 1, (r * s) / h + 1);
    const int j0 = max(0, (cc * s) / w - 1), j1 = min(s - 1, (cc * s) / w + 1);
    for (int i = i0; i <= i1; ++i) {
      const int rs = (i * h) / s, re = ((i + 1) * h + s - 1) / s;
      if (r < rs || r >= re) continue;
      for (int j = j0; j <= j1; ++j) {
        const int cs = (j * w) / s, ce = ((j + 1) * w + s - 1) / s;
        if (cc < cs || cc >= ce) continue;
        const float inv = 1.0f / (float)((re - rs) * (ce - cs));
        const float* row = dAh + (long)(i * s + j) * d;
#pragma unroll
        for (int c = 0; c < MAXD; ++c)
          if (c < d) g[c] = fmaf(row[c], inv, g[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < MAXD; ++c)
    if (c < d) {
      G[ro + c] = from_f32<T>(g[c]);
      if (KV) Hout[ro + c] = from_f32<T>(hv[c]);
    }
}

// dagents [bh][a][c] (the caller's dtype) = dA.
template <typename T>
__global__ void __launch_bounds__(256)
bwd_store_agents(const float* __restrict__ dA, T* __restrict__ out, long n) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    out[i] = from_f32<T>(dA[i]);
}

}  // namespace aa
