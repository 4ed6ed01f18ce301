// Matrix-core backward of Agent Attention for 16-bit tensors (bfloat16,
// float16) on gfx950.
//
// The forward being differentiated ("Agent Attention: On the Integration of
// Softmax and Linear Attention", paperlayer.ai summary, §4 Agent
// Transformer): A = pool(Q) (or caller agents), V_A = softmax(scale A K^T) V
// (softmax over the N tokens), O = softmax(scale Q A^T) V_A (softmax over
// the k agents).  Its gradients follow from the chain rule and the softmax
// Jacobian, dS = P * (dP - rowsum(P * dP)):
//   broadcast   dV_A = P2^T dO, dS2 from dP2 = dO V_A^T;
//               dQ = scale dS2 A, dA = scale dS2^T Q
//   aggregation dS1 from dP1 = dV_A V^T; dA += scale dS1 K,
//               dK = scale dS1^T A, dV = P1^T dV_A
//   pooling     dq = dQ + each window's share dA / |window| (done afterwards)
//
// Everything per token (a token's probabilities over the agents, its score
// gradients, its rows of dq, dk and dv) is computed in registers from k x d
// operands that a workgroup keeps in LDS; the k x d gradients and the
// aggregation statistics are sums over tokens, reduced in registers per
// workgroup and then across the workgroups of a head by small kernels.
// Passes, each one launch over (head, token range) or (head, agent):
//   stats    per agent: running max and sum of exp over the range's tokens and
//            the unnormalised sum of exp * v
//   merge    -> lse of every agent (log2 units of the scaled scores) and V_A
//   bcast    per token: P2, dP2, dS2, dQ (float32); partials of dA and dV_A
//   reduce   -> dV_A, dA (broadcast part), D1 = rowsum(dV_A * V_A), which is
//            rowsum(P1 * dP1) of the aggregation softmax
//   agg      per token: P1 = exp2(scaled score - lse), dP1, dS1, dk, dv;
//            partials of dA (aggregation part)
//   reduce   -> dA
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{bf16,f16}, wave64): for lane l,
// with r = l % 16 and g = l / 16, the A operand holds row r, the B operand
// column r, both the eight contraction indices of group g; the result holds
// column r and rows 4g..4g+3.  Scores are computed with the agents as rows
// and the wave's 16 tokens as columns, so that every lane holds one token:
// its softmax over the agents is a reduction over its own registers and the
// three other lanes of its column, and products contracting over the agents
// (dQ, dk, dv) take the probabilities or score gradients straight from the
// result registers as B operands (a pair of 16-agent tiles gives a lane the
// agents {4g..4g+3, 16+4g..16+4g+3}; the k x d operand is read from its
// transposed LDS copy in that order).  Products contracting over tokens (dA,
// dV_A) need the tokens along the contraction: the workgroup stages its 64
// tokens' probabilities, score gradients and input rows transposed in LDS,
// and the four waves share the k x d result tiles.  The stats pass instead
// takes the tokens as rows (lanes hold agents), which makes the running max
// per agent a per-lane value, and stages only V^T, per wave.
#pragma once

#include "kernels_mfma.hpp"

namespace aa {
namespace bw {

constexpr int kNW = 4;                  // waves per workgroup
constexpr int kThr = 64 * kNW;
constexpr int kStep = 16 * kNW;         // tokens per workgroup step (bcast, agg)
constexpr int kStatTok = 32 * kNW;      // tokens per workgroup step (stats)
constexpr int kSS = kStep + 8;          // staging rows [*][token]: 144 bytes
constexpr int kVS = 32 + 4;             // stats: per-wave V^T rows [channel][token]: 72 bytes
constexpr float kNegBig = -1e30f;       // running-max start (exp2 of differences stays finite)

// Precision.  The matrix cores take 16-bit operands.  Q, K, V and dO are
// exact in their format; the k x d operands (A, V_A, dV_A) and the
// probabilities and score gradients are not, and rounding them once to 16
// bits costs up to a few percent of the gradients' size: the softmax
// gradients are small differences (rowsum(dS) = 0), e.g. dP2 - rowsum(P2 dP2)
// cancels the part of V_A common to all agents.  Wherever that matters, such
// an operand enters as a pair hi + lo of 16-bit values (hi = x rounded, lo =
// x - hi rounded), i.e. two products, which leaves about 2^-16 of x: A in
// all scores and in dQ, V_A in dP2, dV_A in dP1 and dv, the probabilities
// in V_A and dV_A, dS2 in dQ and dS1 in dk.  Single 16-bit operands remain
// for A in dk, P1 in dv and the score gradients in dA.
template <int KT, int DT>
struct Geo {
  static constexpr int KP = 16 * KT;        // agents, padded to 16-agent tiles (KT even)
  static constexpr int DP = 32 * DT;        // channels, padded to 32-channel slabs
  static constexpr int DB = 2 * DT;         // 16-channel blocks
  static constexpr int RS = DP + 8;         // [agent][channel] LDS rows (elements)
  static constexpr int TS = KP + 4;         // [channel][agent] LDS rows (elements)
  static constexpr int NTILE = KT * DB;     // 16 x 16 tiles of a k x d result
  static constexpr int TPW = (NTILE + kNW - 1) / kNW;
  static constexpr int ROWS = KP * RS * 2, COLS = DP * TS * 2;
  static constexpr int STG = KP * kSS * 2, STGT = DP * kSS * 2;
  static constexpr int STATS_LOOP = 2 * ROWS + kNW * DP * kVS * 2;
  static constexpr int STATS_MERGE = 2 * KP * DP * 4 + 2 * kNW * KP * 4;
  static constexpr int STATS = STATS_LOOP > STATS_MERGE ? STATS_LOOP : STATS_MERGE;
  static constexpr int BCAST = 4 * ROWS + 2 * COLS + 2 * STG + STGT;
  static constexpr int AGG = 4 * ROWS + 3 * COLS + STG + STGT;
  // floats per workgroup partial
  static constexpr long PART_STATS = 2 * KP + (long)KP * DP;
  static constexpr long PART_BCAST = 2L * KP * DP;
  static constexpr long PART_AGG = (long)KP * DP;
};

struct BwdParams {
  const uint16_t* q;      // [BH, N, d] bits of the 16-bit format
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  uint16_t* dk;
  uint16_t* dv;
  const float* A;         // agents [BH, nag, d]
  float* VA;              // V_A [BH, nag, d]
  float* lse;             // [BH, nch, KP]: log2 of the aggregation softmax denominators
  float* dVA;             // [BH, nag, d]
  float* dA;              // [BH, nag, d]
  float* D1;              // [BH, nch, KP]
  float* dQ;              // [BH, N, d] float32 (without the pooling share)
  float* part;            // workgroup partials of the current pass
  const uint16_t* agents_in;   // caller agents [BH, nag, d], or null (pool q)
  uint16_t* dq;
  uint16_t* dagents;      // gradient of the caller agents (with agents_in)
  int BH, N, d, nag;
  int h, w, s;            // token grid and agent grid side
  // agent chunks (more than 64 agents: chunks of 64 run one launch each)
  int nch, chunk;         // chunks per head, this launch's chunk
  int a0, nagc;           // first agent and agent count of the chunk
  float* tst;             // [nch, BH, N, 4]: max, sum, sum of P dP of a chunk per token
  float* dKf;             // [BH, N, d] float32 sums of dk, dv over all chunks but the last
  float* dVf;
  int P, T;               // workgroups per head and tokens per workgroup of the pass
  float sl2, scale;       // scale * log2(e), scale
  long long* trace;       // phase timestamps (trace builds only)
};

// Phase timestamps for profiling builds (-DAGENT_ATTN_PHASE_TRACE): 16
// wall-clock stamps per workgroup of each token-tiled pass (region 0 stats,
// 1 bcast, 2 agg; 4096 workgroups each).  Compiled out otherwise.
#ifdef AGENT_ATTN_PHASE_TRACE
#define BW_STAMP(region, i)                                                                  \
  do {                                                                                       \
    if (p.trace && threadIdx.x == 0 && blockIdx.x < 4096)                                    \
      p.trace[((long)(region) * 4096 + blockIdx.x) * 16 + (i)] = (long long)wall_clock64();  \
  } while (0)
#else
#define BW_STAMP(region, i) \
  do {                      \
  } while (0)
#endif

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ bf16x8 as_frag(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// Two 4-element runs (8 bytes each) as one operand.
__device__ __forceinline__ bf16x8 lds8x2(const uint16_t* p0, const uint16_t* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  return as_frag(uint4{a.x, a.y, b.x, b.y});
}
template <int E>
__device__ __forceinline__ uint16_t elem(const uint4& f) {
  const unsigned w = (E >> 1) == 0 ? f.x : (E >> 1) == 1 ? f.y : (E >> 1) == 2 ? f.z : f.w;
  return (uint16_t)(w >> (16 * (E & 1)));
}
// The two values of a packed dword, widened (lo half first).
template <class El>
__device__ __forceinline__ float2 unpack2(unsigned w);
template <>
__device__ __forceinline__ float2 unpack2<ElemBF16>(unsigned w) {
  return float2{__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
}
template <>
__device__ __forceinline__ float2 unpack2<ElemF16>(unsigned w) {
  return float2{ElemF16::value((uint16_t)(w & 0xffffu)), ElemF16::value((uint16_t)(w >> 16))};
}
// Eight values as an operand: a's four, then b's four.
template <class El>
__device__ __forceinline__ bf16x8 pack8(const float (&a)[4], const float (&b)[4]) {
  return as_frag(uint4{El::pack2(a[0], a[1]), El::pack2(a[2], a[3]), El::pack2(b[0], b[1]),
                       El::pack2(b[2], b[3])});
}
// The same eight values as a pair hi + lo of operands.
template <class El>
__device__ __forceinline__ void split8(const float (&a)[4], const float (&b)[4], bf16x8& hi,
                                       bf16x8& lo) {
  const unsigned h[4] = {El::pack2(a[0], a[1]), El::pack2(a[2], a[3]), El::pack2(b[0], b[1]),
                         El::pack2(b[2], b[3])};
  const float2 u0 = unpack2<El>(h[0]), u1 = unpack2<El>(h[1]), u2 = unpack2<El>(h[2]),
               u3 = unpack2<El>(h[3]);
  hi = as_frag(uint4{h[0], h[1], h[2], h[3]});
  lo = as_frag(uint4{El::pack2(a[0] - u0.x, a[1] - u0.y), El::pack2(a[2] - u1.x, a[3] - u1.y),
                     El::pack2(b[0] - u2.x, b[1] - u2.y), El::pack2(b[2] - u3.x, b[3] - u3.y)});
}
__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wmax(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// A k x d float32 matrix into LDS as 16-bit hi and lo parts, zero outside
// nag x d: rows rh/rl [a * RS + c], columns (transpose) ch/cl [c * TS + a];
// any of rl, ch, cl may be null.  Each thread takes 2 x 2 blocks (agents a,
// a+1; channels c, c+1), so that every LDS write is a 4-byte pair; all the
// thread's loads are issued before the first is used.
template <class El, int KP, int DP, int RS, int TS>
__device__ void stage_kd(uint16_t* rh, uint16_t* rl, uint16_t* ch, uint16_t* cl,
                         const float* src, int nag, int d, int tid) {
  constexpr int NB = KP * DP / 4 / kThr;   // 2 x 2 blocks per thread
  static_assert(NB * 4 * kThr == KP * DP, "k x d tile not a multiple of the block");
  const rsrc_t rs = rsrc_of(src, (unsigned)(nag * d * 4));
  u32x2 x0[NB], x1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int blk = tid + b * kThr, a = 2 * (blk / (DP / 2)), c = 2 * (blk % (DP / 2));
    // rows past nag fall outside the range and read zeros; so do channels past d
    const unsigned o0 = c < d ? (unsigned)((a * d + c) * 4) : kOOB;
    const unsigned o1 = c < d ? (unsigned)(((a + 1) * d + c) * 4) : kOOB;
    x0[b] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)o0, 0, kPlain);
    x1[b] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)o1, 0, kPlain);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int blk = tid + b * kThr, a = 2 * (blk / (DP / 2)), c = 2 * (blk % (DP / 2));
    const float v00 = __uint_as_float(x0[b][0]), v01 = __uint_as_float(x0[b][1]);
    const float v10 = __uint_as_float(x1[b][0]), v11 = __uint_as_float(x1[b][1]);
    const unsigned h0 = El::pack2(v00, v01), h1 = El::pack2(v10, v11);   // rows a, a+1
    const float2 u0 = unpack2<El>(h0), u1 = unpack2<El>(h1);
    const unsigned l0 = El::pack2(v00 - u0.x, v01 - u0.y), l1 = El::pack2(v10 - u1.x, v11 - u1.y);
    *reinterpret_cast<unsigned*>(rh + a * RS + c) = h0;
    *reinterpret_cast<unsigned*>(rh + (a + 1) * RS + c) = h1;
    if (rl) {
      *reinterpret_cast<unsigned*>(rl + a * RS + c) = l0;
      *reinterpret_cast<unsigned*>(rl + (a + 1) * RS + c) = l1;
    }
    // columns c, c+1: the pairs (a, a+1)
    if (ch) {
      *reinterpret_cast<unsigned*>(ch + c * TS + a) = (h0 & 0xffffu) | (h1 << 16);
      *reinterpret_cast<unsigned*>(ch + (c + 1) * TS + a) = (h0 >> 16) | (h1 & 0xffff0000u);
    }
    if (cl) {
      *reinterpret_cast<unsigned*>(cl + c * TS + a) = (l0 & 0xffffu) | (l1 << 16);
      *reinterpret_cast<unsigned*>(cl + (c + 1) * TS + a) = (l0 >> 16) | (l1 & 0xffff0000u);
    }
  }
}

// Eight channels 32 s + 8 g .. of one token per slab s (zeros for channels
// past d and tokens not taken).
template <int DT>
__device__ __forceinline__ void load_frags(uint4 (&f)[DT], rsrc_t r, int tok, bool take, int d,
                                           int g) {
#pragma unroll
  for (int s = 0; s < DT; ++s) {
    const int c = 32 * s + 8 * g;
    f[s] = bld16<kPlain>(r, (take && c < d) ? (unsigned)((tok * d + c) * 2) : kOOB);
  }
}

// Writes the eight channels of frag f (this lane's token, channels 32 s + 8 g
// ..) into a [channel][token] staging column.
__device__ __forceinline__ void stage_col(uint16_t* p, const uint4& f, int stride) {
  p[0 * stride] = elem<0>(f);
  p[1 * stride] = elem<1>(f);
  p[2 * stride] = elem<2>(f);
  p[3 * stride] = elem<3>(f);
  p[4 * stride] = elem<4>(f);
  p[5 * stride] = elem<5>(f);
  p[6 * stride] = elem<6>(f);
  p[7 * stride] = elem<7>(f);
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (and those reads before the next writes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ stats
// Workgroup (head, slot) covers tokens [slot T, slot T + T); wave w takes the
// 32-token steps w, w + 4, ...  Scores have tokens as rows and agents as
// columns (lane = agent 16 kb + r).  Partial layout per workgroup: max[KP],
// sum[KP] (log2 units of the scaled scores), then U[KP][DP] = sum over the
// range of exp2(score - max) v.
template <class El, int KT, int DT>
__global__ void __launch_bounds__(kThr) bwd_stats_kernel(BwdParams p) {
  using C = Geo<KT, DT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x / p.P, slot = blockIdx.x - head * p.P;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int t0 = slot * p.T, t1 = min(p.N, t0 + p.T);
  const long hd = (long)head * p.N * p.d;
  BW_STAMP(0, 0);
  uint16_t* sAh = (uint16_t*)smem;
  uint16_t* sAl = sAh + C::KP * C::RS;
  uint16_t* sVT = sAl + C::KP * C::RS + wave * C::DP * kVS;
  const unsigned hbytes = (unsigned)(p.N * p.d * 2);
  const rsrc_t rk = rsrc_of(p.k + hd, hbytes), rv = rsrc_of(p.v + hd, hbytes);
  // the first step's rows travel while the agents are staged
  uint4 kf[2][DT], vf[2][DT];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tok = t0 + 32 * wave + 16 * h + r;
    load_frags<DT>(kf[h], rk, tok, tok < t1, p.d, g);
    load_frags<DT>(vf[h], rv, tok, tok < t1, p.d, g);
  }
  BW_STAMP(0, 1);
  const long agl = ((long)head * p.nag + p.a0) * p.d;   // the chunk's first agent row
  const long vh = (long)head * p.nch + p.chunk;            // (head, chunk)
  stage_kd<El, C::KP, C::DP, C::RS, C::TS>(sAh, sAl, nullptr, nullptr, p.A + agl, p.nagc, p.d,
                                           tid);
  __syncthreads();
  BW_STAMP(0, 2);
  float m[KT], ls[KT];
  f32x4 U[KT][C::DB];
#pragma unroll
  for (int kb = 0; kb < KT; ++kb) {
    m[kb] = kNegBig;
    ls[kb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) U[kb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int tok0 = t0 + 32 * wave; tok0 < t1; tok0 += 32 * kNW) {
    // V^T of the step: [channel][token] rows of this wave
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < DT; ++s) stage_col(sVT + (32 * s + 8 * g) * kVS + 16 * h + r, vf[h][s], kVS);
    bool tv[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[h][i] = tok0 + 16 * h + 4 * g + i < t1;
    bf16x8 pbh[KT], pbl[KT];
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      f32x4 x[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DT; ++s) {
          const int o = (16 * kb + r) * C::RS + 32 * s + 8 * g;
          acc = El::mma(as_frag(kf[h][s]), lds16(sAh + o), acc);
          acc = El::mma(as_frag(kf[h][s]), lds16(sAl + o), acc);
        }
        x[h] = acc;
      }
      float mx = kNegBig;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tv[h][i]) mx = fmaxf(mx, x[h][i] * p.sl2);
      mx = group4_max(mx);
      const float mn = fmaxf(m[kb], mx);
      const float f = fast_exp2(m[kb] - mn);
      m[kb] = mn;
      float pv[2][4], sum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[h][i] = tv[h][i] ? fast_exp2(x[h][i] * p.sl2 - mn) : 0.f;
          sum += pv[h][i];
        }
      ls[kb] = ls[kb] * f + sum;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) U[kb][db] *= f;
      split8<El>(pv[0], pv[1], pbh[kb], pbl[kb]);
    }
    BW_STAMP(0, 3);
    // the next step's rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tok = tok0 + 32 * kNW + 16 * h + r;
      load_frags<DT>(kf[h], rk, tok, tok < t1, p.d, g);
      load_frags<DT>(vf[h], rv, tok, tok < t1, p.d, g);
    }
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const uint16_t* row = sVT + (16 * db + r) * kVS;
      const bf16x8 va = lds8x2(row + 4 * g, row + 16 + 4 * g);
#pragma unroll
      for (int kb = 0; kb < KT; ++kb) {
        U[kb][db] = El::mma(va, pbh[kb], U[kb][db]);
        U[kb][db] = El::mma(va, pbl[kb], U[kb][db]);
      }
    }
    wave_lds_sync();
  }
  // combine the four waves: common max, then sums of the rescaled partials
#pragma unroll
  for (int kb = 0; kb < KT; ++kb) ls[kb] = group4_sum(ls[kb]);
  BW_STAMP(0, 4);
  __syncthreads();   // the agents and the V^T rows are dead from here
  BW_STAMP(0, 5);
  float* sU = (float*)smem;                       // [2][KP][DP]
  float* sM = sU + 2 * C::KP * C::DP;             // [kNW][KP]
  float* sL = sM + kNW * C::KP;                   // [kNW][KP]
  if (g == 0) {
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      sM[wave * C::KP + 16 * kb + r] = m[kb];
      sL[wave * C::KP + 16 * kb + r] = ls[kb];
    }
  }
  __syncthreads();
  float Mt[KT], Lt[KT];
#pragma unroll
  for (int kb = 0; kb < KT; ++kb) {
    const int a = 16 * kb + r;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, sM[w * C::KP + a]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) L += sL[w * C::KP + a] * fast_exp2(sM[w * C::KP + a] - M);
    Mt[kb] = M;
    Lt[kb] = L;
    const float f = fast_exp2(m[kb] - M);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) U[kb][db] *= f;
  }
  auto uaddr = [&](int buf, int kb, int db) {
    return reinterpret_cast<f32x4*>(sU + buf * C::KP * C::DP + (16 * kb + r) * C::DP + 16 * db +
                                    4 * g);
  };
  if (wave >= 2) {
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *uaddr(wave - 2, kb, db) = U[kb][db];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) U[kb][db] += *uaddr(wave, kb, db);
  }
  if (wave == 1) {   // reads and writes the same elements of buffer 1, lane by lane
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db) *uaddr(1, kb, db) = U[kb][db];
  }
  __syncthreads();
  BW_STAMP(0, 6);
  if (wave == 0 && p.P == 1) {
    // the workgroup holds the whole head: lse and V_A directly
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      const int a = 16 * kb + r;
      if (a >= p.nagc) continue;
      if (g == 0) p.lse[vh * C::KP + a] = Mt[kb] + log2f(Lt[kb]);
      const float inv = 1.0f / Lt[kb];
      float* va = p.VA + agl + (long)a * p.d;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        if (16 * db + 4 * g < p.d)
          *reinterpret_cast<f32x4*>(va + 16 * db + 4 * g) = (U[kb][db] + *uaddr(1, kb, db)) * inv;
    }
  } else if (wave == 0) {
    float* base = p.part + (vh * p.P + slot) * C::PART_STATS;
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      const int a = 16 * kb + r;
      if (g == 0) {
        base[a] = Mt[kb];
        base[C::KP + a] = Lt[kb];
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const f32x4 u = U[kb][db] + *uaddr(1, kb, db);
        *reinterpret_cast<f32x4*>(base + 2 * C::KP + a * C::DP + 16 * db + 4 * g) = u;
      }
    }
  }
  BW_STAMP(0, 7);
}

// Reductions over the workgroup partials of a head: one 256-thread block per
// (head, agent a < nag); wave w takes partials w, w + 4, ... in batches of 8
// loads in flight, lanes take channels lane and lane + 64, and the four waves
// add their sums through LDS.
constexpr int kRedBatch = 8;

// Sum over the four waves of (x0, x1) for channels (lane, lane + 64); the
// result is valid in wave 0.
__device__ __forceinline__ void block4_add(float& x0, float& x1, int wave, int lane) {
  __shared__ float red[kNW][128];
  red[wave][lane] = x0;
  red[wave][lane + 64] = x1;
  __syncthreads();
  if (wave == 0) {
    x0 = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    x1 = (red[0][lane + 64] + red[1][lane + 64]) + (red[2][lane + 64] + red[3][lane + 64]);
  }
}

// Block -> (head, agent) of a reduction: WPA = 4 waves per agent (one agent
// per block, many partials), or WPA = 1 (four agents per block, few
// partials).  `wave` is the wave's index within its agent.
template <int WPA>
__device__ __forceinline__ bool red_item(const BwdParams& p, int& head, int& a, int& wave,
                                         int& lane) {
  const int w = threadIdx.x >> 6;
  lane = threadIdx.x & 63;
  const int item = WPA > 1 ? blockIdx.x : blockIdx.x * kNW + w;
  wave = WPA > 1 ? w : 0;
  if (item >= p.BH * p.nag) return false;
  head = item / p.nag;
  a = item - head * p.nag;
  return true;
}

// lse[a] = M + log2(L) and V_A[a] = sum_j 2^(m_j - M) U_j[a] / L over the
// head's stats partials (M = max_j m_j, L = sum_j 2^(m_j - M) l_j).
template <int KT, int DT, int WPA>
__global__ void __launch_bounds__(256) bwd_stats_merge(BwdParams p) {
  using C = Geo<KT, DT>;
  int head, a, wave, lane;
  if (!red_item<WPA>(p, head, a, wave, lane)) return;
  const int c = a / C::KP, al = a - c * C::KP;   // agent chunk and index within it
  const long vh = (long)head * p.nch + c;
  const float* base = p.part + vh * p.P * C::PART_STATS;
  float M = kNegBig;
  for (int j = lane; j < p.P; j += 64) M = fmaxf(M, base[j * C::PART_STATS + al]);
  M = wmax(M);
  float L = 0.f;
  for (int j = lane; j < p.P; j += 64)
    L += base[j * C::PART_STATS + C::KP + al] * fast_exp2(base[j * C::PART_STATS + al] - M);
  L = wsum(L);
  const int c1 = C::DP > 64 ? lane + 64 : lane;   // second channel (DP = 128 only)
  float u0 = 0.f, u1 = 0.f;
  for (int j0 = wave; j0 < p.P; j0 += WPA * kRedBatch) {
    float w[kRedBatch], x0[kRedBatch], x1[kRedBatch];
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      const int j = min(j0 + WPA * e, p.P - 1);
      const float* pj = base + j * C::PART_STATS;
      w[e] = pj[al];
      x0[e] = pj[2 * C::KP + al * C::DP + (lane & (C::DP - 1))];
      x1[e] = pj[2 * C::KP + al * C::DP + c1];
    }
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      const float we = j0 + WPA * e < p.P ? fast_exp2(w[e] - M) : 0.f;
      u0 += we * x0[e];
      u1 += we * x1[e];
    }
  }
  if (WPA > 1) {
    block4_add(u0, u1, wave, lane);
    if (wave != 0) return;
  }
  const float inv = 1.0f / L;
  float* va = p.VA + ((long)head * p.nag + a) * p.d;
  if (lane < p.d) va[lane] = u0 * inv;
  if (C::DP > 64 && lane + 64 < p.d) va[lane + 64] = u1 * inv;
  if (lane == 0) p.lse[vh * C::KP + al] = M + log2f(L);
}

// ------------------------------------------------------------------ bcast
// Workgroup (head, slot) covers tokens [slot T, slot T + T) in steps of 64;
// wave w holds tokens 16 w .. 16 w + 15 of a step (lane column r).
// Partial layout per workgroup: dA[KP][DP] (unscaled), then dV_A[KP][DP].
// MODE 0: the head's agents form one chunk.  With several chunks of 64
// agents the softmax over agents spans launches: MODE 1 records, per token
// and chunk, the chunk's score maximum, its sum of exponentials and their
// dP2-weighted sum; MODE 2 combines those into the full normalisation and
// D = rowsum(P2 dP2), then runs the gradient products of its chunk.
template <class El, int KT, int DT, int MODE>
__global__ void __launch_bounds__(kThr) bwd_bcast_kernel(BwdParams p) {
  using C = Geo<KT, DT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x / p.P, slot = blockIdx.x - head * p.P;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int t0 = slot * p.T, t1 = min(p.N, t0 + p.T);
  const long hd = (long)head * p.N * p.d;
  BW_STAMP(1, 0);
  uint16_t* sAh = (uint16_t*)smem;           // A rows, hi and lo
  uint16_t* sAl = sAh + C::KP * C::RS;
  uint16_t* sVh = sAl + C::KP * C::RS;       // V_A rows, hi and lo
  uint16_t* sVl = sVh + C::KP * C::RS;
  uint16_t* sCh = sVl + C::KP * C::RS;       // A^T rows, hi and lo
  uint16_t* sCl = sCh + C::DP * C::TS;
  uint16_t* stg0 = sCl + C::DP * C::TS;      // [agent][token]: dS2 hi, then P2 hi
  uint16_t* stg1 = stg0 + C::KP * kSS;       // [agent][token]: P2 lo
  uint16_t* stgT = stg1 + C::KP * kSS;       // [channel][token]: Q, then dO
  const long ah = ((long)head * p.nag + p.a0) * p.d;   // the chunk's first agent row
  const long vh = (long)head * p.nch + p.chunk;          // (head, chunk)
  const int col = 16 * wave + r;
  const unsigned hbytes = (unsigned)(p.N * p.d * 2);
  const rsrc_t rq = rsrc_of(p.q + hd, hbytes), ro = rsrc_of(p.dout + hd, hbytes);
  // the first step's rows travel while the operands are staged
  uint4 qf[DT], of[DT];
  load_frags<DT>(qf, rq, t0 + col, t0 + col < t1, p.d, g);
  load_frags<DT>(of, ro, t0 + col, t0 + col < t1, p.d, g);
  stage_kd<El, C::KP, C::DP, C::RS, C::TS>(sAh, sAl, MODE == 1 ? nullptr : sCh,
                                           MODE == 1 ? nullptr : sCl, p.A + ah, p.nagc, p.d, tid);
  stage_kd<El, C::KP, C::DP, C::RS, C::TS>(sVh, sVl, nullptr, nullptr, p.VA + ah, p.nagc, p.d,
                                           tid);
  __syncthreads();
  BW_STAMP(1, 1);
  int step = 0;
  float* dQh = p.dQ + hd;
  f32x4 accA[C::TPW], accV[C::TPW];
#pragma unroll
  for (int u = 0; u < C::TPW; ++u) accA[u] = accV[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  // scores of padding agents get -inf (probability 0)
  float nb[KT][4];
#pragma unroll
  for (int kb = 0; kb < KT; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) nb[kb][i] = 16 * kb + 4 * g + i < p.nagc ? 0.f : -INFINITY;
  for (int tok0 = t0; tok0 < t1; tok0 += kStep) {
    const int tok = tok0 + col;
    const bool tv = tok < t1;
    uint4 qn[DT], on[DT];   // the next step's rows
    load_frags<DT>(qn, rq, tok + kStep, tok + kStep < t1, p.d, g);
    load_frags<DT>(on, ro, tok + kStep, tok + kStep < t1, p.d, g);
    // scores and dP2: rows = agents 16 kb + 4 g + i, column = this lane's token
    float x[KT][4], dp[KT][4];
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
      for (int s = 0; s < DT; ++s) {
        const int o = (16 * kb + r) * C::RS + 32 * s + 8 * g;
        a = El::mma(lds16(sAh + o), as_frag(qf[s]), a);
        a = El::mma(lds16(sAl + o), as_frag(qf[s]), a);
        b = El::mma(lds16(sVh + o), as_frag(of[s]), b);
        b = El::mma(lds16(sVl + o), as_frag(of[s]), b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[kb][i] = a[i] + nb[kb][i];
        dp[kb][i] = b[i];
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kb][i]);
    mx = group4_max(mx);
    float l = 0.f;
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[kb][i] = fast_exp2((x[kb][i] - mx) * p.sl2);
        l += x[kb][i];
      }
    l = group4_sum(l);
    if (MODE == 1) {
      // per-token statistics of this agent chunk: max, sum of 2^(x - max),
      // and the sum of 2^(x - max) dP2
      float S = 0.f;
#pragma unroll
      for (int kb = 0; kb < KT; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S += x[kb][i] * dp[kb][i];
      S = group4_sum(S);
      if (tv && g == 0)
        *reinterpret_cast<float4*>(p.tst + (((long)p.chunk * p.BH + head) * p.N + tok) * 4) =
            float4{mx, l, S, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < DT; ++s2) {
        qf[s2] = qn[s2];
        of[s2] = on[s2];
      }
      ++step;
      continue;
    }
    float inv, D = 0.f;
    if (MODE == 2) {
      // the softmax over all agents from every chunk's statistics of this token
      // (running maximum: sums rescale when it grows)
      float M = mx, L = 1.f, S = 0.f;
      if (tv) {
        M = -INFINITY;
        L = 0.f;
        for (int c2 = 0; c2 < p.nch; ++c2) {
          const float4 st = *reinterpret_cast<const float4*>(
              p.tst + (((long)c2 * p.BH + head) * p.N + tok) * 4);
          const float Mn = fmaxf(M, st.x);
          const float fo = fast_exp2((M - Mn) * p.sl2), fn = fast_exp2((st.x - Mn) * p.sl2);
          L = L * fo + st.y * fn;
          S = S * fo + st.z * fn;
          M = Mn;
        }
      }
      inv = tv ? fast_exp2((mx - M) * p.sl2) / L : 0.f;
#pragma unroll
      for (int kb = 0; kb < KT; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kb][i] *= inv;
      D = tv ? S / L : 0.f;
    } else {
      inv = tv ? 1.0f / l : 0.f;   // tokens past the range: P2 = dS2 = 0
#pragma unroll
      for (int kb = 0; kb < KT; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[kb][i] *= inv;
          D += x[kb][i] * dp[kb][i];
        }
      D = group4_sum(D);
    }
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[kb][i] = x[kb][i] * (dp[kb][i] - D);   // dS2
    if (step < 2) BW_STAMP(1, 2 + 5 * step);
    // dQ = scale dS2 A: rows = channels 16 db + 4 g + i, column = token
    bf16x8 dsh[KT / 2], dsl[KT / 2];
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) split8<El>(dp[2 * j], dp[2 * j + 1], dsh[j], dsl[j]);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* rh = sCh + (16 * db + r) * C::TS;
      const uint16_t* rl = sCl + (16 * db + r) * C::TS;
#pragma unroll
      for (int j = 0; j < KT / 2; ++j) {
        const bf16x8 ch = lds8x2(rh + 32 * j + 4 * g, rh + 32 * j + 16 + 4 * g);
        const bf16x8 cl = lds8x2(rl + 32 * j + 4 * g, rl + 32 * j + 16 + 4 * g);
        acc = El::mma(ch, dsh[j], acc);
        acc = El::mma(ch, dsl[j], acc);
        acc = El::mma(cl, dsh[j], acc);
      }
      if (tv && 16 * db + 4 * g < p.d) {
        f32x4* dst = reinterpret_cast<f32x4*>(dQh + (long)tok * p.d + 16 * db + 4 * g);
        *dst = p.chunk > 0 ? *dst + acc * p.scale : acc * p.scale;   // sum over agent chunks
      }
    }
    // dA += dS2^T Q over the step's tokens: tile (kb, db) has rows = agents
    // 16 kb + 4 g + i and column = channel 16 db + r
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) stg0[(16 * kb + 4 * g + i) * kSS + col] = El::bits(dp[kb][i]);
#pragma unroll
    for (int s = 0; s < DT; ++s) stage_col(stgT + (32 * s + 8 * g) * kSS + col, qf[s], kSS);
    if (step < 2) BW_STAMP(1, 3 + 5 * step);
    __syncthreads();
    if (step < 2) BW_STAMP(1, 4 + 5 * step);
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = wave + kNW * u;
      if (C::NTILE % kNW == 0 || t < C::NTILE) {
        const int kb = t / C::DB, db = t - kb * C::DB;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          accA[u] = El::mma(lds16(stg0 + (16 * kb + r) * kSS + 32 * j + 8 * g),
                            lds16(stgT + (16 * db + r) * kSS + 32 * j + 8 * g), accA[u]);
      }
    }
    __syncthreads();
    // dV_A += P2^T dO, P2 as hi + lo
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t hb = El::bits(x[kb][i]);
        stg0[(16 * kb + 4 * g + i) * kSS + col] = hb;
        stg1[(16 * kb + 4 * g + i) * kSS + col] = El::bits(x[kb][i] - El::value(hb));
      }
#pragma unroll
    for (int s = 0; s < DT; ++s) stage_col(stgT + (32 * s + 8 * g) * kSS + col, of[s], kSS);
    __syncthreads();
    if (step < 2) BW_STAMP(1, 5 + 5 * step);
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = wave + kNW * u;
      if (C::NTILE % kNW == 0 || t < C::NTILE) {
        const int kb = t / C::DB, db = t - kb * C::DB;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ao = (16 * kb + r) * kSS + 32 * j + 8 * g;
          const bf16x8 bo = lds16(stgT + (16 * db + r) * kSS + 32 * j + 8 * g);
          accV[u] = El::mma(lds16(stg0 + ao), bo, accV[u]);
          accV[u] = El::mma(lds16(stg1 + ao), bo, accV[u]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < DT; ++s2) {
      qf[s2] = qn[s2];
      of[s2] = on[s2];
    }
    if (step < 2) BW_STAMP(1, 6 + 5 * step);
    ++step;
  }
  if (MODE == 1) return;   // statistics only
  if (p.P == 1) {
    // the workgroup holds the whole head: dA, dV_A and D1 = rowsum(dV_A V_A)
    // directly; D1 from per-tile partial sums in LDS (staging rows are free)
    float* sD = reinterpret_cast<float*>(stg0);   // [DB][KP]
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = wave + kNW * u;
      if (C::NTILE % kNW == 0 || t < C::NTILE) {
        const int kb = t / C::DB, db = t - kb * C::DB, c = 16 * db + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = 16 * kb + 4 * g + i;
          float prod = 0.f;
          if (a < p.nagc && c < p.d) {
            const long o = ah + (long)a * p.d + c;
            p.dA[o] = accA[u][i] * p.scale;
            p.dVA[o] = accV[u][i];
            prod = accV[u][i] * p.VA[o];
          }
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) prod += __shfl_xor(prod, m);
          if (r == 0) sD[db * C::KP + a] = prod;
        }
      }
    }
    __syncthreads();
    if (tid < p.nagc) {
      float dd = 0.f;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) dd += sD[db * C::KP + tid];
      p.D1[vh * C::KP + tid] = dd;
    }
    return;
  }
  float* base = p.part + (vh * p.P + slot) * C::PART_BCAST;
#pragma unroll
  for (int u = 0; u < C::TPW; ++u) {
    const int t = wave + kNW * u;
    if (C::NTILE % kNW == 0 || t < C::NTILE) {
      const int kb = t / C::DB, db = t - kb * C::DB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (16 * kb + 4 * g + i) * C::DP + 16 * db + r;
        base[o] = accA[u][i];
        base[C::KP * C::DP + o] = accV[u][i];
      }
    }
  }
  BW_STAMP(1, 12);
}

// dA = scale sum_j dA_j and dV_A = sum_j dV_A_j over the head's bcast
// partials, and D1[a] = sum_c dV_A[a][c] V_A[a][c].
template <int KT, int DT, int WPA>
__global__ void __launch_bounds__(256) bwd_reduce_bcast(BwdParams p) {
  using C = Geo<KT, DT>;
  int head, a, wave, lane;
  if (!red_item<WPA>(p, head, a, wave, lane)) return;
  const int ch = a / C::KP, al = a - ch * C::KP;   // agent chunk and index within it
  const long vh = (long)head * p.nch + ch;
  const float* base = p.part + vh * p.P * C::PART_BCAST + al * C::DP;
  const int ca = lane & (C::DP - 1), cb = C::DP > 64 ? lane + 64 : lane;
  float sa0 = 0.f, sa1 = 0.f, sv0 = 0.f, sv1 = 0.f;
  for (int j0 = wave; j0 < p.P; j0 += WPA * kRedBatch) {
    float xa[kRedBatch], xb[kRedBatch], ya[kRedBatch], yb[kRedBatch];
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      const float* pj = base + min(j0 + WPA * e, p.P - 1) * C::PART_BCAST;
      xa[e] = pj[ca];
      xb[e] = pj[cb];
      ya[e] = pj[C::KP * C::DP + ca];
      yb[e] = pj[C::KP * C::DP + cb];
    }
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      if (j0 + WPA * e < p.P) {
        sa0 += xa[e];
        sa1 += xb[e];
        sv0 += ya[e];
        sv1 += yb[e];
      }
    }
  }
  if (WPA > 1) {
    block4_add(sa0, sa1, wave, lane);
    __syncthreads();
    block4_add(sv0, sv1, wave, lane);
    if (wave != 0) return;
  }
  const long o = ((long)head * p.nag + a) * p.d;
  float dd = 0.f;
  if (lane < p.d) {
    p.dA[o + lane] = sa0 * p.scale;
    p.dVA[o + lane] = sv0;
    dd += sv0 * p.VA[o + lane];
  }
  if (C::DP > 64 && lane + 64 < p.d) {
    p.dA[o + lane + 64] = sa1 * p.scale;
    p.dVA[o + lane + 64] = sv1;
    dd += sv1 * p.VA[o + lane + 64];
  }
  dd = wsum(dd);
  if (lane == 0) p.D1[vh * C::KP + al] = dd;
}

// ------------------------------------------------------------------ agg
// Workgroup (head, slot) covers tokens [slot T, slot T + T) in steps of 64.
// Writes dk and dv of its tokens; partial per workgroup: dA[KP][DP] (unscaled).
template <class El, int KT, int DT>
__global__ void __launch_bounds__(kThr) bwd_agg_kernel(BwdParams p) {
  using C = Geo<KT, DT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x / p.P, slot = blockIdx.x - head * p.P;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int t0 = slot * p.T, t1 = min(p.N, t0 + p.T);
  const long hd = (long)head * p.N * p.d;
  BW_STAMP(2, 0);
  uint16_t* sAh = (uint16_t*)smem;           // A rows, hi and lo
  uint16_t* sAl = sAh + C::KP * C::RS;
  uint16_t* sGh = sAl + C::KP * C::RS;       // dV_A rows, hi and lo
  uint16_t* sGl = sGh + C::KP * C::RS;
  uint16_t* sCh = sGl + C::KP * C::RS;       // A^T rows (hi)
  uint16_t* sHh = sCh + C::DP * C::TS;       // dV_A^T rows, hi and lo
  uint16_t* sHl = sHh + C::DP * C::TS;
  uint16_t* stg0 = sHl + C::DP * C::TS;      // dS1 hi [agent][token]
  uint16_t* stgT = stg0 + C::KP * kSS;       // K [channel][token]
  const long ah = ((long)head * p.nag + p.a0) * p.d;   // the chunk's first agent row
  const long vh = (long)head * p.nch + p.chunk;          // (head, chunk)
  const int col = 16 * wave + r;
  const unsigned hbytes = (unsigned)(p.N * p.d * 2);
  const rsrc_t rk = rsrc_of(p.k + hd, hbytes), rv = rsrc_of(p.v + hd, hbytes);
  // the first step's rows travel while the operands are staged
  uint4 kf[DT], vf[DT];
  load_frags<DT>(kf, rk, t0 + col, t0 + col < t1, p.d, g);
  load_frags<DT>(vf, rv, t0 + col, t0 + col < t1, p.d, g);
  stage_kd<El, C::KP, C::DP, C::RS, C::TS>(sAh, sAl, sCh, nullptr, p.A + ah, p.nagc, p.d, tid);
  stage_kd<El, C::KP, C::DP, C::RS, C::TS>(sGh, sGl, sHh, sHl, p.dVA + ah, p.nagc, p.d, tid);
  // lse and D1 of this lane's agent rows 16 kb + 4 g + i (padding agents: P1 = 0)
  float Lr[KT][4], Dr[KT][4];
#pragma unroll
  for (int kb = 0; kb < KT; ++kb) {
    const float4 l4 = *reinterpret_cast<const float4*>(p.lse + vh * C::KP + 16 * kb + 4 * g);
    const float4 d4 = *reinterpret_cast<const float4*>(p.D1 + vh * C::KP + 16 * kb + 4 * g);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool real = 16 * kb + 4 * g + i < p.nagc;
      Lr[kb][i] = real ? lv[i] : 1e30f;
      Dr[kb][i] = real ? dv4[i] : 0.f;
    }
  }
  __syncthreads();
  BW_STAMP(2, 1);
  int step = 0;
  uint16_t* dkh = p.dk + hd;
  uint16_t* dvh = p.dv + hd;
  f32x4 accA[C::TPW];
#pragma unroll
  for (int u = 0; u < C::TPW; ++u) accA[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int tok0 = t0; tok0 < t1; tok0 += kStep) {
    const int tok = tok0 + col;
    const bool tv = tok < t1;
    uint4 kn[DT], vn[DT];   // the next step's rows
    load_frags<DT>(kn, rk, tok + kStep, tok + kStep < t1, p.d, g);
    load_frags<DT>(vn, rv, tok + kStep, tok + kStep < t1, p.d, g);
    float pr[KT][4], ds[KT][4];
#pragma unroll
    for (int kb = 0; kb < KT; ++kb) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
      for (int s = 0; s < DT; ++s) {
        const int o = (16 * kb + r) * C::RS + 32 * s + 8 * g;
        a = El::mma(lds16(sAh + o), as_frag(kf[s]), a);
        a = El::mma(lds16(sAl + o), as_frag(kf[s]), a);
        b = El::mma(lds16(sGh + o), as_frag(vf[s]), b);
        b = El::mma(lds16(sGl + o), as_frag(vf[s]), b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[kb][i] = tv ? fast_exp2(a[i] * p.sl2 - Lr[kb][i]) : 0.f;
        ds[kb][i] = pr[kb][i] * (b[i] - Dr[kb][i]);
      }
    }
    if (step < 2) BW_STAMP(2, 2 + 4 * step);
    // dk = scale dS1^T A and dv = P1^T dV_A: rows = channels, column = token
    bf16x8 dsh[KT / 2], dsl[KT / 2], ph[KT / 2];
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) {
      split8<El>(ds[2 * j], ds[2 * j + 1], dsh[j], dsl[j]);
      ph[j] = pack8<El>(pr[2 * j], pr[2 * j + 1]);
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = ak;
      const uint16_t* ra = sCh + (16 * db + r) * C::TS;
      const uint16_t* rh = sHh + (16 * db + r) * C::TS;
      const uint16_t* rl = sHl + (16 * db + r) * C::TS;
#pragma unroll
      for (int j = 0; j < KT / 2; ++j) {
        const int o0 = 32 * j + 4 * g, o1 = 32 * j + 16 + 4 * g;
        const bf16x8 ca = lds8x2(ra + o0, ra + o1);
        ak = El::mma(ca, dsh[j], ak);
        ak = El::mma(ca, dsl[j], ak);
        av = El::mma(lds8x2(rh + o0, rh + o1), ph[j], av);
        av = El::mma(lds8x2(rl + o0, rl + o1), ph[j], av);
      }
      if (tv && 16 * db + 4 * g < p.d) {
        const long o = (long)tok * p.d + 16 * db + 4 * g;
        // over several agent chunks: float32 sums, rounded by the last chunk
        f32x4* fk = reinterpret_cast<f32x4*>(p.dKf + hd + o);
        f32x4* fv = reinterpret_cast<f32x4*>(p.dVf + hd + o);
        ak *= p.scale;
        if (p.chunk > 0) {
          ak += *fk;
          av += *fv;
        }
        if (p.chunk + 1 < p.nch) {
          *fk = ak;
          *fv = av;
        } else {
          *reinterpret_cast<uint2*>(dkh + o) =
              uint2{El::pack2(ak[0], ak[1]), El::pack2(ak[2], ak[3])};
          *reinterpret_cast<uint2*>(dvh + o) =
              uint2{El::pack2(av[0], av[1]), El::pack2(av[2], av[3])};
        }
      }
    }
    if (step < 2) BW_STAMP(2, 3 + 4 * step);
    // dA += dS1 K over the step's tokens
#pragma unroll
    for (int kb = 0; kb < KT; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) stg0[(16 * kb + 4 * g + i) * kSS + col] = El::bits(ds[kb][i]);
#pragma unroll
    for (int s = 0; s < DT; ++s) stage_col(stgT + (32 * s + 8 * g) * kSS + col, kf[s], kSS);
    __syncthreads();
    if (step < 2) BW_STAMP(2, 4 + 4 * step);
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = wave + kNW * u;
      if (C::NTILE % kNW == 0 || t < C::NTILE) {
        const int kb = t / C::DB, db = t - kb * C::DB;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          accA[u] = El::mma(lds16(stg0 + (16 * kb + r) * kSS + 32 * j + 8 * g),
                            lds16(stgT + (16 * db + r) * kSS + 32 * j + 8 * g), accA[u]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < DT; ++s2) {
      kf[s2] = kn[s2];
      vf[s2] = vn[s2];
    }
    if (step < 2) BW_STAMP(2, 5 + 4 * step);
    ++step;
  }
  if (p.P == 1) {   // the workgroup holds the whole head: add to dA directly
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int t = wave + kNW * u;
      if (C::NTILE % kNW == 0 || t < C::NTILE) {
        const int kb = t / C::DB, db = t - kb * C::DB, c = 16 * db + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = 16 * kb + 4 * g + i;
          if (a < p.nagc && c < p.d) p.dA[ah + (long)a * p.d + c] += accA[u][i] * p.scale;
        }
      }
    }
    return;
  }
  float* base = p.part + (vh * p.P + slot) * C::PART_AGG;
#pragma unroll
  for (int u = 0; u < C::TPW; ++u) {
    const int t = wave + kNW * u;
    if (C::NTILE % kNW == 0 || t < C::NTILE) {
      const int kb = t / C::DB, db = t - kb * C::DB;
#pragma unroll
      for (int i = 0; i < 4; ++i) base[(16 * kb + 4 * g + i) * C::DP + 16 * db + r] = accA[u][i];
    }
  }
  BW_STAMP(2, 10);
}

// dA += scale sum_j dA_j over the head's agg partials.
template <int KT, int DT, int WPA>
__global__ void __launch_bounds__(256) bwd_reduce_agg(BwdParams p) {
  using C = Geo<KT, DT>;
  int head, a, wave, lane;
  if (!red_item<WPA>(p, head, a, wave, lane)) return;
  const int ch = a / C::KP, al = a - ch * C::KP;   // agent chunk and index within it
  const float* base = p.part + ((long)head * p.nch + ch) * p.P * C::PART_AGG + al * C::DP;
  const int ca = lane & (C::DP - 1), cb = C::DP > 64 ? lane + 64 : lane;
  float s0 = 0.f, s1 = 0.f;
  for (int j0 = wave; j0 < p.P; j0 += WPA * kRedBatch) {
    float xa[kRedBatch], xb[kRedBatch];
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      const float* pj = base + min(j0 + WPA * e, p.P - 1) * C::PART_AGG;
      xa[e] = pj[ca];
      xb[e] = pj[cb];
    }
#pragma unroll
    for (int e = 0; e < kRedBatch; ++e) {
      if (j0 + WPA * e < p.P) {
        s0 += xa[e];
        s1 += xb[e];
      }
    }
  }
  if (WPA > 1) {
    block4_add(s0, s1, wave, lane);
    if (wave != 0) return;
  }
  const long o = ((long)head * p.nag + a) * p.d;
  if (lane < p.d) p.dA[o + lane] += s0 * p.scale;
  if (C::DP > 64 && lane + 64 < p.d) p.dA[o + lane + 64] += s1 * p.scale;
}

// ------------------------------------------------------------------ pooling and dq
// A = 2-D average pool of q over the s x s windows (rows [i h / s, ceil((i+1)
// h / s)), likewise for columns).  A group of U lanes (a power of two up to
// 64, about the window size) per (head, agent, 8-channel chunk); lane u sums
// the window's tokens u, u + U, ... and the group adds its U sums.
template <class El>
__global__ void __launch_bounds__(256) bwd_pool(const uint16_t* __restrict__ q,
                                                float* __restrict__ A, int BH, int N, int h,
                                                int w, int d, int s, int U) {
  const int nag = s * s, nch = d >> 3;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int item = gid / U, u = gid & (U - 1);
  const bool live = item < BH * nag * nch;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int bh = 0, agent = 0, ch = 0, cnt = 1;
  if (live) {
    ch = item % nch;
    const int ba = item / nch;
    agent = ba % nag;
    bh = ba / nag;
    const int i = agent / s, j = agent - i * s;
    const int r0 = (i * h) / s, r1 = ((i + 1) * h + s - 1) / s;
    const int c0 = (j * w) / s, c1 = ((j + 1) * w + s - 1) / s;
    const int ww = c1 - c0;
    cnt = (r1 - r0) * ww;
    const uint16_t* qh = q + (long)bh * N * d + ch * 8;
#pragma unroll 4
    for (int t = u; t < cnt; t += U) {
      const int rr = r0 + t / ww, cc = c0 + t % ww;
      const uint4 x = *reinterpret_cast<const uint4*>(qh + (long)(rr * w + cc) * d);
      const unsigned wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 f = unpack2<El>(wd[e]);
        acc[2 * e] += f.x;
        acc[2 * e + 1] += f.y;
      }
    }
  }
  for (int o = 1; o < U; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
  if (live && u == 0) {
    const float inv = 1.0f / (float)cnt;
    float* dst = A + ((long)bh * nag + agent) * d + ch * 8;
    *reinterpret_cast<float4*>(dst) = float4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<float4*>(dst + 4) =
        float4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
}

// dq (16-bit) = dQ + the pooling's share of dA: each window's agent gradient
// divided by its token count, for every window holding the token (dA null:
// supplied agents, dq = dQ).  One thread per (token, 8-channel chunk) of head
// blockIdx.y.  When s divides h and w the windows tile the grid and a token
// lies in exactly one (`tiled`); otherwise windows may overlap and the
// three candidates around r s / h (and c s / w) are tested.
template <class El>
__global__ void __launch_bounds__(256) bwd_finish_dq(const float* __restrict__ dQ,
                                                     const float* __restrict__ dA,
                                                     uint16_t* __restrict__ dq, int N, int h,
                                                     int w, int d, int s, int tiled) {
  const int nch = d >> 3;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= N * nch) return;
  const int bh = blockIdx.y;
  const int n = idx / nch, ch = idx - n * nch;
  const long e0 = ((long)bh * N + n) * d + ch * 8;
  float4 a = *reinterpret_cast<const float4*>(dQ + e0);
  float4 b = *reinterpret_cast<const float4*>(dQ + e0 + 4);
  auto add = [&](const float* pa, float inv) {
    const float4 x = *reinterpret_cast<const float4*>(pa);
    const float4 y = *reinterpret_cast<const float4*>(pa + 4);
    a = float4{a.x + x.x * inv, a.y + x.y * inv, a.z + x.z * inv, a.w + x.w * inv};
    b = float4{b.x + y.x * inv, b.y + y.y * inv, b.z + y.z * inv, b.w + y.w * inv};
  };
  if (dA) {
    const int nag = s * s;
    const int r = n / w, cc = n - r * w;
    const float* dAh = dA + (long)bh * nag * d + ch * 8;
    if (tiled) {
      const int wh = h / s, wwid = w / s;
      add(dAh + ((r / wh) * s + cc / wwid) * d, 1.0f / (float)(wh * wwid));
    } else {
      const int i0 = max(0, (r * s) / h - 1), i1 = min(s - 1, (r * s) / h + 1);
      const int j0 = max(0, (cc * s) / w - 1), j1 = min(s - 1, (cc * s) / w + 1);
      for (int i = i0; i <= i1; ++i) {
        const int rs = (i * h) / s, re = ((i + 1) * h + s - 1) / s;
        if (r < rs || r >= re) continue;
        for (int j = j0; j <= j1; ++j) {
          const int cs = (j * w) / s, ce = ((j + 1) * w + s - 1) / s;
          if (cc < cs || cc >= ce) continue;
          add(dAh + (i * s + j) * d, 1.0f / (float)((re - rs) * (ce - cs)));
        }
      }
    }
  }
  *reinterpret_cast<uint4*>(dq + e0) =
      uint4{El::pack2(a.x, a.y), El::pack2(a.z, a.w), El::pack2(b.x, b.y), El::pack2(b.z, b.w)};
}

// dst = src widened (float32) or narrowed (16-bit), n elements.
template <class El>
__global__ void __launch_bounds__(256) bwd_widen(const uint16_t* __restrict__ src,
                                                 float* __restrict__ dst, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
    dst[i] = El::value(src[i]);
}
template <class El>
__global__ void __launch_bounds__(256) bwd_narrow(const float* __restrict__ src,
                                                  uint16_t* __restrict__ dst, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
    dst[i] = El::bits(src[i]);
}

// ------------------------------------------------------------------ host side
// One pass's launch shape.
struct Pass {
  int P, T;   // workgroups per head, tokens per workgroup
};

template <int KT, int DT>
struct Lds {
  static constexpr int stats = Geo<KT, DT>::STATS, bcast = Geo<KT, DT>::BCAST,
                       agg = Geo<KT, DT>::AGG;
};

// Launches stats, merge, bcast, reduce, agg, reduce for the agents in p.A.
// `pp` carries the three passes' shapes (stats, bcast, agg).
template <class El, int KT, int DT>
int run_passes(BwdParams p, const Pass (&pp)[3], hipStream_t st) {
  using C = Geo<KT, DT>;
  // reductions: four waves per agent from 8 partials, else one
  const unsigned items = (unsigned)(p.BH * p.nag);
  auto rgrid = [&](int P) { return dim3(P > 8 ? items : (items + kNW - 1) / kNW); };
  auto set_chunk = [&](int c) {
    p.chunk = c;
    p.a0 = c * C::KP;
    p.nagc = min(C::KP, p.nag - p.a0);
  };
  const int nkd = p.BH * p.nag * p.d;
  const unsigned g_kd = (unsigned)std::min(4096, (nkd + 255) / 256);
  hipError_t e;
  if (p.agents_in) {
    bwd_widen<El><<<dim3(g_kd), dim3(256), 0, st>>>(p.agents_in, const_cast<float*>(p.A), nkd);
  } else {
    // lanes per window: about an eighth of its tokens (largest window), 1 to 8
    const int wmax = ((p.h + p.s - 1) / p.s + 1) * ((p.w + p.s - 1) / p.s + 1);
    int U = 1;
    while (U < 8 && 8 * U < wmax) U <<= 1;
    const long threads = (long)p.BH * p.nag * (p.d / 8) * U;
    bwd_pool<El><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(
        p.q, const_cast<float*>(p.A), p.BH, p.N, p.h, p.w, p.d, p.s, U);
  }
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  // aggregation statistics, chunk by chunk, then lse and V_A of every agent
  p.P = pp[0].P;
  p.T = pp[0].T;
  for (int c = 0; c < p.nch; ++c) {
    set_chunk(c);
    bwd_stats_kernel<El, KT, DT><<<dim3((unsigned)(p.BH * p.P)), dim3(kThr), C::STATS, st>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if (p.P > 8) bwd_stats_merge<KT, DT, 4><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  else if (p.P > 1) bwd_stats_merge<KT, DT, 1><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  // broadcast: one chunk directly; several through per-token statistics
  p.P = pp[1].P;
  p.T = pp[1].T;
  const dim3 gb((unsigned)(p.BH * p.P));
  if (p.nch == 1) {
    bwd_bcast_kernel<El, KT, DT, 0><<<gb, dim3(kThr), C::BCAST, st>>>(p);
  } else {
    for (int c = 0; c < p.nch; ++c) {
      set_chunk(c);
      bwd_bcast_kernel<El, KT, DT, 1><<<gb, dim3(kThr), C::BCAST, st>>>(p);
    }
    for (int c = 0; c < p.nch; ++c) {
      set_chunk(c);
      bwd_bcast_kernel<El, KT, DT, 2><<<gb, dim3(kThr), C::BCAST, st>>>(p);
    }
  }
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (p.P > 8) bwd_reduce_bcast<KT, DT, 4><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  else if (p.P > 1) bwd_reduce_bcast<KT, DT, 1><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  // aggregation gradients, chunk by chunk
  p.P = pp[2].P;
  p.T = pp[2].T;
  for (int c = 0; c < p.nch; ++c) {
    set_chunk(c);
    bwd_agg_kernel<El, KT, DT><<<dim3((unsigned)(p.BH * p.P)), dim3(kThr), C::AGG, st>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  if (p.P > 8) bwd_reduce_agg<KT, DT, 4><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  else if (p.P > 1) bwd_reduce_agg<KT, DT, 1><<<rgrid(p.P), dim3(256), 0, st>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  const int nq = p.N * (p.d / 8);
  const int tiled = (p.h % p.s == 0 && p.w % p.s == 0) ? 1 : 0;
  bwd_finish_dq<El><<<dim3((unsigned)((nq + 255) / 256), (unsigned)p.BH), dim3(256), 0, st>>>(
      p.dQ, p.agents_in ? nullptr : p.dA, p.dq, p.N, p.h, p.w, p.d, p.s, tiled);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (p.agents_in) bwd_narrow<El><<<dim3(g_kd), dim3(256), 0, st>>>(p.dA, p.dagents, nkd);
  return (int)hipGetLastError();
}

// Entry of the instance files: KT in {2, 4}, DT in {1, 2, 4}.
template <class El>
int run_backward_mfma(const BwdParams& p, int KT, int DT, const Pass (&pp)[3], hipStream_t st);

template <class El>
int run_backward_mfma_impl(const BwdParams& p, int KT, int DT, const Pass (&pp)[3],
                           hipStream_t st) {
  if (KT == 2) {
    if (DT == 1) return run_passes<El, 2, 1>(p, pp, st);
    if (DT == 2) return run_passes<El, 2, 2>(p, pp, st);
    return run_passes<El, 2, 4>(p, pp, st);
  }
  if (DT == 1) return run_passes<El, 4, 1>(p, pp, st);
  if (DT == 2) return run_passes<El, 4, 2>(p, pp, st);
  return run_passes<El, 4, 4>(p, pp, st);
}

// LDS bytes of the largest of the three token-tiled kernels.
inline int lds_bytes(int KT, int DT) {
  auto mx = [](int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); };
#define AA_BW_LDS(kt, dt) \
  if (KT == kt && DT == dt) return mx(Lds<kt, dt>::stats, Lds<kt, dt>::bcast, Lds<kt, dt>::agg);
  AA_BW_LDS(2, 1) AA_BW_LDS(2, 2) AA_BW_LDS(2, 4) AA_BW_LDS(4, 1) AA_BW_LDS(4, 2)
  AA_BW_LDS(4, 4)
#undef AA_BW_LDS
  return 1 << 30;
}

// Floats of one pass's partials for the whole batch.
inline long part_floats(int KT, int DT, long BH, const Pass (&pp)[3]) {
  const long KP = 16L * KT, DP = 32L * DT;
  const long s = BH * pp[0].P * (2 * KP + KP * DP), b = BH * pp[1].P * 2 * KP * DP,
             a = BH * pp[2].P * KP * DP;
  return s > b ? (s > a ? s : a) : (b > a ? b : a);
}

}  // namespace bw
}  // namespace aa
