// Matrix-core (MFMA) Agent Attention forward for bfloat16 I/O on gfx950.
//
// One kernel template runs any subset of the four phases of the forward
// (sources: "Agent Attention: On the Integration of Softmax and Linear
// Attention", paperlayer.ai summary, §4 Agent Transformer and §6 Conclusion;
// "Agent Attention：Transformer计算量太大？…", jsqmd.com, §1 pseudocode):
//   POOL       A   = 2-D average pool of Q (agents from the query space)
//   AGGREGATE  split-N partials of V_A = softmax(scale A K^T) V
//   MERGE      log-sum-exp merge of the partials into V_A
//   BROADCAST  O   = softmax(scale Q A^T) V_A
// Work is split into groups of P workgroups per (batch, head); workgroup j
// of a group owns tokens [j*T, (j+1)*T) for the aggregation and the
// broadcast and agents {j, j+P, ...} for pooling and merging.  In fused mode
// all phases run in one launch of a co-resident grid and the P workgroups of
// a head meet at three group barriers (after pooling, after the partials,
// after merging); otherwise the host launches the phases one after another
// and kernel boundaries order them.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): for lane l, with
// r = l % 16 and g = l / 16, the A operand holds row r, the B operand column
// r, and both hold the eight contraction indices of group g; the result holds
// column r and rows 4g..4g+3.  Contractions over the head dimension use the
// same index order on both operands (chunk DC*g + c of 8 channels), so the
// order never matters.  The two probability matrices are produced in the
// result layout and consumed directly as B operands: a pair of 16-wide tiles
// gives each lane the 8 contraction indices {4g..4g+3, 16+4g..16+4g+3}, and
// the value operands (V^T, V_A^T) are read in that same order.
#pragma once

#include "common.hpp"

namespace aa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

enum : int { PH_POOL = 1, PH_AGG = 2, PH_MERGE = 4, PH_BCAST = 8 };

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRoundTokens = 256;        // tokens of V staged in LDS at a time
constexpr int kVtPad = 8;                // LDS row padding (bf16) of staged V^T
constexpr int kBarriers = 3;
constexpr int kSyncStride = 32;          // dwords between counters (own 128 B line)
constexpr long kSpinLimit = 1L << 20;    // bounded waits: ~1 s, then an error

struct MfmaParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* out;
  const bf16_t* agents_in;      // caller agents [BH, nag, d] (bf16) or null
  const float* agents_f32_in;   // agents [BH, nag, d] fp32 (step calls) or null
  const float* values_f32_in;   // V_A [BH, nag, d] fp32 (step calls) or null
  float* agents_f32;            // pooled agents out [BH, nag, d]
  float* values_f32;            // V_A out [BH, nag, d]
  float* part;                  // partials [BH, nag, P, d + 2]
  unsigned* sync;               // group counters, zero between launches
  int* status;                  // nonzero after a barrier timed out
  int BH, N, h, w, d, s, nag;
  int P, T;                     // workgroups per head, tokens per workgroup
  float sl2;                    // scale * log2(e)
  int phases;
  int fused;
  int xcd_heads;                // >0: heads per XCD for the XCD-aware mapping
};

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float group4_max(float x) {
  x = fmaxf(x, shfl_xor_f(x, 16));
  return fmaxf(x, shfl_xor_f(x, 32));
}
__device__ __forceinline__ float group4_sum(float x) {
  x += shfl_xor_f(x, 16);
  return x + shfl_xor_f(x, 32);
}

// Device-coherent exchange of small data between the workgroups of a group:
// relaxed agent-scope accesses bypass the non-coherent caches; ordering comes
// from s_waitcnt before the barrier arrival (see group_barrier).
__device__ __forceinline__ void st_dev(float* p, float x) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}

// Barrier of the P workgroups of one head.  Counters start at zero in every
// launch: the last workgroup to finish the kernel resets them.  Every wave
// first waits for its own stores to complete, so data stored before the
// barrier is visible to device-coherent loads after it.
__device__ __forceinline__ bool group_barrier(unsigned* ctr, unsigned n, int* status) {
  __shared__ int ok;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    ok = 1;
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    long spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
      if (++spins > kSpinLimit) {
        ok = 0;
        __hip_atomic_store(reinterpret_cast<unsigned*>(status), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return ok != 0;
}

// Agent index held at contraction position e (0..7) of lane group g in the
// 32-wide chunk j of a probability tile pair.
__device__ __forceinline__ int pair_index(int j, int g, int e) {
  return 32 * j + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
}

// ------------------------------------------------------------ LDS operands
// A fragments: [KT][DC][64 lanes] x 8 bf16; fragment (t, c, lane) holds
// agents 16t + lane%16, channels 8*(DC*(lane/16) + c) .. +8.
template <int DC>
__device__ void load_agent_frags(bf16x8* lds, const MfmaParams& p, int head, bool device_coherent) {
  const int KT = (p.nag + 15) / 16;
  const int total = KT * DC * 64;
  const long hb = (long)head * p.nag * p.d;
  for (int f = threadIdx.x; f < total; f += kThreads) {
    const int lane = f & 63, c = (f >> 6) % DC, t = (f >> 6) / DC;
    const int agent = 16 * t + (lane & 15);
    const int ch0 = 8 * (DC * (lane >> 4) + c);
    union { bf16x8 v; __bf16 e[8]; } u;
    if (agent < p.nag && ch0 < p.d) {
      if (p.agents_in) {
        u.v = ld_bf16x8(p.agents_in + hb + (long)agent * p.d + ch0);
      } else {
        const float* src = (p.agents_f32_in ? p.agents_f32_in : p.agents_f32) + hb +
                           (long)agent * p.d + ch0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          u.e[e] = (__bf16)(device_coherent ? ld_dev(src + e) : src[e]);
      }
    } else {
      u.v = zero_bf16x8();
    }
    lds[f] = u.v;
  }
}

// V_A fragments: [KC][DT][64 lanes] x 8 bf16; fragment (j, dt, lane) holds
// channel 16dt + lane%16 of agents pair_index(j, lane/16, e).
template <int DC>
__device__ void load_value_frags(bf16x8* lds, const float* VA, const MfmaParams& p, int head,
                                 bool device_coherent) {
  constexpr int DT = 2 * DC;
  const int KC = (p.nag + 31) / 32;
  const int total = KC * DT * 64;
  const long hb = (long)head * p.nag * p.d;
  for (int f = threadIdx.x; f < total; f += kThreads) {
    const int lane = f & 63, dt = (f >> 6) % DT, j = (f >> 6) / DT;
    const int ch = 16 * dt + (lane & 15), g = lane >> 4;
    union { bf16x8 v; __bf16 e[8]; } u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int agent = pair_index(j, g, e);
      float x = 0.f;
      if (agent < p.nag && ch < p.d) {
        const float* src = VA + hb + (long)agent * p.d + ch;
        x = device_coherent ? ld_dev(src) : *src;
      }
      u.e[e] = (__bf16)x;
    }
    lds[f] = u.v;
  }
}

// ------------------------------------------------------------------ pooling
// Agents a = j, j+P, ... of the head: mean of Q over the agent's window.
// Wave w pools the agents with (a - j)/P = w mod 4.  Lane layout: DCH = d/8
// lanes per token, 64/DCH tokens per pass.
__device__ void pool_phase(const MfmaParams& p, int head, int j, float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int DCH = p.d >> 3;
  const int tpp = 64 / DCH;                    // tokens per pass
  const int ltok = lane / DCH, lch = lane - ltok * DCH;
  const bool lane_on = ltok < tpp;
  const bf16_t* Qh = p.q + (long)head * p.N * p.d;
  float* red_w = red + wave * 64 * 8;
  for (int a = j + p.P * wave; a < p.nag; a += p.P * kWaves) {
    const int ai = a / p.s, aj = a - ai * p.s;
    const int r0 = (ai * p.h) / p.s, r1 = ((ai + 1) * p.h + p.s - 1) / p.s;
    const int c0 = (aj * p.w) / p.s, c1 = ((aj + 1) * p.w + p.s - 1) / p.s;
    const int wc = c1 - c0;
    const int cnt = (r1 - r0) * wc;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (lane_on) {
      for (int t = ltok; t < cnt; t += tpp) {
        const int rr = r0 + t / wc, cc = c0 + t % wc;
        const bf16x8 x = ld_bf16x8(Qh + ((long)rr * p.w + cc) * p.d + 8 * lch);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red_w[lane * 8 + e] = acc[e];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // lanes < d: channel = lane (two passes for d > 64)
    const float inv = 1.0f / (float)cnt;
    for (int ch = lane; ch < p.d; ch += 64) {
      const int cchunk = ch >> 3, ce = ch & 7;
      float sum = 0.f;
      for (int t = 0; t < tpp; ++t) sum += red_w[(t * DCH + cchunk) * 8 + ce];
      float* dst = p.agents_f32 + ((long)head * p.nag + a) * p.d + ch;
      if (p.fused && p.P > 1) st_dev(dst, sum * inv); else *dst = sum * inv;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ------------------------------------------------------------ aggregation
// Per wave: agent tiles [4*ag, 4*ag+4) over the token blocks (32 tokens)
// b = tg, tg+TG, ... of the workgroup's slice.
template <int DC>
struct AggState {
  float m[4], l[4];
  f32x4 acc[4][2 * DC];
};

template <int DC>
__device__ __forceinline__ void agg_block(AggState<DC>& st, const bf16x8 (&kf)[2][DC],
                                          const bf16x8* Af, const bf16_t* Vt, int vt_stride,
                                          int blk_col, int ag, int KT, int valid, float sl2) {
  constexpr int DT = 2 * DC;
  const int lane = threadIdx.x & 63, g = lane >> 4;
  f32x4 S[2][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = 4 * ag + a;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) S[tt][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < KT) {
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 af = Af[(t * DC + c) * 64 + lane];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          S[tt][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt][c], af, S[tt][a], 0, 0, 0);
      }
    }
  }
  // mask tokens past the slice end (rows 16tt + 4g + i of the block)
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (16 * tt + 4 * g + i >= valid)
#pragma unroll
        for (int a = 0; a < 4; ++a) S[tt][a][i] = -INFINITY;
  // V^T fragments for this block: channel row 16dt + lane%16, tokens
  // {4g..4g+3} and {16+4g..16+4g+3} of the block.
  bf16x8 vf[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const bf16_t* row = Vt + (16 * dt + (lane & 15)) * vt_stride + blk_col + 4 * g;
    const uint2 lo = *reinterpret_cast<const uint2*>(row);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
    vf[dt] = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if (4 * ag + a >= KT) continue;
    float bm = fmaxf(fmaxf(fmaxf(S[0][a][0], S[0][a][1]), fmaxf(S[0][a][2], S[0][a][3])),
                     fmaxf(fmaxf(S[1][a][0], S[1][a][1]), fmaxf(S[1][a][2], S[1][a][3])));
    bm = group4_max(bm);
    const float mn = fmaxf(st.m[a], bm);
    const float corr = fast_exp2((st.m[a] - mn) * sl2);
    const float off = mn * sl2;
    union { bf16x8 v; __bf16 e[8]; } pf;
    float ps = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(S[tt][a][i], sl2, -off));
        ps += pv;
        pf.e[4 * tt + i] = (__bf16)pv;
      }
    st.l[a] = fmaf(st.l[a], corr, ps);
    st.m[a] = mn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.acc[a][dt] *= corr;
      st.acc[a][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf.v, st.acc[a][dt], 0, 0, 0);
    }
  }
}

template <int DC>
__device__ __forceinline__ void load_k_block(bf16x8 (&kf)[2][DC], const bf16_t* Kh, int tok0,
                                             int tok_end, int d) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tok = tok0 + 16 * tt + r;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int ch0 = 8 * (DC * g + c);
      kf[tt][c] = (tok < tok_end && ch0 < d) ? ld_bf16x8(Kh + (long)tok * d + ch0) : zero_bf16x8();
    }
  }
}

// Eight consecutive bf16 channels of one token -> one column of Vt (rows
// dst, dst + stride, ...).  Elements are taken out of the 32-bit words with
// shifts so that each 16-bit store gets its own element.
__device__ __forceinline__ void store_transposed8(bf16_t* dst, int stride, uint4 x) {
  const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    dst[e * stride] = static_cast<bf16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
}

// Stage V[tok0, tok0+cnt) of the head transposed into LDS: Vt[ch][col].
__device__ __forceinline__ void stage_v(bf16_t* Vt, int vt_stride, const bf16_t* Vh, int tok0,
                                        int cnt, int d) {
  const int DCH = d >> 3;
  const int total = cnt * DCH;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int t = i / DCH, ch = i - t * DCH;
    const uint4 x = *reinterpret_cast<const uint4*>(Vh + (long)(tok0 + t) * d + 8 * ch);
    store_transposed8(Vt + 8 * ch * vt_stride + t, vt_stride, x);
  }
}

// Zero the staged columns [cnt, cnt_pad) so that masked tokens contribute
// 0 * finite instead of 0 * garbage (garbage could be NaN).
__device__ __forceinline__ void zero_v_tail(bf16_t* Vt, int vt_stride, int cnt, int cnt_pad,
                                            int dpad) {
  const int w = cnt_pad - cnt;
  if (w <= 0) return;
  for (int i = threadIdx.x; i < w * dpad; i += kThreads) {
    const int ch = i / w, t = cnt + (i - ch * w);
    Vt[ch * vt_stride + t] = 0;
  }
}

// ------------------------------------------------------------ broadcast
template <int DC>
__device__ __forceinline__ void load_q_tile(bf16x8 (&qf)[DC], const bf16_t* Qh, int tok0,
                                            int tok_end, int d) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int tok = tok0 + r;
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const int ch0 = 8 * (DC * g + c);
    qf[c] = (tok < tok_end && ch0 < d) ? ld_bf16x8(Qh + (long)tok * d + ch0) : zero_bf16x8();
  }
}

template <int DC>
__device__ __forceinline__ void bcast_tile(const bf16x8 (&qf)[DC], const bf16x8* Af,
                                           const bf16x8* VAf, bf16_t* Oh, int tok0, int tok_end,
                                           int d, int nag, float sl2) {
  constexpr int DT = 2 * DC;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int KT = (nag + 15) / 16;
  const int nch = (KT + 3) / 4;
  f32x4 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, L = 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    f32x4 S[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = 4 * ch + a;
      S[a] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < KT) {
#pragma unroll
        for (int c = 0; c < DC; ++c)
          S[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Af[(t * DC + c) * 64 + lane], qf[c], S[a],
                                                         0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * t + 4 * g + i >= nag) S[a][i] = -INFINITY;
    }
    float cm = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      cm = fmaxf(cm, fmaxf(fmaxf(S[a][0], S[a][1]), fmaxf(S[a][2], S[a][3])));
    cm = group4_max(cm);
    const float mn = fmaxf(M, cm);
    const float corr = fast_exp2((M - mn) * sl2);
    const float off = mn * sl2;
    M = mn;
    L *= corr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] *= corr;
#pragma unroll
    for (int j2 = 0; j2 < 2; ++j2) {
      const int jj = 2 * ch + j2;
      if (32 * jj >= nag) break;
      union { bf16x8 v; __bf16 e[8]; } pf;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(S[2 * j2 + h2][i], sl2, -off));
          L += pv;
          pf.e[4 * h2 + i] = (__bf16)pv;
        }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(VAf[(jj * DT + dt) * 64 + lane], pf.v,
                                                        O[dt], 0, 0, 0);
    }
  }
  L = group4_sum(L);
  const float inv = 1.0f / L;
  const int tok = tok0 + r;
  if (tok < tok_end) {
    bf16_t* orow = Oh + (long)tok * d;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int ch = 16 * dt + 4 * g;
      if (ch < d) {
        union { uint2 u; __bf16 e[4]; } o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o.e[i] = (__bf16)(O[dt][i] * inv);
        *reinterpret_cast<uint2*>(orow + ch) = o.u;
      }
    }
  }
}

// ------------------------------------------------------------- the kernel
// LDS plan (bytes), computed identically on the host by mfma_lds_bytes():
//   [0, a_bytes)                  A fragments, KT*DC KiB
//   [a_bytes, a_bytes + big)      union of: staged V^T + pool scratch,
//                                 cross-wave partials, V_A fragments
template <int DC>
struct LdsPlan {
  int KT, KC, AG, TG;
  int a_bytes, vt_stride, vt_bytes, comb_bytes, va_bytes, pool_bytes, big, total;
  __host__ __device__ LdsPlan(int nag) {
    constexpr int DPAD = 32 * DC;
    KT = (nag + 15) / 16;
    KC = (nag + 31) / 32;
    AG = KT <= 4 ? 1 : (KT <= 8 ? 2 : 4);
    TG = kWaves / AG;
    a_bytes = KT * DC * 1024;
    vt_stride = kRoundTokens + kVtPad;
    vt_bytes = DPAD * vt_stride * 2;
    comb_bytes = (TG - 1) * AG * 64 * 4 * (2 * DC * 4 + 2) * 4;
    va_bytes = KC * 2 * DC * 1024;
    pool_bytes = kWaves * 64 * 8 * 4;
    big = vt_bytes;
    if (comb_bytes > big) big = comb_bytes;
    if (va_bytes > big) big = va_bytes;
    if (pool_bytes > big) big = pool_bytes;
    total = a_bytes + big;
  }
};

template <int DC>
__global__ void __launch_bounds__(kThreads)
agent_mfma_kernel(MfmaParams p) {
  constexpr int DT = 2 * DC;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const LdsPlan<DC> L(p.nag);
  bf16x8* Af = reinterpret_cast<bf16x8*>(smem);
  unsigned char* big = smem + L.a_bytes;

  // workgroup -> (head, slot)
  int head, slot;
  if (p.xcd_heads > 0) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    head = x * p.xcd_heads + i / p.P;
    slot = i % p.P;
  } else {
    head = blockIdx.x / p.P;
    slot = blockIdx.x % p.P;
  }
  if (head >= p.BH) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = slot * p.T;
  const int n1 = min(p.N, n0 + p.T);
  const long hoff = (long)head * p.N * p.d;
  unsigned* ctr = p.sync + (long)head * (kBarriers + 1) * kSyncStride;
  const bool sync_group = p.fused && p.P > 1;
  bool ok = true;

  // ---- prefetch: first K block pair of this wave and first query tiles
  const int ag = wave % L.AG, tg = wave / L.AG;
  bf16x8 kf[2][DC];
  const int nblk = n1 > n0 ? (n1 - n0 + 31) / 32 : 0;
  if ((p.phases & PH_AGG) && tg < nblk) load_k_block<DC>(kf, p.k + hoff, n0 + 32 * tg, n1, p.d);
  // V of the first round (up to kRoundTokens tokens), held in registers until
  // the pooling loads have been issued, then written transposed to LDS
  constexpr int VPF = 4 * DC;  // 16-byte pieces per thread for a full round
  uint4 vpf[VPF];
  const int DCH = p.d >> 3;
  const int r0cnt = n1 > n0 ? min(kRoundTokens, n1 - n0) : 0;
  if (p.phases & PH_AGG) {
#pragma unroll
    for (int u = 0; u < VPF; ++u) {
      const int f = threadIdx.x + kThreads * u;
      const int t = f / DCH, ch = f - t * DCH;
      if (t < r0cnt)
        vpf[u] = *reinterpret_cast<const uint4*>(p.v + hoff + (long)(n0 + t) * p.d + 8 * ch);
    }
  }
  constexpr int QPF = 2;  // query tiles prefetched per wave
  bf16x8 qf[QPF][DC];
  const int nqt = n1 > n0 ? (n1 - n0 + 15) / 16 : 0;
  if (p.phases & PH_BCAST) {
#pragma unroll
    for (int u = 0; u < QPF; ++u)
      if (wave + kWaves * u < nqt) load_q_tile<DC>(qf[u], p.q + hoff, n0 + 16 * (wave + kWaves * u), n1, p.d);
  }

  // ---- POOL
  if (p.phases & PH_POOL) {
    pool_phase(p, head, slot, reinterpret_cast<float*>(big));
    if (sync_group) ok = group_barrier(ctr + 0 * kSyncStride, p.P, p.status);
    __syncthreads();
  }
  const bool coherent = sync_group;  // data crosses workgroups only when P > 1

  // ---- agents -> LDS fragments
  if (p.phases & (PH_AGG | PH_BCAST)) {
    load_agent_frags<DC>(Af, p, head, coherent);
    __syncthreads();
  }

  // ---- AGGREGATE
  if (p.phases & PH_AGG) {
    AggState<DC> st;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      st.m[a] = -INFINITY;
      st.l[a] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.acc[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16_t* Vt = reinterpret_cast<bf16_t*>(big);
    const bf16_t* Kh = p.k + hoff;
    bool have_k = true;  // kf holds this wave's first block of the slice
    for (int rt0 = n0; rt0 < n1; rt0 += kRoundTokens) {
      const int rcnt = min(kRoundTokens, n1 - rt0);
      const int rcnt_pad = (rcnt + 31) / 32 * 32;
      __syncthreads();
      if (rt0 == n0) {
#pragma unroll
        for (int u = 0; u < VPF; ++u) {
          const int f = threadIdx.x + kThreads * u;
          const int t = f / DCH, ch = f - t * DCH;
          if (t < rcnt) store_transposed8(Vt + 8 * ch * L.vt_stride + t, L.vt_stride, vpf[u]);
        }
      } else {
        stage_v(Vt, L.vt_stride, p.v + hoff, rt0, rcnt, p.d);
      }
      zero_v_tail(Vt, L.vt_stride, rcnt, rcnt_pad, 32 * DC);
      __syncthreads();
      const int rblk = rcnt_pad / 32;
      for (int b = tg; b < rblk; b += L.TG) {
        const int tok0 = rt0 + 32 * b;
        if (!have_k) load_k_block<DC>(kf, Kh, tok0, n1, p.d);
        have_k = false;
        agg_block<DC>(st, kf, Af, Vt, L.vt_stride, 32 * b, ag, L.KT, min(32, n1 - tok0), p.sl2);
      }
      // a wave with no block in this round keeps its prefetched block for the next one
      if (tg >= rblk) have_k = false;
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) st.l[a] = group4_sum(st.l[a]);

    // combine the TG token groups of each agent group through LDS
    float* comb = reinterpret_cast<float*>(big);
    constexpr int REC = 2 * DC * 4 + 2;  // floats per lane per agent tile
    __syncthreads();
    if (tg > 0) {
      float* dst = comb + (((tg - 1) * L.AG + ag) * 64 * 4) * REC;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float* r = dst + (a * 64 + lane) * REC;
        r[0] = st.m[a];
        r[1] = st.l[a];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) r[2 + dt * 4 + i] = st.acc[a][dt][i];
      }
    }
    __syncthreads();
    if (tg == 0) {
      for (int o = 1; o < L.TG; ++o) {
        // the partner of wave (ag, 0) in token group o is wave o*AG + ag
        const float* src = comb + (((o - 1) * L.AG + ag) * 64 * 4) * REC;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float* r = src + (a * 64 + lane) * REC;
          const float m2 = r[0], l2 = r[1];
          const float mn = fmaxf(st.m[a], m2);
          const float c1 = (mn == -INFINITY) ? 0.f : fast_exp2((st.m[a] - mn) * p.sl2);
          const float c2 = (mn == -INFINITY) ? 0.f : fast_exp2((m2 - mn) * p.sl2);
          st.l[a] = st.l[a] * c1 + l2 * c2;
          st.m[a] = mn;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              st.acc[a][dt][i] = st.acc[a][dt][i] * c1 + r[2 + dt * 4 + i] * c2;
        }
      }
      // this wave now holds the workgroup's partial for agent tiles 4ag..4ag+3
      const int g = lane >> 4;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int agent = 16 * (4 * ag + a) + (lane & 15);
        if (agent >= p.nag) continue;
        if (p.P == 1) {
          // single slice: V_A directly
          const float inv = 1.0f / st.l[a];
          float* dst = p.values_f32 + ((long)head * p.nag + agent) * p.d;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ch = 16 * dt + 4 * g + i;
              if (ch < p.d) dst[ch] = st.acc[a][dt][i] * inv;
            }
        } else {
          float* dst = p.part + (((long)head * p.nag + agent) * p.P + slot) * (p.d + 2);
          if (g == 0) {
            if (coherent) { st_dev(dst, st.m[a]); st_dev(dst + 1, st.l[a]); }
            else { dst[0] = st.m[a]; dst[1] = st.l[a]; }
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ch = 16 * dt + 4 * g + i;
              if (ch < p.d) {
                if (coherent) st_dev(dst + 2 + ch, st.acc[a][dt][i]);
                else dst[2 + ch] = st.acc[a][dt][i];
              }
            }
        }
      }
    }
    if (sync_group && ok) ok = group_barrier(ctr + 1 * kSyncStride, p.P, p.status);
  }

  // ---- MERGE: agents a = slot, slot+P, ... ; one wave per agent, lanes over channels
  if ((p.phases & PH_MERGE) && p.P > 1 && ok) {
    for (int a = slot + p.P * wave; a < p.nag; a += p.P * kWaves) {
      const float* src = p.part + ((long)head * p.nag + a) * p.P * (p.d + 2);
      float M = -INFINITY;
      for (int sl = 0; sl < p.P; ++sl) M = fmaxf(M, coherent ? ld_dev(src + sl * (p.d + 2)) : src[sl * (p.d + 2)]);
      float Lsum = 0.f;
      float acc0 = 0.f, acc1 = 0.f;
      for (int sl = 0; sl < p.P; ++sl) {
        const float* r = src + sl * (p.d + 2);
        const float m = coherent ? ld_dev(r) : r[0];
        const float wgt = (m == -INFINITY) ? 0.f : fast_exp2((m - M) * p.sl2);
        Lsum = fmaf(coherent ? ld_dev(r + 1) : r[1], wgt, Lsum);
        if (lane < p.d) acc0 = fmaf(coherent ? ld_dev(r + 2 + lane) : r[2 + lane], wgt, acc0);
        if (lane + 64 < p.d)
          acc1 = fmaf(coherent ? ld_dev(r + 2 + lane + 64) : r[2 + lane + 64], wgt, acc1);
      }
      const float inv = 1.0f / Lsum;
      float* dst = p.values_f32 + ((long)head * p.nag + a) * p.d;
      if (lane < p.d) { if (coherent) st_dev(dst + lane, acc0 * inv); else dst[lane] = acc0 * inv; }
      if (lane + 64 < p.d) {
        if (coherent) st_dev(dst + lane + 64, acc1 * inv); else dst[lane + 64] = acc1 * inv;
      }
    }
    if (sync_group && ok) ok = group_barrier(ctr + 2 * kSyncStride, p.P, p.status);
  }

  // ---- BROADCAST
  if ((p.phases & PH_BCAST) && ok) {
    __syncthreads();
    bf16x8* VAf = reinterpret_cast<bf16x8*>(big);
    const float* VA = p.values_f32_in ? p.values_f32_in : p.values_f32;
    // single-slice fused runs read V_A written by this workgroup: a
    // workgroup barrier orders it (plain loads suffice)
    load_value_frags<DC>(VAf, VA, p, head, coherent && p.P > 1);
    __syncthreads();
    bf16_t* Oh = p.out + hoff;
    const bf16_t* Qh = p.q + hoff;
    int u = 0;
    for (int qt = wave; qt < nqt; qt += kWaves, ++u) {
      bf16x8 qcur[DC];
      if (u < QPF) {
#pragma unroll
        for (int uu = 0; uu < QPF; ++uu)
          if (uu == u)
#pragma unroll
            for (int c = 0; c < DC; ++c) qcur[c] = qf[uu][c];
      } else {
        load_q_tile<DC>(qcur, Qh, n0 + 16 * qt, n1, p.d);
      }
      bcast_tile<DC>(qcur, Af, VAf, Oh, n0 + 16 * qt, n1, p.d, p.nag, p.sl2);
    }
  }

  // ---- reset the group's counters once every workgroup of the group is done
  if (sync_group) {
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned* done = ctr + kBarriers * kSyncStride;
      const unsigned old = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (unsigned)p.P - 1) {
        for (int b = 0; b < kBarriers; ++b)
          __hip_atomic_store(ctr + b * kSyncStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace aa
