// Token-feature projections of the attention module on matrix cores.
//
// The module ("Agent Attention: On the Integration of Softmax and Linear
// Attention", paperlayer.ai summary, §3 Preliminaries: projections W_Q, W_K,
// W_V map the channels to per-head queries, keys and values; "别再死磕Softmax
// 了！…", coreui.cn, §3.1: AgentAttention(dim, num_heads, num_agents) maps
// [B, N, dim] to [B, N, dim]) computes q, k, v = x W_qkv^T + b_qkv, agent
// attention per head, and y = o W_out^T + b_out.  The two projections here
// are plain products with fused layouts:
//   MODE 0 (q, k, v): rows of x [B*N, C] times the 3C rows of W_qkv; the
//     epilogue adds the bias and writes each output feature straight into
//     the head-major q, k, v tensors [B, H, N, d] that the attention reads
//     (feature f: tensor f / C, head (f % C) / d, channel f % d);
//   MODE 1 (output): the attention output o [B, H, N, d] read as token rows
//     of C = H d features (feature c = head c / d, channel c % d) times the
//     C rows of W_out, written as y [B*N, C].
// Weights are in the Linear layout [out_features, in_features], in the
// tensors' format; biases are float32.  Accumulation is float32 and each
// output is rounded once.
//
// Matrix-core mapping: output features are the MFMA rows (A operand = weight
// rows, contiguous in the input features) and tokens the columns (B operand
// = input rows), so a lane's result holds four consecutive output features
// of one token and stores them as one 8-byte (16-bit) or 16-byte (float32)
// piece.  proj_kernel (float32): workgroup tile 64 tokens (16 per wave) x 64
// output features, operands straight from memory.  16-bit formats use v_mfma_f32_16x16x32_{bf16,f16} (lane group g holds the
// eight inputs 32 j + 8 g ..); float32 uses v_mfma_f32_16x16x4f32 eight
// times per 32-wide slab, instruction e taking element e of every lane's
// eight (inputs {e, 8+e, 16+e, 24+e} of the slab), the same order on both
// operands.
#pragma once

#include "kernels_mfma.hpp"

namespace aa {
namespace pj {

constexpr int kThr = 256;
constexpr int kTok = 64;    // tokens per workgroup
constexpr int kFeat = 64;   // output features per workgroup (4 tiles of 16)

struct ProjParams {
  const void* x;        // MODE 0: [B*N, C]; MODE 1: o [B, H, N, d]
  const void* w;        // [Nout, C]
  const float* bias;    // [Nout] or null
  void* y;              // MODE 0: q, k, v, each [B, H, N, d], consecutive; MODE 1: [B*N, C]
  int M, C, Nout;       // tokens B*N, input features, output features
  int N, H, d;          // tokens per image, heads, head dim (C = H d)
};

// One 32-wide slab of input features for one row: 8 elements per lane.
template <class T>
struct Slab {
  uint4 v[sizeof(T) == 4 ? 2 : 1];
};

template <class T>
__device__ __forceinline__ Slab<T> load_slab(rsrc_t r, unsigned elem_off, bool ok) {
  Slab<T> s;
  if constexpr (sizeof(T) == 4) {
    s.v[0] = bld16<kPlain>(r, ok ? elem_off * 4 : kOOB);
    s.v[1] = bld16<kPlain>(r, ok ? elem_off * 4 + 16 : kOOB);
  } else {
    s.v[0] = bld16<kPlain>(r, ok ? elem_off * 2 : kOOB);
  }
  return s;
}

// acc += A-slab (weight row) x B-slab (input row).
template <class T, class El>
__device__ __forceinline__ f32x4 slab_mma(const Slab<T>& a, const Slab<T>& b, f32x4 acc) {
  if constexpr (sizeof(T) == 4) {
    const float* fa = reinterpret_cast<const float*>(a.v);
    const float* fb = reinterpret_cast<const float*>(b.v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[e], fb[e], acc, 0, 0, 0);
    return acc;
  } else {
    return El::mma(__builtin_bit_cast(bf16x8, a.v[0]), __builtin_bit_cast(bf16x8, b.v[0]), acc);
  }
}

// Four consecutive outputs of one token, rounded to the format, at dst.
template <class T, class El>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(dst) = float4{a, b, c, d};
  } else {
    *reinterpret_cast<uint2*>(dst) = uint2{El::pack2(a, b), El::pack2(c, d)};
  }
}

template <class T, class El, int MODE>
__global__ void __launch_bounds__(kThr) proj_kernel(ProjParams p) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int m = blockIdx.x * kTok + 16 * wave + r;   // this lane's token (B operand column)
  const int f0 = blockIdx.y * kFeat;
  const bool mv = m < p.M;
  const unsigned xbytes = (unsigned)((long)p.M * p.C * sizeof(T));
  const unsigned wbytes = (unsigned)((long)p.Nout * p.C * sizeof(T));
  const rsrc_t rx = rsrc_of(p.x, xbytes), rw = rsrc_of(p.w, wbytes);
  // MODE 1: token m of image b sits at row (b H + head) N + n of o
  int b = 0, n = 0;
  if (MODE == 1 && mv) {
    b = m / p.N;
    n = m - b * p.N;
  }
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < p.C; c0 += 32) {
    const int c = c0 + 8 * g;   // this lane's eight input features
    const bool cv = c < p.C;
    unsigned xo;
    if (MODE == 0) {
      xo = (unsigned)(m * p.C + c);
    } else {
      const int hd = c / p.d, ch = c - hd * p.d;
      xo = (unsigned)(((b * p.H + hd) * p.N + n) * p.d + ch);
    }
    const Slab<T> xs = load_slab<T>(rx, xo, mv && cv);
    Slab<T> ws[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int f = f0 + 16 * t + r;
      ws[t] = load_slab<T>(rw, (unsigned)(f * p.C + c), cv && f < p.Nout);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = slab_mma<T, El>(ws[t], xs, acc[t]);
  }
  if (!mv) return;
  T* y = reinterpret_cast<T*>(p.y);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int f = f0 + 16 * t + 4 * g;   // outputs f .. f+3 of token m
    if (f >= p.Nout) continue;
    float v[4] = {acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
    if (p.bias) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += p.bias[f + i];
    }
    T* dst;
    if (MODE == 0) {
      const int which = f / p.C, fc = f - which * p.C, hd = fc / p.d, ch = fc - hd * p.d;
      const int bb = m / p.N, nn = m - bb * p.N;
      dst = y + (long)which * p.M * p.C + ((long)(bb * p.H + hd) * p.N + nn) * p.d + ch;
    } else {
      dst = y + (long)m * p.Nout + f;
    }
    store4<T, El>(dst, v[0], v[1], v[2], v[3]);
  }
}

// 16-bit formats: LDS-tiled product.  Workgroup tile 128 tokens x 32 FT
// output features; the inputs are taken 64 at a time (two MFMA slabs of 32)
// through two LDS buffers (one when a single step covers the inputs), so that
// the next step's global loads travel while the current step's MFMAs run.  The four waves form a 2 x 2 grid: wave
// (wf, wt) computes features wf*16FT .. and tokens wt*64 .. (FT x 4 tiles of
// 16 x 16).  LDS rows hold 64 inputs padded to 72 (144 bytes), which spreads
// the 16 rows of an operand read over distinct banks.  The output tile is
// staged in LDS so that every store is a whole 16-byte piece of a row.
constexpr int kKStep = 64, kRow = kKStep + 8;

// LDS bytes: nbuf operand buffers (one when a single step covers the
// inputs), or the output tile staged in the epilogue if larger.
template <int FT>
constexpr int gemm16_lds_bytes(int nbuf) {
  return nbuf * (32 * FT + 128) * kRow * 2 > 128 * (32 * FT + 8) * 2
             ? nbuf * (32 * FT + 128) * kRow * 2
             : 128 * (32 * FT + 8) * 2;
}

// At most 128 registers per lane with 64-wide feature tiles: four workgroups
// per CU (the short products are latency-bound; more of them in flight).
template <class El, int MODE, int FT>
__global__ void __launch_bounds__(kThr, FT <= 2 ? 4 : 2) proj_gemm16(ProjParams p) {
  constexpr int WF = 32 * FT, WT = 128;
  constexpr int CPR = kKStep / 8;                                  // 16-byte chunks per row
  constexpr int NA = WF * CPR / kThr, NX = WT * CPR / kThr;       // chunks per thread
  static_assert(NA >= 1 && NA * kThr == WF * CPR, "feature tile");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nbuf = p.C > kKStep ? 2 : 1;
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem);               // [nbuf][WF][kRow]
  uint16_t* sX = sA + nbuf * WF * kRow;                           // [nbuf][WT][kRow]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int wf = wave & 1, wt = wave >> 1;
  // feature tiles fastest: the workgroups sharing a token tile run together
  // and read its inputs from the L2
  const int m0 = blockIdx.y * WT, f0 = blockIdx.x * WF;
  const unsigned xbytes = (unsigned)((long)p.M * p.C * 2);
  const unsigned wbytes = (unsigned)((long)p.Nout * p.C * 2);
  const rsrc_t rx = rsrc_of(p.x, xbytes), rw = rsrc_of(p.w, wbytes);
  // this thread's chunks c = tid + 256 e: row c / CPR, inputs (c % CPR) * 8 ..
  // (the same input offset for every e)
  const int kc = (tid % CPR) * 8;
  int xbase[NX];   // element offset of a chunk's token row, -1 past the tokens
#pragma unroll
  for (int e = 0; e < NX; ++e) {
    const int m = m0 + (tid + kThr * e) / CPR;
    if (MODE == 0) {
      xbase[e] = m < p.M ? m * p.C : -1;
    } else {
      const int b = m / p.N, n = m - b * p.N;
      xbase[e] = m < p.M ? (b * p.H * p.N + n) * p.d : -1;
    }
  }
  uint4 ra[NA], rxv[NX];
  auto gload = [&](int k0) {
    const int kk = k0 + kc;
    const bool kv = kk < p.C;
#pragma unroll
    for (int e = 0; e < NA; ++e) {
      const int f = f0 + (tid + kThr * e) / CPR;
      ra[e] = bld16<kPlain>(rw, (kv && f < p.Nout) ? (unsigned)((f * p.C + kk) * 2) : kOOB);
    }
    int xo = kk;
    if (MODE == 1) {
      const int hd = kk / p.d;
      xo = hd * p.N * p.d + (kk - hd * p.d);
    }
#pragma unroll
    for (int e = 0; e < NX; ++e)
      rxv[e] = bld16<kPlain>(rx, (kv && xbase[e] >= 0) ? (unsigned)((xbase[e] + xo) * 2) : kOOB);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int e = 0; e < NA; ++e)
      *reinterpret_cast<uint4*>(sA + (buf * WF + (tid + kThr * e) / CPR) * kRow + kc) = ra[e];
#pragma unroll
    for (int e = 0; e < NX; ++e)
      *reinterpret_cast<uint4*>(sX + (buf * WT + (tid + kThr * e) / CPR) * kRow + kc) = rxv[e];
  };
  gload(0);
  lstore(0);
  __syncthreads();
  f32x4 acc[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[ft][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  for (int k0 = 0; k0 < p.C; k0 += kKStep) {
    const bool more = k0 + kKStep < p.C;
    if (more) gload(k0 + kKStep);
    const uint16_t* A = sA + (buf * WF + wf * 16 * FT + r) * kRow + 8 * g;
    const uint16_t* X = sX + (buf * WT + wt * 64 + r) * kRow + 8 * g;
#pragma unroll
    for (int j = 0; j < kKStep / 32; ++j) {
      bf16x8 a[FT], b[4];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        a[ft] = *reinterpret_cast<const bf16x8*>(A + 16 * ft * kRow + 32 * j);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        b[tt] = *reinterpret_cast<const bf16x8*>(X + 16 * tt * kRow + 32 * j);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[ft][tt] = El::mma(a[ft], b[tt], acc[ft][tt]);
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // epilogue: the tile (bias added, rounded) goes through LDS [token][feature]
  // (the operand buffers are free after the last barrier), then every thread
  // stores whole 16-byte pieces of 8 features
  constexpr int OR = WF + 8;   // output tile row (elements)
  uint16_t* sO = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int fl = wf * 16 * FT + 16 * ft + 4 * g;   // tile-local outputs fl .. fl+3
    const int f = f0 + fl;
    float bias[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)   // biases are 4-byte aligned: scalar loads
      bias[i] = (p.bias && f < p.Nout) ? p.bias[f + i] : 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const f32x4 v = acc[ft][tt];
      *reinterpret_cast<uint2*>(sO + (wt * 64 + 16 * tt + r) * OR + fl) =
          uint2{El::pack2(v[0] + bias[0], v[1] + bias[1]), El::pack2(v[2] + bias[2], v[3] + bias[3])};
    }
  }
  __syncthreads();
  uint16_t* y = reinterpret_cast<uint16_t*>(p.y);
  constexpr int CPO = WF / 8;                  // 16-byte pieces per tile row
  constexpr int NO = WT * CPO / kThr;          // pieces per thread
  static_assert(NO * kThr == WT * CPO, "output tile");
#pragma unroll
  for (int e = 0; e < NO; ++e) {
    const int c = tid + kThr * e, row = c / CPO, fc = (c - row * CPO) * 8;
    const int m = m0 + row, f = f0 + fc;
    if (m >= p.M || f >= p.Nout) continue;
    long off;
    if (MODE == 0) {
      const int which = f / p.C, fr = f - which * p.C, hd = fr / p.d, ch = fr - hd * p.d;
      const int bb = m / p.N, nn = m - bb * p.N;
      off = (long)which * p.M * p.C + ((long)(bb * p.H + hd) * p.N + nn) * p.d + ch;
    } else {
      off = (long)m * p.Nout + f;
    }
    *reinterpret_cast<uint4*>(y + off) = *reinterpret_cast<const uint4*>(sO + row * OR + fc);
  }
}

// y [B*N, C] = the heads of o [B, H, N, d] side by side (module without an
// output projection).  One thread per (token, 8 channels).
template <class T>
__global__ void __launch_bounds__(256) heads_concat(const T* __restrict__ o, T* __restrict__ y,
                                                    int M, int N, int H, int d) {
  const int C = H * d, nch = C >> 3;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * nch) return;
  const int m = idx / nch, c = (idx - m * nch) * 8;
  const int b = m / N, n = m - b * N, hd = c / d, ch = c - hd * d;
  const T* src = o + ((long)(b * H + hd) * N + n) * d + ch;
  T* dst = y + (long)m * C + c;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
    *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(src + 4);
  } else {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
}

// Launchers (instantiated in proj.hip): float32 takes proj_kernel, 16-bit
// formats proj_gemm16 (128 output features per workgroup from 256 outputs,
// else 64).
int launch_proj(const ProjParams& p, int mode, int dtype, hipStream_t st);
int launch_heads_concat(const void* o, void* y, int M, int N, int H, int d, int dtype,
                        hipStream_t st);

}  // namespace pj
}  // namespace aa
