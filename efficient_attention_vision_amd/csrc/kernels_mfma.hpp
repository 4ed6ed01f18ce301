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
// after merging); with P = 1 one workgroup does everything for its head.
// Otherwise the host launches the phases one after another and kernel
// boundaries order them.
//
// Memory: every stream of Q, K, V goes through buffer loads whose range is
// the head (or the workgroup's slice), so that loads past the end return
// zeros without branches, and all loads a phase needs are issued before any
// of them is waited for.  The pooling loads are issued first (they start
// the dependency chain), then this workgroup's K blocks, V round and query
// tiles.  Data exchanged between the workgroups of a head (agents, partials,
// V_A) is written and read with the device-coherent cache policy in
// contiguous 16-byte pieces.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_bf16, wave64): for lane l, with
// r = l % 16 and g = l / 16, the A operand holds row r, the B operand column
// r, and both hold the eight contraction indices of group g; the result holds
// column r and rows 4g..4g+3.  Contractions over the head dimension use the
// same index order on both operands (chunk DC*g + c of 8 channels), so the
// order never matters.  The two probability matrices are produced in the
// result layout and consumed directly as B operands: a pair of 16-wide tiles
// gives each lane the 8 contraction indices {4g..4g+3, 16+4g..16+4g+3}, and
// the value operands (V^T, V_A^T) are read in that same order.  V_A enters
// the matrix cores as a bf16 pair hi + lo (two products) where LDS allows,
// so that only the agents, the probabilities and O itself are rounded.
#pragma once

#include "common.hpp"

namespace aa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

enum : int { PH_POOL = 1, PH_AGG = 2, PH_MERGE = 4, PH_BCAST = 8 };

constexpr int kWaves = 8;                // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBarriers = 3;
// Per-head synchronisation block (512 B): one flag byte per workgroup of the
// group (flag barriers), then the counters of the counting barriers and the
// counter of finished workgroups.
constexpr int kSyncDwords = 128;
constexpr int kMaxGroup = 256;           // flag bytes: at most 256 workgroups per head
constexpr int kCtrDword = 64;            // counters at dwords 64, 80, 96
constexpr int kCtrStride = 16;
constexpr int kDoneDword = kCtrDword + kBarriers * kCtrStride;
constexpr long kSpinLimit = 1L << 20;    // bounded waits: ~1 s, then an error
constexpr int kPoolTok = 8;              // window tokens per pooling work item
constexpr unsigned kOOB = 0x7ffffff0u;   // an offset past every buffer range

struct MfmaParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* out;
  const bf16_t* agents_in;      // caller agents [BH, nag, d] (bf16) or null
  const float* agents_f32_in;   // agents [BH, nag, d] fp32 (step calls) or null
  const float* values_f32_in;   // V_A [BH, nag, d] fp32 (step calls) or null
  float* agents_f32;            // agents [BH, nag, d] (exchange, or step output)
  float* values_f32;            // V_A [BH, nag, d] (exchange, staging, or step output)
  float* part_acc;              // partials [BH][P] x (KT*16 x DPAD), see Cfg::ROW_PARTIALS
  float* part_ml;               // partial max and sum [BH][P][KT][16][2]
  unsigned* sync;               // group counters, zero between launches
  int* status;                  // fault word (kFault* bits)
  int BH, N, h, w, d, s, nag;
  int P, T;                     // workgroups per head, tokens per workgroup
  int pool_tgp;                 // pooling token groups per (agent, chunk): power of 2
  int pool_tgp_log2;
  int pool_maxcnt;              // largest pooling window, in tokens
  float sl2;                    // scale * log2(e)
  int phases;
  unsigned char fused;          // one launch for all phases, groups synchronised inside
  unsigned char waves;          // host: 4 selects a four-wave instance (else 8)
  unsigned char dwc_halo_in_plan;   // 1: the staged DWC rows (dwc_halo_rows) sit in the
                                    // plan's LDS left free by the broadcast, else after it
  int xcd_heads;                // >0: heads per XCD for the XCD-aware mapping
  long spin_limit;              // polls before a group wait gives up (kSpinLimit)
  long long* trace;             // phase timestamps (trace builds only)
  long sb, sh;                  // q/k/v/out element strides of batch and head
  int H;                        // heads per batch entry (head index = b*H + h)
  int sn;                       // element stride between tokens (channels contiguous)
  // module terms (instances with MOD only; each pointer may be null)
  const float* bias_agg;        // B1 [H, nag, N], added to the scaled aggregation logits
  const float* bias_bcast;      // B2 [H, N, nag], added to the scaled broadcast logits
  const float* dwc_w;           // depth-wise 3x3 weights [H*d, 3, 3]
  const float* dwc_b;           // their bias [H*d] (null: zero)
  float inv_scale;              // 1 / scale: biases in units of the unscaled scores
  int dwc_halo_rows;            // > 0: V rows of a workgroup's tokens and their 3 x 3
                                // neighbourhood staged in LDS (this many at most)
};

// Module terms as a kernel sees them for its head (see MfmaParams).
struct ModCtx {
  rsrc_t b1, b2, rv;            // B1 and B2 of the head's parameters; V of the head
  const float* wl;              // DWC weights in LDS: [9][DPAD] taps, then [DPAD] bias
  const bf16_t* hv;             // V rows hr0 .. hr0 + hrows - 1 in LDS (hrows > 0)
  bool has_b1, has_b2, has_dwc;
  float inv_scale;
  int N, nag, w;
  int hr0, hrows;
};

// LDS of the DWC weights and bias in the MOD instances.
template <int DC>
constexpr int dwc_lds_bytes() { return 10 * 32 * DC * 4; }
// Elements per staged V row of the DWC (channels padded by 8: rows 16-byte
// aligned, and the 8-byte tap reads of 16 consecutive rows fall in distinct
// banks).
template <int DC>
constexpr int dwc_halo_stride() { return 32 * DC + 8; }
template <int DC>
constexpr long dwc_halo_lds_bytes(int rows) { return (long)rows * dwc_halo_stride<DC>() * 2; }

// Phase timestamps for profiling builds (-DAGENT_ATTN_PHASE_TRACE): 32
// wall-clock stamps per workgroup.  Compiled out otherwise.
#ifdef AGENT_ATTN_PHASE_TRACE
#define AA_STAMP(i)                                                            \
  do {                                                                         \
    if (p.trace && threadIdx.x == 0)                                           \
      p.trace[(long)blockIdx.x * 32 + (i)] = (long long)wall_clock64();        \
  } while (0)
#define AA_STAMP_BY(i, thread)                                                 \
  do {                                                                         \
    if (p.trace && threadIdx.x == (thread))                                    \
      p.trace[(long)blockIdx.x * 32 + (i)] = (long long)wall_clock64();        \
  } while (0)
#else
#define AA_STAMP(i) \
  do {              \
  } while (0)
#define AA_STAMP_BY(i, thread) \
  do {                         \
  } while (0)
#endif

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u});
}
// Reductions over the four 16-lane groups of a wave (lanes r, r+16, r+32,
// r+48) with the gfx950 row-swap permutes: after permlane16_swap(x, x) the
// two results hold x of lanes l and l^16 (in some order), after
// permlane32_swap those of l and l^32.
__device__ __forceinline__ float group4_max(float x) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// a / b for 0 <= a < 2^22, 1 <= b, given rb = 1/b (approximate reciprocal):
// the float estimate is within one of the quotient and one step fixes it.
__device__ __forceinline__ int idiv(int a, int b, float rb) {
  int q = (int)((float)a * rb);
  const int r = a - q * b;
  q += (r >= b) ? 1 : 0;
  q -= (r < 0) ? 1 : 0;
  return q;
}
__device__ __forceinline__ float rcp_approx(int b) { return __builtin_amdgcn_rcpf((float)b); }
__device__ __forceinline__ bf16_t bf16_bits(float x) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_value(bf16_t b) {
  return __uint_as_float(static_cast<unsigned>(b) << 16);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> one dword of two bfloat16 (lo in bits 0..15), one
// v_cvt_pk_bf16_f32 (round to nearest even)
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 16-bit element formats of the I/O tensors and of the matrix-core operands.
// Fragments are kept as 16-byte vectors (bf16x8) for both; only the
// conversions and the matrix-core instruction depend on the format.
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
struct ElemBF16 {
  static constexpr unsigned kOnes2 = 0x3f803f80u;   // two ones
  static __device__ __forceinline__ uint16_t bits(float x) { return bf16_bits(x); }
  static __device__ __forceinline__ float value(uint16_t b) { return bf16_value(b); }
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) { return pack_bf16(lo, hi); }
  static __device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
struct ElemF16 {
  static constexpr unsigned kOnes2 = 0x3c003c00u;
  static __device__ __forceinline__ uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));   // round to nearest even
  }
  static __device__ __forceinline__ float value(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
  }
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {   // v_cvt_pk_f16_f32
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
  }
  static __device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <class E>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  return E::pack2(lo, hi);
}
template <class E>
__device__ __forceinline__ bf16x8 ones8() {
  return __builtin_bit_cast(bf16x8, uint4{E::kOnes2, E::kOnes2, E::kOnes2, E::kOnes2});
}

// Buffer accesses.  CPol: kPlain = default caching; kL2 = sc0, which skips
// the CU's vector cache and is served by the XCD's L2 (coherent among the
// workgroups of one XCD); kCoherent = sc1, the device-coherent policy of
// agent-scope atomics (coherent across XCDs).
constexpr int kPlain = 0;
constexpr int kL2 = 1;
constexpr int kCoherent = 16;
constexpr int kStream = 2;   // nt: output written once and not read again here

// Policy of data that other workgroups of the group read after a barrier:
// 0 = no group (only this workgroup reads it), 1 = the group lives on one
// XCD (exchange through that XCD's L2), 2 = the group spans XCDs.
enum XPol { kXNone = 0, kXL2 = 1, kXDevice = 2 };

__device__ __forceinline__ rsrc_t rsrc_of(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
template <int POL>
__device__ __forceinline__ uint4 bld16(rsrc_t r, unsigned off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL);
  return uint4{x[0], x[1], x[2], x[3]};
}
template <int POL>
__device__ __forceinline__ float bld4(rsrc_t r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL));
}
template <int POL>
__device__ __forceinline__ void bst16(rsrc_t r, unsigned off, uint4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, r, (int)off, 0, POL);
}
template <int POL>
__device__ __forceinline__ void bst8(rsrc_t r, unsigned off, uint2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.x, x.y}, r, (int)off, 0, POL);
}
template <int POL>
__device__ __forceinline__ void bst4(rsrc_t r, unsigned off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)off, 0, POL);
}
// Runs f with the cache policy of the loads of exchange policy xp as a
// compile-time constant, so that loops of loads are instantiated per policy
// rather than branching around every load.
template <int V>
struct PolC {
  static constexpr int value = V;
};
// Loads of exchanged data are device-coherent (sc1) for both kinds of
// group: they skip the CU's vector cache, which may hold stale lines, and
// are served by the L2 when the writer is on the same XCD.
template <class F>
__device__ __forceinline__ void with_pol(int xp, F&& f) {
  if (xp != kXNone) f(PolC<kCoherent>{});
  else f(PolC<kPlain>{});
}
__device__ __forceinline__ void xst16(int xp, rsrc_t r, unsigned off, uint4 x) {
  if (xp == kXDevice) bst16<kCoherent>(r, off, x);
  else if (xp == kXL2) bst16<kL2>(r, off, x);
  else bst16<kPlain>(r, off, x);
}
__device__ __forceinline__ void xst8(int xp, rsrc_t r, unsigned off, uint2 x) {
  if (xp == kXDevice) bst8<kCoherent>(r, off, x);
  else if (xp == kXL2) bst8<kL2>(r, off, x);
  else bst8<kPlain>(r, off, x);
}
__device__ __forceinline__ uint4 f4_bits(float4 x) {
  return uint4{__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z),
               __float_as_uint(x.w)};
}
__device__ __forceinline__ float4 bits_f4(uint4 x) {
  return float4{__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                __uint_as_float(x.w)};
}

// Barrier of the P workgroups of one head, in two halves so that loads can
// be issued between the arrival and the wait.  Before arriving, every wave
// waits for its own loads and stores to complete, so data stored before the
// barrier is visible to the device-coherent (sc1) loads made after it.
//  - Group on one XCD: workgroup `slot` writes barrier number k+1 into its
//    flag byte through the XCD's L2; waiters read all P flags with sc1 loads
//    (one dword of four flags per lane of wave 0), which the L2 serves.
//  - Group over several XCDs: agent-scope atomic counter per barrier.
// Flags and counters are zero at the start of every launch: the last
// workgroup of the group to finish clears them.  Waits are bounded: on
// timeout the fault word gets kFaultBarrier and the workgroup stops.
struct GroupSync {
  unsigned* blk;   // this head's synchronisation block
  int slot, P;
  bool flags;      // flag barrier (group on one XCD)
  int* status;
  long spin_limit; // polls before a wait gives up
};
// Every wave that stored data the group reads after the barrier must pass
// `wait` (its stores complete before the flag or counter is published).
__device__ __forceinline__ void group_arrive(const GroupSync& g, int k, bool wait = true) {
  if (wait) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (g.flags) {
      const rsrc_t r = rsrc_of(g.blk, kMaxGroup);
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(k + 1), r, g.slot, 0, kL2);
    } else {
      __hip_atomic_fetch_add(g.blk + kCtrDword + k * kCtrStride, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}
// One wave (`poll_wave`) polls; a wave with no vector loads in flight sees
// the flags soonest (its poll results do not queue behind those loads).
__device__ __forceinline__ bool group_wait(const GroupSync& g, int k, int poll_wave = 0) {
  __shared__ int ok;
  if (g.flags) {
    if ((int)(threadIdx.x >> 6) == poll_wave) {
      const int lane = threadIdx.x & 63;
      const rsrc_t r = rsrc_of(g.blk, kMaxGroup);
      const int nw = (g.P + 3) >> 2;
      // bytes past P count as arrived
      const int past = 4 * lane + 4 - g.P;
      const unsigned pad = past <= 0 ? 0u : (past >= 4 ? 0xffffffffu : (0xffffffffu << (8 * (4 - past))));
      const unsigned want = 0x01010101u * (unsigned)(k + 1);
      long spins = 0;
      bool good = true;
      while (true) {
        const unsigned w = lane < nw ? (__builtin_amdgcn_raw_buffer_load_b32(r, 4 * lane, 0, kCoherent) | pad)
                                     : 0xffffffffu;
        // every byte >= k+1 (flags only ever hold 0..kBarriers)
        const unsigned lo = (w | 0x80808080u) - want;
        const bool arrived = ((~w & 0x80808080u) & ~lo) == 0u;
        if (__all(arrived)) break;
        if (++spins > g.spin_limit) {
          good = false;
          if (lane == 0)
            __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(g.status), kFaultBarrier,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) ok = good ? 1 : 0;
    }
  } else if (threadIdx.x == 0) {
    ok = 1;
    long spins = 0;
    unsigned* c = g.blk + kCtrDword + k * kCtrStride;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)g.P) {
      if (++spins > g.spin_limit) {
        ok = 0;
        __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(g.status), kFaultBarrier,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return ok != 0;
}
__device__ __forceinline__ bool group_barrier(const GroupSync& g, int k) {
  group_arrive(g, k);
  return group_wait(g, k);
}
// Called by every workgroup after its last barrier: the last one to get here
// clears the group's flags and counters for the next launch.
__device__ __forceinline__ void group_finish(const GroupSync& g) {
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(g.blk + kDoneDword, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last = old == (unsigned)g.P - 1;
  }
  __syncthreads();
  if (last && threadIdx.x < 64) {
    const rsrc_t r = rsrc_of(g.blk, kSyncDwords * 4);
    // flag dwords, the counters and the finished count (all of dwords 0..127
    // that are in use); device-coherent stores so any XCD sees them next time
    const int lane = threadIdx.x;
    bst4<kCoherent>(r, 4 * lane, 0.f);                                  // flags
    if (lane < kBarriers) bst4<kCoherent>(r, 4 * (kCtrDword + lane * kCtrStride), 0.f);
    if (lane == kBarriers) bst4<kCoherent>(r, 4 * kDoneDword, 0.f);
  }
}

// Agent index held at contraction position e (0..7) of lane group g in the
// 32-wide chunk j of a probability tile pair.
__device__ __forceinline__ int pair_index(int j, int g, int e) {
  return 32 * j + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
}

// 8 x 8 transpose of bf16: x[j] holds 8 channels of token j; the result y[e]
// holds channel e of tokens 0..7.
__device__ __forceinline__ void transpose8x8(const uint4 (&x)[8], uint4 (&y)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
    unsigned w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4 a = x[2 * jj], b = x[2 * jj + 1];
      const unsigned wa = (e >> 1) == 0 ? a.x : (e >> 1) == 1 ? a.y : (e >> 1) == 2 ? a.z : a.w;
      const unsigned wb = (e >> 1) == 0 ? b.x : (e >> 1) == 1 ? b.y : (e >> 1) == 2 ? b.z : b.w;
      w[jj] = __builtin_amdgcn_perm(wb, wa, sel);   // {a.elem(e), b.elem(e)}
    }
    y[e] = uint4{w[0], w[1], w[2], w[3]};
  }
}

// ------------------------------------------------------------ configuration
// Compile-time shape of one kernel instance: DC 32-channel chunks of the head
// dimension (DPAD = 32*DC >= d), KTC 16-agent tiles (16*KTC >= agents).
// V_A enters the broadcast products as bf16 hi + lo when there are at most
// 64 agents (registers allow it), as bf16 alone otherwise.
constexpr int vsplit_of(int ktc) { return ktc <= 4 ? 2 : 1; }
// Bytes per head of the agent and V_A fragment sets (bf16x8 per lane).
constexpr long a_frag_bytes(int ktc, int dc) { return (long)ktc * dc * 1024; }
constexpr long va_frag_bytes(int ktc, int dc) { return (long)vsplit_of(ktc) * (ktc / 2) * (2 * dc) * 1024; }

template <int DC, int KTC, int NW = kWaves>
struct Cfg {
  static constexpr int DT = 2 * DC;                // 16-channel output tiles
  static constexpr int DPAD = 32 * DC;
  static constexpr int RT = DC <= 2 ? 256 : 128;   // tokens per K/V round
  static constexpr int AG = KTC < NW ? KTC : NW;   // agent groups of waves
  static constexpr int ATW = KTC / AG;             // agent tiles per wave
  static constexpr int TG = NW / AG;               // token groups of waves
  static constexpr int KC = (KTC + 1) / 2;         // 32-agent chunks
  static constexpr int VSPLIT = vsplit_of(KTC);    // V_A as bf16 hi + lo
  // Partial accumulators as agent rows (coalesced merge reads; measured
  // faster from 128 agents) or in register order (up to 64 agents, where
  // the row addressing costs the kernel more registers than it saves).
  static constexpr bool ROW_PARTIALS = KTC >= 8;
  // LDS layout: [A fragments][big], big = union of
  //   pooling sums | {V^T, K rows} of a round | cross-wave partials |
  //   {V_A staging rows (if they fit), V_A fragments}
  static constexpr int A_BYTES = KTC * DC * 1024;
  static constexpr int VT_STRIDE = RT + 8;         // bf16, row = channel
  static constexpr int VT_BYTES = DPAD * VT_STRIDE * 2;
  static constexpr int KS_STRIDE = DPAD + 8;       // bf16, row = token
  static constexpr int KS_BYTES = RT * KS_STRIDE * 2;
  static constexpr int COMB_BYTES = (TG - 1) * AG * ATW * (DT + 1) * 1024;
  static constexpr int STAGE_BYTES = KTC * 16 * DPAD * 4;
  static constexpr int VA_BYTES = VSPLIT * KC * DT * 1024;
  static constexpr int POOL_BYTES = NW * 64 * 32;
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  static constexpr int BASE = mx(mx(VT_BYTES + KS_BYTES, COMB_BYTES), POOL_BYTES);
  static constexpr int kMaxLds = 160 * 1024 - 64;  // static LDS of the barrier flag
  static constexpr int STAGE_LDS = A_BYTES + mx(BASE, STAGE_BYTES + VA_BYTES) <= kMaxLds;
  static constexpr int BIG = mx(BASE, (STAGE_LDS ? STAGE_BYTES : 0) + VA_BYTES);
  static constexpr int TOTAL = A_BYTES + BIG;
};

// ------------------------------------------------------------------ pooling
// Agents a = slot + P*m (m < na) of the head.  Work item (m, chunk c, token
// group tg) sums window tokens tg, tg + TGP, ... (kPoolTok per pass) over 8
// channels; the TGP groups of a (m, c) pair are then added in a fixed order.
struct PoolGeo {
  int r0, c0, wc, cnt;
};
__device__ __forceinline__ PoolGeo pool_geo(const MfmaParams& p, int a) {
  const float rs = rcp_approx(p.s);
  const int ai = idiv(a, p.s, rs), aj = a - ai * p.s;
  const int r0 = idiv(ai * p.h, p.s, rs), r1 = idiv((ai + 1) * p.h + p.s - 1, p.s, rs);
  const int c0 = idiv(aj * p.w, p.s, rs), c1 = idiv((aj + 1) * p.w + p.s - 1, p.s, rs);
  return PoolGeo{r0, c0, c1 - c0, (r1 - r0) * (c1 - c0)};
}

__device__ __forceinline__ void pool_issue(const MfmaParams& p, rsrc_t rq, int slot, int item,
                                           int items, int tbase, uint4 (&x)[kPoolTok], int sn) {
  const int DCH = p.d >> 3, TGP = p.pool_tgp;
  const int pr = item >> p.pool_tgp_log2, tg = item - pr * TGP;
  const int m = idiv(pr, DCH, rcp_approx(DCH)), c = pr - m * DCH;
  const PoolGeo G = pool_geo(p, slot + p.P * m);
  const float rwc = rcp_approx(G.wc);
#pragma unroll
  for (int u = 0; u < kPoolTok; ++u) {
    const int t = tbase + tg + TGP * u;
    const int tq = idiv(t, G.wc, rwc);
    const int rr = G.r0 + tq, cc = G.c0 + (t - tq * G.wc);
    const unsigned off = (item < items && t < G.cnt)
                             ? (unsigned)(((rr * p.w + cc) * sn + 8 * c) * 2)
                             : kOOB;
    x[u] = bld16<kPlain>(rq, off);
  }
}

template <class E>
__device__ __forceinline__ void pool_accum(const uint4 (&x)[kPoolTok], float (&acc)[8]) {
#pragma unroll
  for (int u = 0; u < kPoolTok; ++u) {
    const unsigned w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc[e] += E::value((uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu)));
  }
}

// ---------------------------------------------------------- K / V staging
// 8-token x 8-channel tiles of K or V: tile `it` covers tokens
// tok0 + 8*(it / DCH) .. +8 and channels 8*(it % DCH) .. +8.  Tokens at or
// past tok_end load as zeros.
__device__ __forceinline__ void load_tile8(uint4 (&x)[8], rsrc_t r, int it, int tok0, int tok_end,
                                           int d, int sn) {
  const int DCH = d >> 3;
  const int t8 = idiv(it, DCH, rcp_approx(DCH)), ch = it - t8 * DCH;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = tok0 + 8 * t8 + j;
    x[j] = bld16<kPlain>(r, tok < tok_end ? (unsigned)((tok * sn + 8 * ch) * 2) : kOOB);
  }
}
// V tile -> transposed rows Vt[channel][token] of the round
__device__ __forceinline__ void store_tile_t(bf16_t* Vt, int vt_stride, const uint4 (&x)[8], int it,
                                             int d) {
  const int DCH = d >> 3;
  const int t8 = idiv(it, DCH, rcp_approx(DCH)), ch = it - t8 * DCH;
  uint4 y[8];
  transpose8x8(x, y);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint4*>(Vt + (8 * ch + e) * vt_stride + 8 * t8) = y[e];
}
// K tile -> rows Ks[token][channel] of the round
__device__ __forceinline__ void store_tile_rows(bf16_t* Ks, int ks_stride, const uint4 (&x)[8],
                                                int it, int d) {
  const int DCH = d >> 3;
  const int t8 = idiv(it, DCH, rcp_approx(DCH)), ch = it - t8 * DCH;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint4*>(Ks + (8 * t8 + j) * ks_stride + 8 * ch) = x[j];
}

// ------------------------------------------------------------ aggregation
// One wave: agent tiles [ATW*ag, ATW*ag + ATW) over its 32-token blocks.
template <int DC, int ATW>
struct AggState {
  float m[ATW], l[ATW], thr[ATW];
  f32x4 acc[ATW][2 * DC];
  f32x4 lacc[ATW];   // row sums of the probabilities, on the matrix cores
};

// B1 of one block for agent tile t of this lane: tokens tok0 + 4 g .. +3
// (b[0]) and tok0 + 16 + 4 g .. +3 (b[1]) of agent row 16 t + r, in score
// units; 16-byte loads when the rows are 16-byte aligned.
__device__ __forceinline__ void load_b1(const ModCtx& mc, int t, int tok0, float4 (&b)[2]) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int a = 16 * t + r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int n = tok0 + 16 * h + 4 * g;
    if ((mc.N & 3) == 0) {
      const unsigned o = (a < mc.nag && n < mc.N) ? (unsigned)((a * mc.N + n) * 4) : kOOB;
      b[h] = bits_f4(bld16<kPlain>(mc.b1, o));
    } else {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned o =
            (a < mc.nag && n + i < mc.N) ? (unsigned)((a * mc.N + n + i) * 4) : kOOB;
        x[i] = bld4<kPlain>(mc.b1, o);
      }
      b[h] = float4{x[0], x[1], x[2], x[3]};
    }
  }
}

template <class E, class C, int DC, int ATW, bool MOD>
__device__ __forceinline__ void agg_block(AggState<DC, ATW>& st, const bf16_t* Ks,
                                          const bf16x8* Af, const bf16_t* Vt, int blk_col, int ag,
                                          int valid, float sl2, const ModCtx& mc,
                                          const float4 (&b1)[ATW][2]) {
  constexpr int DT = 2 * DC;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  // K fragments: token row blk_col + 16tt + r, channel chunk DC*g + c
  // (chunks at or past d hold zeros)
  bf16x8 kf[2][DC];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int c = 0; c < DC; ++c)
      kf[tt][c] = *reinterpret_cast<const bf16x8*>(Ks + (blk_col + 16 * tt + r) * C::KS_STRIDE +
                                                   8 * (DC * g + c));
  // V^T fragments: channel row 16dt + r, tokens {4g..4g+3, 16+4g..16+4g+3}
  bf16x8 vf[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const bf16_t* row = Vt + (16 * dt + r) * C::VT_STRIDE + blk_col + 4 * g;
    const uint2 lo = *reinterpret_cast<const uint2*>(row);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
    vf[dt] = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
  }
#pragma unroll
  for (int a = 0; a < ATW; ++a) {
    const int t = ATW * ag + a;
    f32x4 S0 = f32x4{0.f, 0.f, 0.f, 0.f}, S1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const bf16x8 af = Af[(t * DC + c) * 64 + lane];
      S0 = E::mma(kf[0][c], af, S0);
      S1 = E::mma(kf[1][c], af, S1);
    }
    if constexpr (MOD) {
      if (mc.has_b1) {   // B1 of this block (loaded one block ahead), in score units
        S0[0] = fmaf(b1[a][0].x, mc.inv_scale, S0[0]);
        S0[1] = fmaf(b1[a][0].y, mc.inv_scale, S0[1]);
        S0[2] = fmaf(b1[a][0].z, mc.inv_scale, S0[2]);
        S0[3] = fmaf(b1[a][0].w, mc.inv_scale, S0[3]);
        S1[0] = fmaf(b1[a][1].x, mc.inv_scale, S1[0]);
        S1[1] = fmaf(b1[a][1].y, mc.inv_scale, S1[1]);
        S1[2] = fmaf(b1[a][1].z, mc.inv_scale, S1[2]);
        S1[3] = fmaf(b1[a][1].w, mc.inv_scale, S1[3]);
      }
    }
    if (valid < 32) {   // rows 16tt + 4g + i past the slice end
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= valid) S0[i] = -INFINITY;
        if (16 + 4 * g + i >= valid) S1[i] = -INFINITY;
      }
    }
    // Lazy rescaling: the reference max m of a row moves (and the running
    // sum and accumulators are rescaled) only when a block's max exceeds it
    // by more than 8 in the log2 domain (a score above thr = m + 8 / sl2),
    // so probabilities stay below 2^8: exact in the fp32 sums, and no loss
    // in bf16, whose precision is relative.  The first block always sets m
    // (m and thr start at -inf).  Each lane compares its own 8 scores; only
    // when one exceeds does the row max over the lane groups get formed.
    const float thr = st.thr[a];
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) over = over || S0[i] > thr || S1[i] > thr;
    if (__any(over)) {
      const float lm = fmaxf(fmaxf(fmaxf(S0[0], S0[1]), fmaxf(S0[2], S0[3])),
                             fmaxf(fmaxf(S1[0], S1[1]), fmaxf(S1[2], S1[3])));
      const float bm = group4_max(lm);
      const bool grow = (bm - st.m[a]) * sl2 > 8.f;
      const float mn = grow ? bm : st.m[a];
      const float corr = grow ? fast_exp2((st.m[a] - mn) * sl2) : 1.f;
      st.lacc[a] *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.acc[a][dt] *= corr;
      st.m[a] = mn;
      st.thr[a] = mn + 8.f / sl2;
    }
    const float off = st.m[a] * sl2;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = fast_exp2(fmaf(S0[i], sl2, -off));
      pv[4 + i] = fast_exp2(fmaf(S1[i], sl2, -off));
    }
    union { bf16x8 v; unsigned w[4]; } pf;
#pragma unroll
    for (int e = 0; e < 4; ++e) pf.w[e] = pack2<E>(pv[2 * e], pv[2 * e + 1]);
    // the sum over the block's tokens of the same bf16 probabilities that
    // enter P V (every row of the result holds it)
    st.lacc[a] = E::mma(ones8<E>(), pf.v, st.lacc[a]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      st.acc[a][dt] = E::mma(vf[dt], pf.v, st.acc[a][dt]);
  }
}

// ------------------------------------------------------------ broadcast
template <int DC>
__device__ __forceinline__ void load_q_tile(bf16x8 (&qf)[DC], rsrc_t rq, int tok0, int tok_end,
                                            int d, int sn) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int tok = tok0 + r;
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const int ch0 = 8 * (DC * g + c);
    const unsigned off = (tok < tok_end && ch0 < d) ? (unsigned)((tok * sn + ch0) * 2) : kOOB;
    qf[c] = __builtin_bit_cast(bf16x8, bld16<kPlain>(rq, off));
  }
}

// Initial broadcast logits of one 16-token query tile: B2[token tok0 + r]
// [agents 16t + 4g + i] in score units (module instances with B2), else
// zero.
template <int KTC, bool MOD>
__device__ __forceinline__ void bcast_bias(f32x4 (&S)[KTC], int nag, const ModCtx& mc, int tok0) {
#pragma unroll
  for (int t = 0; t < KTC; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (MOD) {
    if (mc.has_b2) {
      const int lane = threadIdx.x & 63, g = lane >> 4;
      int nag_t = nag;
      if (KTC >= 16) asm volatile("" : "+s"(nag_t));
      const int tok = tok0 + (lane & 15);
#pragma unroll
      for (int t = 0; t < KTC; ++t) {
        const int a0 = 16 * t + 4 * g;
        if ((mc.nag & 3) == 0) {
          const unsigned o = (tok < mc.N && a0 < nag_t) ? (unsigned)((tok * mc.nag + a0) * 4) : kOOB;
          const float4 x = bits_f4(bld16<kPlain>(mc.b2, o));
          S[t] = f32x4{x.x * mc.inv_scale, x.y * mc.inv_scale, x.z * mc.inv_scale,
                       x.w * mc.inv_scale};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const unsigned o =
                (tok < mc.N && a0 + i < nag_t) ? (unsigned)((tok * mc.nag + a0 + i) * 4) : kOOB;
            S[t][i] = bld4<kPlain>(mc.b2, o) * mc.inv_scale;
          }
        }
      }
    }
  }
}

// Broadcast logits and softmax of one 16-token query tile: P2 = softmax over
// the agents of scale * Q A^T (+ the initial logits S, see bcast_bias), as
// bf16 B-operand fragments pf[j] (agent pairs of chunk j, see pair_index)
// and the reciprocal of the row sum.
template <class E, class C, int DC, int KTC>
__device__ __forceinline__ void bcast_probs_from(f32x4 (&S)[KTC], const bf16x8 (&qf)[DC],
                                                 const bf16x8* Af, int nag, float sl2,
                                                 bf16x8 (&pf)[C::KC], float& inv) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  // When the agent and V_A fragments need more than 128 registers they
  // cannot all stay in registers across the caller's tile loop: the LDS
  // index and agent count are then made opaque per tile so that the fragment
  // reads and the padding compares are redone per tile instead of being
  // hoisted (and spilled).
  constexpr int kFragRegs = 4 * (KTC * DC + C::KC * 2 * DC * C::VSPLIT);
  int fl = lane, nag_t = nag;
  if (kFragRegs > 128 || KTC >= 16) {
    asm volatile("" : "+v"(fl));
    asm volatile("" : "+s"(nag_t));
  }
#pragma unroll
  for (int t = 0; t < KTC; ++t) {
#pragma unroll
    for (int c = 0; c < DC; ++c)
      S[t] = E::mma(Af[(t * DC + c) * 64 + fl], qf[c], S[t]);
  }
#pragma unroll
  for (int t = 0; t < KTC; ++t)
    if (16 * t + 16 > nag_t)   // padding agents of this tile
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * t + 4 * g + i >= nag_t) S[t][i] = -INFINITY;
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < KTC; ++t) M = fmaxf(M, fmaxf(fmaxf(S[t][0], S[t][1]), fmaxf(S[t][2], S[t][3])));
  M = group4_max(M);
  const float off = M * sl2;
  // row sums of the same bf16 probabilities that enter P V, on the matrix
  // cores (every row of the result holds the token's sum)
  f32x4 Lacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::KC; ++j) {
    float pv[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pv[4 * h2 + i] = fast_exp2(fmaf(S[2 * j + h2][i], sl2, -off));
    union { bf16x8 v; unsigned w[4]; } u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u.w[e] = pack2<E>(pv[2 * e], pv[2 * e + 1]);
    pf[j] = u.v;
    Lacc = E::mma(ones8<E>(), u.v, Lacc);
  }
  inv = 1.0f / Lacc[0];
}

template <class E, class C, int DC, int KTC, bool MOD>
__device__ __forceinline__ void bcast_probs(const bf16x8 (&qf)[DC], const bf16x8* Af, int nag,
                                            float sl2, bf16x8 (&pf)[C::KC], float& inv,
                                            const ModCtx& mc, int tok0) {
  f32x4 S[KTC];
  bcast_bias<KTC, MOD>(S, nag, mc, tok0);
  bcast_probs_from<E, C, DC, KTC>(S, qf, Af, nag, sl2, pf, inv);
}

// Depth-wise 3 x 3 convolution of V at grid position (row, col) for
// channels ch .. ch+3 and ch+16 .. ch+19: bias + sum over the taps inside
// the grid of weight * V (weights and bias from LDS, [9][32 DC] then
// [32 DC]).  Not inlined, so that its 18 loads stay within one call instead
// of being hoisted across the caller's tiles.
struct F8 {
  float4 lo, hi;
};
template <class E, int DC>
__device__ __attribute__((noinline)) F8 dwc8(rsrc_t rv, const float* wl, int rows, int w, int row,
                                             int col, int ch, int d, int sn) {
  constexpr int DPAD = 32 * DC;
  u32x2 v[2][9];
#pragma unroll
  for (int tap = 0; tap < 9; ++tap) {
    const int rr = row + tap / 3 - 1, cc = col + tap % 3 - 1;
    const bool in = rr >= 0 && rr < rows && cc >= 0 && cc < w;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[h][tap] = __builtin_amdgcn_raw_buffer_load_b64(
          rv, (in && ch + 16 * h < d) ? (int)(((rr * w + cc) * sn + ch + 16 * h) * 2) : (int)kOOB,
          0, kPlain);
  }
  float acc[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 b = *reinterpret_cast<const float4*>(wl + 9 * DPAD + ch + 16 * h);
    acc[h][0] = b.x;
    acc[h][1] = b.y;
    acc[h][2] = b.z;
    acc[h][3] = b.w;
#pragma unroll
    for (int tap = 0; tap < 9; ++tap) {
      const float4 wt = *reinterpret_cast<const float4*>(wl + tap * DPAD + ch + 16 * h);
      acc[h][0] = fmaf(wt.x, E::value((uint16_t)(v[h][tap][0] & 0xffffu)), acc[h][0]);
      acc[h][1] = fmaf(wt.y, E::value((uint16_t)(v[h][tap][0] >> 16)), acc[h][1]);
      acc[h][2] = fmaf(wt.z, E::value((uint16_t)(v[h][tap][1] & 0xffffu)), acc[h][2]);
      acc[h][3] = fmaf(wt.w, E::value((uint16_t)(v[h][tap][1] >> 16)), acc[h][3]);
    }
  }
  return F8{float4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]},
            float4{acc[1][0], acc[1][1], acc[1][2], acc[1][3]}};
}

// The same sum from V rows staged in LDS (ModCtx::hv, rows hr0 ..): the
// taps of every token of the workgroup lie in the staged range.
template <class E, int DC>
__device__ __forceinline__ F8 dwc8_lds(const ModCtx& mc, int rows, int row, int col, int ch) {
  constexpr int DPAD = 32 * DC, HS = dwc_halo_stride<DC>();
  float acc[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float4 b = *reinterpret_cast<const float4*>(mc.wl + 9 * DPAD + ch + 16 * h);
    acc[h][0] = b.x;
    acc[h][1] = b.y;
    acc[h][2] = b.z;
    acc[h][3] = b.w;
  }
#pragma unroll
  for (int tap = 0; tap < 9; ++tap) {
    const int rr = row + tap / 3 - 1, cc = col + tap % 3 - 1;
    if (rr < 0 || rr >= rows || cc < 0 || cc >= mc.w) continue;
    const bf16_t* src = mc.hv + (rr * mc.w + cc - mc.hr0) * HS + ch;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(src + 16 * h);
      const float4 wt = *reinterpret_cast<const float4*>(mc.wl + tap * DPAD + ch + 16 * h);
      acc[h][0] = fmaf(wt.x, E::value((uint16_t)(x[0] & 0xffffu)), acc[h][0]);
      acc[h][1] = fmaf(wt.y, E::value((uint16_t)(x[0] >> 16)), acc[h][1]);
      acc[h][2] = fmaf(wt.z, E::value((uint16_t)(x[1] & 0xffffu)), acc[h][2]);
      acc[h][3] = fmaf(wt.w, E::value((uint16_t)(x[1] >> 16)), acc[h][3]);
    }
  }
  return F8{float4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]},
            float4{acc[1][0], acc[1][1], acc[1][2], acc[1][3]}};
}

// Stores one normalised 16-token output tile held in the matrix-core result
// layout (O[dt]: channels 16 dt + 4 g .. +3 of token tok0 + r in lane (r, g)),
// with the depth-wise convolution term added in the MOD instances.
template <class E, int DC, bool MOD>
__device__ __forceinline__ void store_o_tile(const f32x4 (&O)[2 * DC], float inv, rsrc_t ro,
                                             int tok0, int tok_end, int d, int sn,
                                             const ModCtx& mc) {
  constexpr int DT = 2 * DC;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int tok = tok0 + r;
  float val[DT][4];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) val[dt][i] = O[dt][i] * inv;
  if constexpr (MOD) {
    if (mc.has_dwc) {
      // + DWC(V) for token tok = row * w + col (see dwc4)
      const int row = tok < tok_end ? idiv(tok, mc.w, rcp_approx(mc.w)) : -4;
      const int col = tok - row * mc.w;
#pragma unroll
      for (int dt = 0; dt < DT; dt += 2) {   // tiles dt and dt + 1 (channels +16)
        const F8 x = mc.hrows > 0
                         ? dwc8_lds<E, DC>(mc, mc.N / mc.w, row, col, 16 * dt + 4 * g)
                         : dwc8<E, DC>(mc.rv, mc.wl, mc.N / mc.w, mc.w, row, col,
                                       16 * dt + 4 * g, d, sn);
        val[dt][0] += x.lo.x;
        val[dt][1] += x.lo.y;
        val[dt][2] += x.lo.z;
        val[dt][3] += x.lo.w;
        val[dt + 1][0] += x.hi.x;
        val[dt + 1][1] += x.hi.y;
        val[dt + 1][2] += x.hi.z;
        val[dt + 1][3] += x.hi.w;
      }
    }
  }
  // Lane (r, g) holds channels 16 dt + 4 g .. +3 of token r for every dt.
  // Two 2 x 2 transposes between lane groups (permlane32_swap exchanges
  // lane-group bit 1 with the dt bit 0, permlane16_swap then exchanges
  // lane-group bit 0 with the source group's bit 1) leave lane (r, g) with
  // channels 64 q + 32 s + 8 g .. +7, so every store instruction writes
  // whole 64-byte segments of 16 rows instead of 8-byte pieces.
  unsigned pk[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    pk[dt][0] = pack2<E>(val[dt][0], val[dt][1]);
    pk[dt][1] = pack2<E>(val[dt][2], val[dt][3]);
  }
  constexpr int NS = DT >= 4 ? 2 : 1;
#pragma unroll
  for (int q = 0; q < (DT + 3) / 4; ++q)
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int d0 = 4 * q + 2 * s2, d1 = d0 + 1;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const u32x2 x = __builtin_amdgcn_permlane32_swap(pk[d0][w], pk[d1][w], false, false);
        const u32x2 y = __builtin_amdgcn_permlane16_swap(x[0], x[1], false, false);
        pk[d0][w] = y[0];
        pk[d1][w] = y[1];
      }
      const int c0 = 64 * q + 32 * s2 + 8 * g;
      const unsigned off2 = (tok < tok_end && c0 < d) ? (unsigned)((tok * sn + c0) * 2) : kOOB;
      bst16<kStream>(ro, off2, uint4{pk[d0][0], pk[d0][1], pk[d1][0], pk[d1][1]});
    }
}

// Broadcast output of one query tile: O = P2 V_A (V_A as bf16 hi + lo when
// VSPLIT = 2), normalised, rounded to bf16 and stored.
template <class E, class C, int DC, int KTC, bool MOD>
__device__ __forceinline__ void bcast_out(const bf16x8 (&pf)[C::KC], float inv, const bf16x8* VAf,
                                          rsrc_t ro, int tok0, int tok_end, int d, int sn,
                                          const ModCtx& mc) {
  constexpr int DT = 2 * DC;
  constexpr int VA_PART = C::KC * DT * 64;
  const int lane = threadIdx.x & 63;
  constexpr int kFragRegs = 4 * (KTC * DC + C::KC * DT * C::VSPLIT);
  int fl = lane;
  if (kFragRegs > 128 || KTC >= 16) asm volatile("" : "+v"(fl));
  f32x4 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < C::KC; ++j)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int f = (j * DT + dt) * 64 + fl;
      O[dt] = E::mma(VAf[f], pf[j], O[dt]);
      if (C::VSPLIT > 1)
        O[dt] = E::mma(VAf[VA_PART + f], pf[j], O[dt]);
    }
  store_o_tile<E, DC, MOD>(O, inv, ro, tok0, tok_end, d, sn, mc);
}

// One 16-query tile: S^T = A Q^T over all agents at once, softmax over the
// agents (lane group reductions), O^T = V_A^T P^T.  VAf: [VSPLIT][KC][DT][64].
template <class E, class C, int DC, int KTC, bool MOD>
__device__ __forceinline__ void bcast_tile(const bf16x8 (&qf)[DC], const bf16x8* Af,
                                           const bf16x8* VAf, rsrc_t ro, int tok0, int tok_end,
                                           int d, int sn, int nag, float sl2, const ModCtx& mc) {
  bf16x8 pf[C::KC];
  float inv;
  bcast_probs<E, C, DC, KTC, MOD>(qf, Af, nag, sl2, pf, inv, mc, tok0);
  bcast_out<E, C, DC, KTC, MOD>(pf, inv, VAf, ro, tok0, tok_end, d, sn, mc);
}

// ------------------------------------------------------------- the kernel
// NW waves per workgroup: 8, or 4 for heads held by one workgroup each when
// there are more heads than CUs (two workgroups per CU then, capped at two
// waves per SIMD, so that every head is on the chip at once).
template <int DC, int KTC, bool STRIDED, class E, bool MOD, int NW = kWaves>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
agent_mfma_kernel(MfmaParams p) {
  constexpr int kWaves = NW;             // these shadow the 8-wave defaults
  constexpr int kThreads = 64 * NW;
  using C = Cfg<DC, KTC, NW>;
  constexpr int DT = C::DT;
  constexpr int DPAD = C::DPAD;
  constexpr int RT = C::RT;
  constexpr int ATW = C::ATW;
  constexpr int A_FRAGS = KTC * DC * 64;          // bf16x8 fragments
  constexpr int VA_FRAGS = C::KC * DT * 64;       // per hi / lo part
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16x8* Af = reinterpret_cast<bf16x8*>(smem);
  unsigned char* big = smem + C::A_BYTES;
  bf16_t* Vt = reinterpret_cast<bf16_t*>(big);
  bf16_t* Ks = reinterpret_cast<bf16_t*>(big + C::VT_BYTES);
  float* stage = reinterpret_cast<float*>(big);   // V_A rows [KTC*16][DPAD] (single mode)
  bf16x8* VAf = reinterpret_cast<bf16x8*>(big + (C::STAGE_LDS ? C::STAGE_BYTES : 0));

  // The parameters span four 64-byte lines of the kernel-argument segment.
  // Fetch them into the scalar cache together, so that the parameter reads
  // below hit it instead of each paying a dependent miss.
  {
    static_assert(sizeof(MfmaParams) <= 256, "parameters beyond four lines");
    const auto* ka = __builtin_amdgcn_kernarg_segment_ptr();
    unsigned x0, x1, x2, x3;
    asm volatile(
        "s_load_dword %0, %4, 0x0\n\t"
        "s_load_dword %1, %4, 0x40\n\t"
        "s_load_dword %2, %4, 0x80\n\t"
        "s_load_dword %3, %4, 0xc0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(x0), "=&s"(x1), "=&s"(x2), "=&s"(x3)   // results must not overwrite the address
        : "s"(ka));
    asm volatile("" ::"s"(x0 ^ x1 ^ x2 ^ x3));
  }

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
  AA_STAMP(0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int d = p.d, DCH = d >> 3;
  const int n0 = slot * p.T;
  const int n1 = min(p.N, n0 + p.T);
  // token stride and head offset: dense [B, H, N, d], or the caller's strides
  const int sn = STRIDED ? p.sn : d;
  long hoff = (long)head * p.N * d;
  if (STRIDED) {
    const int hb = idiv(head, p.H, rcp_approx(p.H));   // batch entry of the head
    hoff = (long)hb * p.sb + (long)(head - hb * p.H) * p.sh;
  }
  const unsigned head_bytes = (unsigned)(((long)(p.N - 1) * sn + d) * 2);
  GroupSync gs{p.sync + (long)head * kSyncDwords, slot, p.P, false, p.status, p.spin_limit};
  const bool sync_group = p.fused && p.P > 1;
  const bool single = p.fused && p.P == 1;   // whole head in this workgroup
  const int xp = sync_group ? (p.xcd_heads > 0 ? kXL2 : kXDevice) : kXNone;
  gs.flags = xp == kXL2;
  bool ok = true;
  // groups placed on one XCD rely on workgroup b running on XCD b % 8
  if (xp == kXL2 && tid == 0 && xcc_id() != (int)(blockIdx.x & 7))
    __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(p.status), kFaultXcd, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);

  const rsrc_t rq = rsrc_of(p.q + hoff, head_bytes);
  const rsrc_t rk = rsrc_of(p.k + hoff, head_bytes);
  const rsrc_t rv = rsrc_of(p.v + hoff, head_bytes);
  // module terms: the parameters of head hh of the batch entry
  ModCtx mc{};
  int hh = 0;
  if constexpr (MOD) {
    static_assert(C::TOTAL % 16 == 0, "DWC weights follow the LDS plan, 16-byte aligned");
    hh = head - idiv(head, p.H, rcp_approx(p.H)) * p.H;
    mc.has_b1 = p.bias_agg != nullptr;
    mc.has_b2 = p.bias_bcast != nullptr;
    mc.has_dwc = p.dwc_w != nullptr;
    const unsigned pb = (unsigned)(p.nag * p.N * 4);
    mc.b1 = rsrc_of(p.bias_agg + (mc.has_b1 ? (long)hh * p.nag * p.N : 0), mc.has_b1 ? pb : 0u);
    mc.b2 = rsrc_of(p.bias_bcast + (mc.has_b2 ? (long)hh * p.nag * p.N : 0), mc.has_b2 ? pb : 0u);
    mc.rv = rv;
    mc.wl = reinterpret_cast<const float*>(smem + C::TOTAL);
    mc.inv_scale = p.inv_scale;
    mc.N = p.N;
    mc.nag = p.nag;
    mc.w = p.w;
  }
  const long ahb = (long)head * p.nag * d;    // offset of this head's agent rows
  const unsigned arow_bytes = (unsigned)(p.nag * d * 4);

  // ---- pooling loads first: they start the dependency chain
  const int pool_na = p.nag > slot ? (p.nag - slot + p.P - 1) / p.P : 0;
  const int pool_items = pool_na * DCH * p.pool_tgp;
  const int pool_chunk = p.pool_tgp * kPoolTok;       // window tokens per item pass
  const int pool_npass = (p.pool_maxcnt + pool_chunk - 1) / pool_chunk;
  const int r0cnt = n1 > n0 ? min(RT, n1 - n0) : 0;
  const int r0tiles = ((r0cnt + 31) / 32 * 4) * DCH;   // 8x8 K/V tiles of round 0
  // In a group, when both fit in half the workgroup, the pooling runs on
  // waves 4..7 while waves 0..3 load the first round's keys and values:
  // arrival at barrier 0 then waits only for the pooling waves' agent
  // stores, not for those loads.
  const bool split_kv = sync_group && (p.phases & PH_POOL) && (p.phases & PH_AGG) &&
                        pool_items <= kThreads / 2 && r0tiles <= kThreads / 2;
  const int pool_threads = split_kv ? kThreads / 2 : kThreads;
  const int pt = split_kv ? tid - kThreads / 2 : tid;   // pooling thread (< 0: none)
  uint4 px[kPoolTok];
  if ((p.phases & PH_POOL) && pt >= 0) pool_issue(p, rq, slot, pt, pool_items, 0, px, sn);

  // ---- then K and V of the first round (one 8x8 tile per thread)
  const int ag = wave % C::AG, tg = wave / C::AG;
  uint4 kx[8], vx[8];
  // Without pooling they are issued now; with pooling, once the pooling's
  // query loads have landed, so that they do not delay the pooling and
  // arrive during the pooling, barrier 0 and the agent fragments.
  auto load_kv0 = [&]() {
    const int tend = tid < r0tiles ? n0 + r0cnt : -1;
    load_tile8(kx, rk, tid, n0, tend, d, sn);
    load_tile8(vx, rv, tid, n0, tend, d, sn);
  };
  if ((p.phases & PH_AGG) && !(p.phases & PH_POOL)) load_kv0();
  // first query tile of this wave, loaded ahead of the broadcast
  const int nqt = n1 > n0 ? (n1 - n0 + 15) / 16 : 0;
  bf16x8 qcur[DC];
  // With up to 64 agents, the broadcast probabilities of up to kEarly tiles
  // per wave are computed while the group gathers at barrier 1 (they need
  // only A and Q); only P2 V_A is left after V_A arrives.
  constexpr int kEarly = KTC <= 4 ? 2 : 1;
  bf16x8 epf[kEarly][C::KC];
  bf16x8 qe[kEarly][DC];
  float einv[kEarly];
  bool early = false;
  if ((p.phases & PH_BCAST) && !(p.phases & PH_AGG)) load_q_tile<DC>(qcur, rq, n0 + 16 * wave, n1, d, sn);
  AA_STAMP(1);

  // ---- POOL
  if (p.phases & PH_POOL) {
    float* red = reinterpret_cast<float*>(big);
    if (single) {
      for (int f = tid; f < A_FRAGS; f += kThreads) Af[f] = zero_bf16x8();
    }
    const int TGP = p.pool_tgp;
    const float rdch = rcp_approx(DCH);
    for (int b0 = 0; b0 < pool_items; b0 += pool_threads) {
      float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (pt >= 0) {
        for (int ps = 0; ps < pool_npass; ++ps) {
          if (b0 > 0 || ps > 0)
            pool_issue(p, rq, slot, b0 + pt, pool_items, ps * pool_chunk, px, sn);
          pool_accum<E>(px, acc8);
          if (b0 == 0 && ps == 0 && (p.phases & PH_AGG) && !sync_group) load_kv0();
        }
      }
      __syncthreads();   // red free; the pooling loads of Q have landed
      // the key/value waves of a split load now, behind Q (which starts the
      // dependency chain) and while the pooling waves sum and publish
      if (split_kv && b0 == 0 && pt < 0) load_kv0();
      if (pt >= 0) {
        *reinterpret_cast<float4*>(red + pt * 8) = float4{acc8[0], acc8[1], acc8[2], acc8[3]};
        *reinterpret_cast<float4*>(red + pt * 8 + 4) = float4{acc8[4], acc8[5], acc8[6], acc8[7]};
      }
      __syncthreads();
      // pairs (m, c) of this batch (TGP divides the pooling thread count),
      // summed and stored by pooling threads
      const int pr0 = b0 >> p.pool_tgp_log2;
      const int npr = min(pool_threads, pool_items - b0) >> p.pool_tgp_log2;
      for (int o = pt; o >= 0 && o < npr; o += pool_threads) {
        const int pr = pr0 + o;
        const int m = idiv(pr, DCH, rdch), c = pr - m * DCH;
        const int a = slot + p.P * m;
        float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < TGP; ++t) {
          const float4 lo = *reinterpret_cast<const float4*>(red + (o * TGP + t) * 8);
          const float4 hi = *reinterpret_cast<const float4*>(red + (o * TGP + t) * 8 + 4);
          s8[0] += lo.x; s8[1] += lo.y; s8[2] += lo.z; s8[3] += lo.w;
          s8[4] += hi.x; s8[5] += hi.y; s8[6] += hi.z; s8[7] += hi.w;
        }
        const float inv = 1.0f / (float)pool_geo(p, a).cnt;
#pragma unroll
        for (int e = 0; e < 8; ++e) s8[e] *= inv;
        if (single) {
          // one whole A fragment: agent a, channels 8c..8c+7
          const int t16 = a >> 4, r = a & 15, g = c / DC, cc = c - g * DC;
          union { bf16x8 v; unsigned u[4]; } fr;
#pragma unroll
          for (int e = 0; e < 4; ++e) fr.u[e] = pack2<E>(s8[2 * e], s8[2 * e + 1]);
          Af[(t16 * DC + cc) * 64 + 16 * g + r] = fr.v;
        } else if (sync_group) {
          // the group exchanges A as bf16 MFMA fragments: one 16-byte
          // fragment per (agent, 8-channel chunk)
          const int t16 = a >> 4, r = a & 15, g = c / DC, cc = c - g * DC;
          union { uint4 v; unsigned u[4]; } fr;
#pragma unroll
          for (int e = 0; e < 4; ++e) fr.u[e] = pack2<E>(s8[2 * e], s8[2 * e + 1]);
          const rsrc_t rf = rsrc_of(reinterpret_cast<char*>(p.agents_f32) + head * C::A_BYTES,
                                    C::A_BYTES);
          const unsigned off = (unsigned)(((t16 * DC + cc) * 64 + 16 * g + r) * 16);
          if (xp == kXL2 && !C::ROW_PARTIALS) bst16<kL2 | kStream>(rf, off, fr.v);   // see partials
          else xst16(xp, rf, off, fr.v);
        } else {
          const rsrc_t ra = rsrc_of(p.agents_f32 + ahb, arow_bytes);
          const unsigned off = (unsigned)((a * d + 8 * c) * 4);
          const uint4 lo = f4_bits(float4{s8[0], s8[1], s8[2], s8[3]});
          const uint4 hi = f4_bits(float4{s8[4], s8[5], s8[6], s8[7]});
          xst16(xp, ra, off, lo);
          xst16(xp, ra, off + 16, hi);
        }
      }
    }
    if (pool_items == 0 && (p.phases & PH_AGG) && (!sync_group || (split_kv && pt < 0)))
      load_kv0();   // no agents to pool here: the loop above did not load them
    AA_STAMP(2);
    if (sync_group) {
      // the key/value waves of a split have nothing to publish: they skip
      // arrival's wait for their memory operations
      group_arrive(gs, 0, !(split_kv && pt < 0));
      // Without the split, the first round's keys and values are loaded
      // only now (arrival waits for every load in flight of its wave, so
      // loads issued during the pooling would hold it back until they
      // land); they travel while the group gathers.  The last wave, which
      // has none of them, polls.
      if (!split_kv && (p.phases & PH_AGG) && wave * 64 < r0tiles) load_kv0();
      ok = group_wait(gs, 0, kWaves - 1);
    }
    AA_STAMP(3);
  }

  // ---- agents -> LDS fragments (zero for padding agents and channels)
  if (sync_group && !p.agents_in && (p.phases & PH_POOL)) {
    // fragments exchanged by the pooling workgroups (padding ones read zero)
    const rsrc_t rf = rsrc_of(reinterpret_cast<char*>(p.agents_f32) + head * C::A_BYTES, C::A_BYTES);
#pragma unroll
    for (int f0 = 0; f0 < A_FRAGS; f0 += kThreads) {
      const int f = f0 + tid;
      const int fl = f & 63, c = (f >> 6) % DC, t = (f >> 6) / DC;
      const int agent = 16 * t + (fl & 15), ch0 = 8 * (DC * (fl >> 4) + c);
      const bool in = f < A_FRAGS && agent < p.nag && ch0 < d;
      const uint4 x = bld16<kCoherent>(rf, in ? (unsigned)(f * 16) : kOOB);
      if (f < A_FRAGS) Af[f] = __builtin_bit_cast(bf16x8, x);
    }
  } else if ((p.phases & (PH_AGG | PH_BCAST)) && !(single && (p.phases & PH_POOL))) {
    const bool from_rows = !p.agents_in;
    const float* rows = p.agents_f32_in ? p.agents_f32_in : p.agents_f32;
    const rsrc_t ra = from_rows ? rsrc_of(rows + ahb, arow_bytes)
                                : rsrc_of(p.agents_in + ahb, (unsigned)(p.nag * d * 2));
    with_pol(xp, [&](auto pc) {
    constexpr int POL = decltype(pc)::value;
#pragma unroll
    for (int f0 = 0; f0 < A_FRAGS; f0 += kThreads) {
      const int f = f0 + tid;
      const int fl = f & 63, c = (f >> 6) % DC, t = (f >> 6) / DC;
      const int agent = 16 * t + (fl & 15), ch0 = 8 * (DC * (fl >> 4) + c);
      const bool in = f < A_FRAGS && agent < p.nag && ch0 < d;
      if (from_rows) {
        const unsigned off = in ? (unsigned)((agent * d + ch0) * 4) : kOOB;
        uint4 x0, x1;
        x0 = bld16<POL>(ra, off);
        x1 = bld16<POL>(ra, off + 16);
        const float4 a0 = bits_f4(x0), a1 = bits_f4(x1);
        union { bf16x8 v; unsigned w[4]; } fr;
        fr.w[0] = pack2<E>(a0.x, a0.y);
        fr.w[1] = pack2<E>(a0.z, a0.w);
        fr.w[2] = pack2<E>(a1.x, a1.y);
        fr.w[3] = pack2<E>(a1.z, a1.w);
        if (f < A_FRAGS) Af[f] = fr.v;
      } else {
        const uint4 x = bld16<kPlain>(ra, in ? (unsigned)((agent * d + ch0) * 2) : kOOB);
        if (f < A_FRAGS) Af[f] = __builtin_bit_cast(bf16x8, x);
      }
    }
    });
  }
  __syncthreads();
  AA_STAMP(4);

  // ---- AGGREGATE
  if (p.phases & PH_AGG) {
    AggState<DC, ATW> st;
#pragma unroll
    for (int a = 0; a < ATW; ++a) {
      st.m[a] = -INFINITY;
      st.thr[a] = -INFINITY;
      st.l[a] = 0.f;
      st.lacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.acc[a][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int rt0 = n0; rt0 < n1; rt0 += RT) {
      const int rcnt = min(RT, n1 - rt0);
      const int rblk = (rcnt + 31) / 32;
      const int ntile = rblk * 4 * DCH;
      __syncthreads();   // previous round (or the pooling sums) fully read
      if (tid < ntile) {
        store_tile_rows(Ks, C::KS_STRIDE, kx, tid, d);
        store_tile_t(Vt, C::VT_STRIDE, vx, tid, d);
      }
      // the next round's tiles travel while this round is aggregated
      if (rt0 + RT < n1) {
        const int ncnt = min(RT, n1 - rt0 - RT);
        const int ntn = (ncnt + 31) / 32 * 4 * DCH;
        if (wave * 64 < ntn) {
          const int tend = tid < ntn ? rt0 + RT + ncnt : -1;
          load_tile8(kx, rk, tid, rt0 + RT, tend, d, sn);
          load_tile8(vx, rv, tid, rt0 + RT, tend, d, sn);
        }
      }
      // below the padded head dim, the key columns [d, DPAD) that the score
      // products read are cleared (the LDS holds other phases' data)
      const int npad = DPAD / 8 - DCH;
      for (int i = tid; i < rblk * 32 * npad; i += kThreads) {
        const int row = idiv(i, npad, rcp_approx(npad));
        *reinterpret_cast<uint4*>(Ks + row * C::KS_STRIDE + 8 * (DCH + i - row * npad)) =
            uint4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
      AA_STAMP(12);
      // agent biases of this wave's blocks, loaded one block ahead
      float4 b1c[ATW][2], b1n[ATW][2];
      if constexpr (MOD) {
        if (mc.has_b1 && tg < rblk)
#pragma unroll
          for (int a = 0; a < ATW; ++a) load_b1(mc, ATW * ag + a, rt0 + 32 * tg, b1c[a]);
      }
      for (int b = tg; b < rblk; b += C::TG) {
        if constexpr (MOD) {
          if (mc.has_b1 && b + C::TG < rblk)
#pragma unroll
            for (int a = 0; a < ATW; ++a) load_b1(mc, ATW * ag + a, rt0 + 32 * (b + C::TG), b1n[a]);
        }
        agg_block<E, C, DC, ATW, MOD>(st, Ks, Af, Vt, 32 * b, ag, min(32, n1 - (rt0 + 32 * b)),
                                      p.sl2, mc, b1c);
        if constexpr (MOD) {
#pragma unroll
          for (int a = 0; a < ATW; ++a) {
            b1c[a][0] = b1n[a][0];
            b1c[a][1] = b1n[a][1];
          }
        }
#ifdef AGENT_ATTN_PHASE_TRACE
        if (b / C::TG < 4) {
          __builtin_amdgcn_s_waitcnt(0);
          AA_STAMP_BY(18 + b / C::TG, 0);
          AA_STAMP_BY(22 + b / C::TG, 64 * (kWaves - 1));
          if (p.trace && threadIdx.x == 0 && (b == 0 || b / C::TG == 3))
            p.trace[(long)blockIdx.x * 32 + (b == 0 ? 28 : 29)] = (long long)clock64();
        }
#endif
      }
    }
    AA_STAMP(5);
    if (single && (p.phases & PH_BCAST)) load_q_tile<DC>(qcur, rq, n0 + 16 * wave, n1, d, sn);
#pragma unroll
    for (int a = 0; a < ATW; ++a) st.l[a] = st.lacc[a][0];

    // combine the TG token groups of each agent group through LDS:
    // records [rec][a][DT acc | 1 (m, l)][64 lanes] x 16 B
    if (C::TG > 1) {
      float4* comb = reinterpret_cast<float4*>(big);
      constexpr int RQ = DT + 1;
      __syncthreads();
      if (tg > 0) {
        float4* dst = comb + ((tg - 1) * C::AG + ag) * ATW * RQ * 64;
#pragma unroll
        for (int a = 0; a < ATW; ++a) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            dst[(a * RQ + dt) * 64 + lane] =
                float4{st.acc[a][dt][0], st.acc[a][dt][1], st.acc[a][dt][2], st.acc[a][dt][3]};
          dst[(a * RQ + DT) * 64 + lane] = float4{st.m[a], st.l[a], 0.f, 0.f};
        }
      }
      __syncthreads();
      if (tg == 0) {
        for (int o = 1; o < C::TG; ++o) {
          const float4* src = comb + ((o - 1) * C::AG + ag) * ATW * RQ * 64;
#pragma unroll
          for (int a = 0; a < ATW; ++a) {
            const float4 ml = src[(a * RQ + DT) * 64 + lane];
            const float mn = fmaxf(st.m[a], ml.x);
            const float c1 = (mn == -INFINITY) ? 0.f : fast_exp2((st.m[a] - mn) * p.sl2);
            const float c2 = (mn == -INFINITY) ? 0.f : fast_exp2((ml.x - mn) * p.sl2);
            st.l[a] = st.l[a] * c1 + ml.y * c2;
            st.m[a] = mn;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const float4 rr = src[(a * RQ + dt) * 64 + lane];
              st.acc[a][dt][0] = st.acc[a][dt][0] * c1 + rr.x * c2;
              st.acc[a][dt][1] = st.acc[a][dt][1] * c1 + rr.y * c2;
              st.acc[a][dt][2] = st.acc[a][dt][2] * c1 + rr.z * c2;
              st.acc[a][dt][3] = st.acc[a][dt][3] * c1 + rr.w * c2;
            }
          }
        }
      }
    }
    AA_STAMP(26);
    // wave (ag, 0) now holds the workgroup's partial for its agent tiles
    const int g = lane >> 4;
    if (p.P == 1) {
      // V_A rows: staging (LDS or the fp32 scratch) in single mode, the fp32
      // output otherwise
      const bool lds_rows = single && C::STAGE_LDS;
      __syncthreads();   // comb fully read (it aliases the staging rows)
      if (tg == 0) {
        const rsrc_t rvo = rsrc_of(p.values_f32 + ahb, arow_bytes);
#pragma unroll
        for (int a = 0; a < ATW; ++a) {
          const int agent = 16 * (ATW * ag + a) + (lane & 15);
          const float inv = 1.0f / st.l[a];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int ch = 16 * dt + 4 * g;
            const float4 x = float4{st.acc[a][dt][0] * inv, st.acc[a][dt][1] * inv,
                                    st.acc[a][dt][2] * inv, st.acc[a][dt][3] * inv};
            if (lds_rows) {
              *reinterpret_cast<float4*>(stage + agent * DPAD + ch) = x;
            } else {
              const unsigned off = (agent < p.nag && ch < d) ? (unsigned)((agent * d + ch) * 4) : kOOB;
              bst16<kPlain>(rvo, off, f4_bits(x));
            }
          }
        }
      }
    } else if (tg == 0) {
      // partials: agent rows of DPAD channels (the merge reads whole rows),
      // bf16 from 128 agents, fp32 below
      const long pbase = ((long)head * p.P + slot) * KTC;
      const rsrc_t racc = rsrc_of(p.part_acc + pbase * DT * 256, (unsigned)(KTC * DT * 1024));
      const rsrc_t rml = rsrc_of(p.part_ml + pbase * 32, (unsigned)(KTC * 128));
#pragma unroll
      for (int a = 0; a < ATW; ++a) {
        const int t = ATW * ag + a;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // rows of padding agents are never merged: not stored
          const bool real = 16 * t + (lane & 15) < p.nag;
          if (C::ROW_PARTIALS) {
            // bf16 agent rows: V_A itself enters the broadcast as bf16 here
            // (VSPLIT = 1), and rounding the partials adds no measurable
            // error, while it halves the partial traffic
            const unsigned off =
                real ? (unsigned)(((16 * t + (lane & 15)) * DPAD + 16 * dt + 4 * g) * 2) : kOOB;
            xst8(xp, racc, off, uint2{pack_bf16(st.acc[a][dt][0], st.acc[a][dt][1]),
                                      pack_bf16(st.acc[a][dt][2], st.acc[a][dt][3])});
          } else {
            // fp32 agent rows: quad 4 dt + g of agent 16 t + r
            const unsigned off =
                real ? (unsigned)(((16 * t + (lane & 15)) * 4 * DT + 4 * dt + g) * 16) : kOOB;
            const uint4 x = f4_bits(float4{st.acc[a][dt][0], st.acc[a][dt][1], st.acc[a][dt][2],
                                           st.acc[a][dt][3]});
            // small partial sets (up to 64 agents) are streamed (nt), so the
            // L2 writes them back during the kernel rather than at its end;
            // large ones stay cached for the merge
            if (xp == kXL2) bst16<kL2 | kStream>(racc, off, x);
            else xst16(xp, racc, off, x);
          }
        }
        const unsigned moff = (g == 0 && 16 * t + (lane & 15) < p.nag)
                                  ? (unsigned)((t * 16 + (lane & 15)) * 8) : kOOB;
        const uint2 ml = uint2{__float_as_uint(st.m[a]), __float_as_uint(st.l[a])};
        xst8(xp, rml, moff, ml);
      }
    }
    AA_STAMP(6);
    if (sync_group && ok) {
      group_arrive(gs, 1);
      early = KTC <= 4 && (p.phases & PH_BCAST) && (p.phases & PH_MERGE) &&
              nqt <= kEarly * kWaves;
      if (early) {
        // query tiles of the early probabilities (computed during the merge)
#pragma unroll
        for (int i = 0; i < kEarly; ++i)
          load_q_tile<DC>(qe[i], rq, n0 + 16 * (wave + kWaves * i), n1, d, sn);
      } else if (p.phases & PH_BCAST) {
        // the query tile loads travel while the group gathers
        load_q_tile<DC>(qcur, rq, n0 + 16 * wave, n1, d, sn);
      }
      ok = group_wait(gs, 1);
    } else if (sync_group && (p.phases & PH_BCAST)) {
      load_q_tile<DC>(qcur, rq, n0 + 16 * wave, n1, d, sn);
    }
    AA_STAMP(7);
  }

  // ---- MERGE: items (agent a = slot + P*m, channel quad q) over the threads
  if ((p.phases & PH_MERGE) && p.P > 1 && ok) {
    constexpr int nq = DPAD / 4;
    const int items = pool_na * nq;   // agents slot, slot+P, ... (pool_na of them)
    const long hbase = (long)head * p.P * KTC;
    const rsrc_t racc = rsrc_of(p.part_acc + hbase * DT * 256, (unsigned)(p.P * KTC * DT * 1024));
    const rsrc_t rml = rsrc_of(p.part_ml + hbase * 32, (unsigned)(p.P * KTC * 128));
    const rsrc_t rvo = rsrc_of(p.values_f32 + ahb, arow_bytes);
    // Waves without merge items compute their broadcast probabilities now;
    // the merging waves do so between arriving at barrier 2 and waiting.
    // merge items run on the last waves, which hold the fewest query tiles
    // From 128 agents (where groups have up to 32 slots), two adjacent lanes
    // share an item (even and odd slots) and combine their partial merges
    // with one lane exchange, which halves the chain of dependent loads.
    constexpr int nsplit = C::ROW_PARTIALS ? 2 : 1;
    const int units = items * nsplit;
    const int mtid = kThreads - 1 - tid;
    const bool merge_wave = (kWaves - 1 - wave) * 64 < units;
    auto early_probs = [&]() {
#pragma unroll
      for (int i = 0; i < kEarly; ++i)
        if (wave + kWaves * i < nqt)
          bcast_probs<E, C, DC, KTC, MOD>(qe[i], Af, p.nag, p.sl2, epf[i], einv[i], mc,
                                          n0 + 16 * (wave + kWaves * i));
    };
    if (early && !merge_wave) early_probs();
    AA_STAMP_BY(15, 0);
    with_pol(xp, [&](auto pc) {
    constexpr int POL = decltype(pc)::value;
    for (int un = mtid; un < units; un += kThreads) {
      const int it = un / nsplit, part = un - it * nsplit;
      const int m = it / nq, q = it - m * nq;
      const int a = slot + p.P * m;
      const int t = a >> 4, r = a & 15, dt = q >> 2, g = q & 3;
      const unsigned aoff = C::ROW_PARTIALS ? (unsigned)((a * DPAD + 4 * q) * 2)
                                            : (unsigned)((a * nq + q) * 16);
      const unsigned moff = (unsigned)((t * 16 + r) * 8);
      constexpr unsigned sstride_acc = KTC * DT * 1024, sstride_ml = KTC * 128;
      float M = -INFINITY, Ls = 0.f;
      float4 acc = float4{0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < p.P; s0 += 16 * nsplit) {
        uint4 xa[16];
        u32x2 xm[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int sl = s0 + nsplit * u + part;   // this lane's slot
          const bool in = sl < p.P;
          const unsigned so = (unsigned)sl;
          if (C::ROW_PARTIALS) {
            const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(
                racc, (int)(in ? aoff + so * sstride_acc : kOOB), 0, POL);
            xa[u] = uint4{h[0], h[1], 0u, 0u};
          } else {
            xa[u] = bld16<POL>(racc, in ? aoff + so * sstride_acc : kOOB);
          }
          xm[u] = __builtin_amdgcn_raw_buffer_load_b64(
              rml, (int)(in ? moff + so * sstride_ml : kOOB), 0, POL);
        }
        float cm = M;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (s0 + nsplit * u + part < p.P) cm = fmaxf(cm, __uint_as_float(xm[u][0]));
        const float corr = (cm == -INFINITY) ? 0.f : fast_exp2((M - cm) * p.sl2);
        Ls *= corr;
        acc.x *= corr; acc.y *= corr; acc.z *= corr; acc.w *= corr;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (s0 + nsplit * u + part >= p.P) continue;
          const float mu = __uint_as_float(xm[u][0]);
          const float wgt = (mu == -INFINITY) ? 0.f : fast_exp2((mu - cm) * p.sl2);
          const float4 av = C::ROW_PARTIALS
                                ? float4{bf16_value((bf16_t)(xa[u].x & 0xffffu)),
                                         bf16_value((bf16_t)(xa[u].x >> 16)),
                                         bf16_value((bf16_t)(xa[u].y & 0xffffu)),
                                         bf16_value((bf16_t)(xa[u].y >> 16))}
                                : bits_f4(xa[u]);
          Ls = fmaf(__uint_as_float(xm[u][1]), wgt, Ls);
          acc.x = fmaf(av.x, wgt, acc.x);
          acc.y = fmaf(av.y, wgt, acc.y);
          acc.z = fmaf(av.z, wgt, acc.z);
          acc.w = fmaf(av.w, wgt, acc.w);
        }
        M = cm;
      }
      if constexpr (nsplit > 1) {   // both lanes of a pair are active (units come in pairs)
        const float Mo = __shfl_xor(M, 1), Lo = __shfl_xor(Ls, 1);
        const float ax = __shfl_xor(acc.x, 1), ay = __shfl_xor(acc.y, 1);
        const float az = __shfl_xor(acc.z, 1), aw = __shfl_xor(acc.w, 1);
        const float Mn = fmaxf(M, Mo);
        const float w0 = (M == -INFINITY) ? 0.f : fast_exp2((M - Mn) * p.sl2);
        const float w1 = (Mo == -INFINITY) ? 0.f : fast_exp2((Mo - Mn) * p.sl2);
        Ls = Ls * w0 + Lo * w1;
        acc = float4{acc.x * w0 + ax * w1, acc.y * w0 + ay * w1, acc.z * w0 + az * w1,
                     acc.w * w0 + aw * w1};
      }
      const float inv = 1.0f / Ls;
      const int ch = 16 * dt + 4 * g;
      if (sync_group) {
        // V_A goes to the group as bf16 fragments (hi, and lo when VSPLIT
        // = 2) at the positions bcast_out reads: agent a is element e of
        // lane group gg in chunk j, channel ch+i is lane row (ch+i) % 16
        const float v4[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
        const rsrc_t rvf = rsrc_of(reinterpret_cast<char*>(p.values_f32) + head * C::VA_BYTES,
                                   C::VA_BYTES);
        const int u = a & 31, j = a >> 5;
        const int gg = (u & 15) >> 2, e = (u & 3) + (u >= 16 ? 4 : 0);
        const bool keep = part == 0 && a < p.nag && ch < d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ch + i;
          const int f = (j * DT + (c >> 4)) * 64 + 16 * gg + (c & 15);
          const bf16_t hi = E::bits(v4[i]);
          const unsigned off = keep ? (unsigned)((f * 8 + e) * 2) : kOOB;
          if (xp == kXL2 && !C::ROW_PARTIALS)   // streamed like the partials
            __builtin_amdgcn_raw_buffer_store_b16(hi, rvf, (int)off, 0, kL2 | kStream);
          else if (xp == kXL2) __builtin_amdgcn_raw_buffer_store_b16(hi, rvf, (int)off, 0, kL2);
          else __builtin_amdgcn_raw_buffer_store_b16(hi, rvf, (int)off, 0, kCoherent);
          if (C::VSPLIT > 1) {
            const bf16_t lo = E::bits(v4[i] - E::value(hi));
            const unsigned offl = keep ? (unsigned)(((VA_FRAGS + f) * 8 + e) * 2) : kOOB;
            if (xp == kXL2 && !C::ROW_PARTIALS)
              __builtin_amdgcn_raw_buffer_store_b16(lo, rvf, (int)offl, 0, kL2 | kStream);
            else if (xp == kXL2) __builtin_amdgcn_raw_buffer_store_b16(lo, rvf, (int)offl, 0, kL2);
            else __builtin_amdgcn_raw_buffer_store_b16(lo, rvf, (int)offl, 0, kCoherent);
          }
        }
      } else {
        const unsigned off =
            (part == 0 && a < p.nag && ch < d) ? (unsigned)((a * d + ch) * 4) : kOOB;
        const uint4 x = f4_bits(float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv});
        bst16<POL>(rvo, off, x);
      }
    }
    });
    AA_STAMP_BY(14, kThreads - 1);
    AA_STAMP(8);
    if (sync_group && ok) {
      group_arrive(gs, 2);
      if (early && merge_wave) early_probs();
      ok = group_wait(gs, 2);
    } else if (early && merge_wave) {
      early_probs();
    }
    AA_STAMP(9);
  }

  // ---- BROADCAST
  if ((p.phases & PH_BCAST) && ok) {
    // V_A fragments from rows: LDS staging (single mode), the exchanged rows
    // (groups) or the fp32 input (step call); padding positions are zero
    const bool lds_rows = single && C::STAGE_LDS && (p.phases & PH_AGG);
    const float* rows = p.values_f32_in ? p.values_f32_in : p.values_f32;
    const rsrc_t rvr = rsrc_of(rows + ahb, arow_bytes);
    __syncthreads();
    if (sync_group && (p.phases & PH_MERGE)) {
      // fragments written by the merging workgroups; elements of padding
      // agents were never written and are cleared here
      const rsrc_t rvf = rsrc_of(reinterpret_cast<char*>(p.values_f32) + head * C::VA_BYTES,
                                 C::VA_BYTES);
#pragma unroll
      for (int f0 = 0; f0 < VA_FRAGS * C::VSPLIT; f0 += kThreads) {
        const int f = f0 + tid;
        const int fh = f % VA_FRAGS;
        const int fl = fh & 63, dt = (fh >> 6) % DT, j = (fh >> 6) / DT;
        const int ch = 16 * dt + (fl & 15), g = fl >> 4;
        const bool in = f < VA_FRAGS * C::VSPLIT && ch < d;
        union { uint4 v; unsigned w[4]; } x;
        x.v = bld16<kCoherent>(rvf, in ? (unsigned)(f * 16) : kOOB);
        if (32 * j + 32 > p.nag) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (pair_index(j, g, e) >= p.nag) x.w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
        if (f < VA_FRAGS * C::VSPLIT) VAf[f] = __builtin_bit_cast(bf16x8, x.v);
      }
    } else {
    with_pol(xp, [&](auto pc) {
    constexpr int POL = decltype(pc)::value;
#pragma unroll
    for (int f0 = 0; f0 < VA_FRAGS; f0 += kThreads) {
      const int f = f0 + tid;
      const int fl = f & 63, dt = (f >> 6) % DT, j = (f >> 6) / DT;
      const int ch = 16 * dt + (fl & 15), g = fl >> 4;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int agent = pair_index(j, g, e);
        const bool in = f < VA_FRAGS && agent < p.nag && ch < d;
        if (lds_rows) {
          x[e] = in ? stage[agent * DPAD + ch] : 0.f;
        } else {
          const unsigned off = in ? (unsigned)((agent * d + ch) * 4) : kOOB;
          x[e] = bld4<POL>(rvr, off);
        }
      }
      union { bf16x8 v; bf16_t e[8]; } hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi.e[e] = E::bits(x[e]);
        lo.e[e] = E::bits(x[e] - E::value(hi.e[e]));
      }
      if (f < VA_FRAGS) {
        VAf[f] = hi.v;
        if (C::VSPLIT > 1) VAf[VA_FRAGS + f] = lo.v;
      }
    }
    });
    }
    if constexpr (MOD) {
      if (mc.has_dwc) {
        // DWC weights of the head's channels as [9 taps][DPAD], then the
        // bias [DPAD]; channels at or past d hold zeros
        float* wl = reinterpret_cast<float*>(smem + C::TOTAL);
        for (int i = tid; i < 10 * DPAD; i += kThreads) {
          const int tap = i / DPAD, c = i - tap * DPAD;
          const long ch = (long)hh * d + c;
          float x = 0.f;
          if (c < d) x = tap < 9 ? p.dwc_w[ch * 9 + tap] : (p.dwc_b ? p.dwc_b[ch] : 0.f);
          wl[i] = x;
        }
        if (p.dwc_halo_rows > 0) {
          // V rows of this workgroup's tokens and one grid row plus one
          // token on either side (every 3 x 3 tap of its tokens), 16-byte
          // pieces, four loads in flight per thread; channels at or past d
          // read zero
          constexpr int CPR = DPAD / 8, HS = dwc_halo_stride<DC>();
          const int hr0 = max(0, n0 - p.w - 1), hr1 = min(p.N, n1 + p.w + 1);
          const int nck = max(0, hr1 - hr0) * CPR;
          bf16_t* hv = reinterpret_cast<bf16_t*>(
              p.dwc_halo_in_plan ? big + (C::STAGE_LDS ? C::STAGE_BYTES : 0) + C::VA_BYTES
                                 : smem + C::TOTAL + dwc_lds_bytes<DC>());
          for (int c0 = 0; c0 < nck; c0 += 4 * kThreads) {
            uint4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int idx = c0 + u * kThreads + tid;
              const int r = idx / CPR, c = idx - r * CPR;
              const bool in = idx < nck && 8 * c < d;
              x[u] = bld16<kPlain>(mc.rv, in ? (unsigned)(((hr0 + r) * sn + 8 * c) * 2) : kOOB);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int idx = c0 + u * kThreads + tid;
              const int r = idx / CPR, c = idx - r * CPR;
              if (idx < nck) *reinterpret_cast<uint4*>(hv + r * HS + 8 * c) = x[u];
            }
          }
          mc.hv = hv;
          mc.hr0 = hr0;
          mc.hrows = max(0, hr1 - hr0);
        }
      }
    }
    __syncthreads();
    AA_STAMP(10);
    const rsrc_t ro = rsrc_of(p.out + hoff, head_bytes);
    if (early) {
#pragma unroll
      for (int i = 0; i < kEarly; ++i) {
        const int qt = wave + kWaves * i;
        if (qt < nqt)
          bcast_out<E, C, DC, KTC, MOD>(epf[i], einv[i], VAf, ro, n0 + 16 * qt, n1, d, sn, mc);
      }
    } else
    for (int qt = wave; qt < nqt; qt += kWaves) {
      bf16x8 qnext[DC];
      load_q_tile<DC>(qnext, rq, n0 + 16 * (qt + kWaves), n1, d, sn);   // zeros past the end
      bcast_tile<E, C, DC, KTC, MOD>(qcur, Af, VAf, ro, n0 + 16 * qt, n1, d, sn, p.nag, p.sl2, mc);
#pragma unroll
      for (int c = 0; c < DC; ++c) qcur[c] = qnext[c];
    }
  }
  AA_STAMP(11);

  // ---- the last workgroup of the group clears the barrier state
  if (sync_group) group_finish(gs);
#ifdef AGENT_ATTN_PHASE_TRACE
  __builtin_amdgcn_s_waitcnt(0);
  AA_STAMP(13);
#endif
}

// Launch helper, instantiated per (DC, element type) in its own translation
// unit (mfma_dc<DC>_<type>.hip) so that the instances compile in parallel.
template <int DC, class E>
int launch_mfma_dc(const MfmaParams& mp, int ktc, int variant, long grid, hipStream_t st);

template <int DC, int KTC, bool STRIDED, class E, bool MOD, int NW = kWaves>
int launch_mfma_one(const MfmaParams& mp, long grid, hipStream_t st) {
  const unsigned lds =
      (unsigned)(Cfg<DC, KTC, NW>::TOTAL + (MOD ? dwc_lds_bytes<DC>() : 0) +
                 (MOD && !mp.dwc_halo_in_plan ? dwc_halo_lds_bytes<DC>(mp.dwc_halo_rows) : 0));
  agent_mfma_kernel<DC, KTC, STRIDED, E, MOD, NW>
      <<<dim3((unsigned)grid), dim3(64 * NW), lds, st>>>(mp);
  return (int)hipGetLastError();
}

// Kernel variants: the dense layout, caller strides, the dense layout with
// the module terms (agent biases, depth-wise convolution), and the dense
// layout without and with the module terms in four-wave workgroups (one head
// each, more heads than CUs; up to 64 agents).
enum Variant { kDense = 0, kStrided = 1, kModule = 2, kDense4 = 3, kModule4 = 4 };

template <int DC, int KTC, class E>
int launch_mfma_variant(const MfmaParams& mp, int variant, long grid, hipStream_t st) {
  switch (variant) {
    case kStrided: return launch_mfma_one<DC, KTC, true, E, false>(mp, grid, st);
    case kModule: return launch_mfma_one<DC, KTC, false, E, true>(mp, grid, st);
    case kDense4:
      if constexpr (KTC == 4) return launch_mfma_one<DC, KTC, false, E, false, 4>(mp, grid, st);
      return (int)hipErrorInvalidValue;
    case kModule4:
      if constexpr (KTC == 4) return launch_mfma_one<DC, KTC, false, E, true, 4>(mp, grid, st);
      return (int)hipErrorInvalidValue;
    default: return launch_mfma_one<DC, KTC, false, E, false>(mp, grid, st);
  }
}

// Agent tiles of 16: KTC = 4 (<= 64 agents), 8 (<= 128), 16 (<= 256).
template <int DC, class E>
int launch_mfma_switch(const MfmaParams& mp, int ktc, int variant, long grid, hipStream_t st) {
  switch (ktc) {
    case 4: return launch_mfma_variant<DC, 4, E>(mp, variant, grid, st);
    case 8: return launch_mfma_variant<DC, 8, E>(mp, variant, grid, st);
    default: return launch_mfma_variant<DC, 16, E>(mp, variant, grid, st);
  }
}

template <int DC, int KTC>
int mfma_lds_bytes_t() { return Cfg<DC, KTC>::TOTAL; }

}  // namespace aa
