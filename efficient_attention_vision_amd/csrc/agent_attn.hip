// Host side of the Agent Attention C ABI (include/agent_attn.h): argument
// validation, workspace layout, kernel selection and launches on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "agent_attn.h"
#include "common.hpp"
#include "kernels_mfma.hpp"
#include "kernels_scalar.hpp"
#include "kernels_backward.hpp"
#include "kernels_gemm.hpp"
#include "kernels_gemm_mfma.hpp"
#include "kernels_bwd_mfma.hpp"
#include "kernels_proj.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(AGENT_ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int elem_size(int dtype) { return dtype == AGENT_ATTN_F32 ? 4 : 2; }

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

bool misaligned(const void* p) { return p && ((uintptr_t)p & 15u) != 0; }

// Sizes shared by every entry point.
struct Dims {
  long B = 0, H = 0, BH = 0;
  long N = 0;
  int h = 0, w = 0, d = 0, s = 0, nag = 0, dtype = 0;
  long sb = 0, sh = 0, sn = 0;   // element strides of q/k/v/out (contiguous by default)
  aa::Strides strides() const { return aa::Strides{sb, sh, sn, (int)(H > 0 ? H : 1)}; }
  // elements from the first to one past the last element of a tensor
  long span() const { return BH == 0 ? 0 : (B - 1) * sb + (H - 1) * sh + (N - 1) * sn + d; }
};

int check_dtype(int dtype) {
  if (dtype != AGENT_ATTN_F32 && dtype != AGENT_ATTN_BF16 && dtype != AGENT_ATTN_F16)
    return fail(AGENT_ATTN_ERR_DTYPE,
                "dtype %d is not AGENT_ATTN_F32, AGENT_ATTN_BF16 or AGENT_ATTN_F16", dtype);
  return AGENT_ATTN_OK;
}

// Validates B, H, N, d, n_agents, dtype (not the grid).
int check_core(Dims& D, int B, int H, long N, int d, int nag, int dtype) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (B < 0 || H < 0) return fail(AGENT_ATTN_ERR_SHAPE, "B=%d and H=%d must be >= 0", B, H);
  if (N < 1) return fail(AGENT_ATTN_ERR_SHAPE, "token count N=%ld must be >= 1", N);
  if (d < 1) return fail(AGENT_ATTN_ERR_SHAPE, "head dim d=%d must be >= 1", d);
  if (nag < 1) return fail(AGENT_ATTN_ERR_SHAPE, "agent count %d must be >= 1", nag);
  if (d % 8 != 0 || d > AGENT_ATTN_MAX_HEAD_DIM)
    return fail(AGENT_ATTN_ERR_UNSUPPORTED, "head dim d=%d: need d %% 8 == 0 and d <= %d", d,
                AGENT_ATTN_MAX_HEAD_DIM);
  if (nag > AGENT_ATTN_MAX_AGENTS)
    return fail(AGENT_ATTN_ERR_UNSUPPORTED, "%d agents exceed the limit of %d", nag,
                AGENT_ATTN_MAX_AGENTS);
  const long BH = (long)B * H;
  if (BH >= (1L << 23))
    return fail(AGENT_ATTN_ERR_SHAPE, "B*H=%ld must be below 2^23", BH);
  if (BH * N * d >= (1L << 40))
    return fail(AGENT_ATTN_ERR_SHAPE, "B*H*N*d=%ld elements exceed 2^40", BH * N * d);
  D.B = B;
  D.H = H;
  D.BH = BH;
  D.N = N;
  D.d = d;
  D.nag = nag;
  D.dtype = dtype;
  D.sn = d;
  D.sh = N * d;
  D.sb = (long)H * N * d;
  return AGENT_ATTN_OK;
}

int check_grid(Dims& D, int B, int H, int h, int w, int d, int s, int dtype) {
  if (h < 1 || w < 1) return fail(AGENT_ATTN_ERR_SHAPE, "grid %dx%d must be at least 1x1", h, w);
  if (h > 32768 || w > 32768)
    return fail(AGENT_ATTN_ERR_SHAPE, "grid %dx%d: each side must be <= 32768", h, w);
  if (s < 1 || s > h || s > w)
    return fail(AGENT_ATTN_ERR_SHAPE, "agent grid side s=%d must satisfy 1 <= s <= min(h=%d, w=%d)",
                s, h, w);
  if (s * s > AGENT_ATTN_MAX_AGENTS)
    return fail(AGENT_ATTN_ERR_UNSUPPORTED, "s*s=%d agents exceed the limit of %d", s * s,
                AGENT_ATTN_MAX_AGENTS);
  int st = check_core(D, B, H, (long)h * w, d, s * s, dtype);
  if (st) return st;
  D.h = h;
  D.w = w;
  D.s = s;
  return AGENT_ATTN_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(AGENT_ATTN_ERR_SCALE, "scale %g must be finite and > 0", (double)scale);
  return AGENT_ATTN_OK;
}

// ---------------------------------------------------------------- plans
// Workspace layout of the forward (every region 256-byte aligned):
//   [group counters, 512 heads * 512 B, zero between calls][status 256 B]
//   [A fp32 BH*k*d][V_A fp32 BH*k*d][partials ...]
// float32 I/O: partials are BH*nchunks*k*(d+2) floats of the scalar split-N
// aggregation.  bfloat16 I/O: agent and V_A hi/lo fragments exchanged
// between the workgroups of a head, then the partial max/sum (BH*k*P*2
// floats) and accumulators (BH*k*P*d floats).
struct Plan {
  // scalar path
  int chunk = 0, nchunks = 0;
  // matrix-core path
  int DC = 0, P = 1, T = 0, fused = 1, xcd_heads = 0, lds = 0;
  int waves = 8;   // 4: one head per four-wave workgroup, two workgroups per CU
  size_t off_sync = 0, off_status = 0, off_A = 0, off_VA = 0, off_part = 0, bytes = 0;
  size_t off_ml = 0;
};

// Matrix-core kernel instance for these sizes: DC 32-channel chunks
// (1, 2 or 4) and KTC 16-agent tiles (4, 8 or 16).
int mfma_dc(int d) { return d <= 32 ? 1 : (d <= 64 ? 2 : 4); }
int mfma_ktc(int nag) { return nag <= 64 ? 4 : (nag <= 128 ? 8 : 16); }

constexpr size_t kSyncBytesPerHead = aa::kSyncDwords * sizeof(unsigned);
// Heads that can own group counters: P > 1 needs B*H*P <= CUs, so at most
// CUs/2 heads.  The counters live in a fixed-size prefix of every workspace
// so that calls of different shapes sharing one workspace never place other
// scratch data on them.
constexpr long kMaxSyncHeads = 512;
constexpr size_t kSyncRegionBytes = kMaxSyncHeads * kSyncBytesPerHead;

void aggregate_split(const Dims& D, int& chunk, int& nchunks) {
  // Enough blocks to give every one of the 256 CUs two of them, but at
  // least 64 tokens per block.
  long want = (512 + D.BH - 1) / D.BH;
  long maxc = (D.N + 63) / 64;
  long nc = want < maxc ? want : maxc;
  if (nc < 1) nc = 1;
  long ch = (D.N + nc - 1) / nc;
  ch = (ch + 31) / 32 * 32;
  chunk = (int)ch;
  nchunks = (int)((D.N + ch - 1) / ch);
}


template <int DC>
int lds_for(int ktc) {
  return ktc == 4 ? aa::Cfg<DC, 4>::TOTAL : ktc == 8 ? aa::Cfg<DC, 8>::TOTAL : aa::Cfg<DC, 16>::TOTAL;
}
int mfma_lds_bytes(int DC, int nag) {
  const int ktc = mfma_ktc(nag);
  return DC == 1 ? lds_for<1>(ktc) : DC == 2 ? lds_for<2>(ktc) : lds_for<4>(ktc);
}
// LDS of the four-wave instance (up to 64 agents).
int mfma_lds_bytes4(int DC) {
  return DC == 1 ? aa::Cfg<1, 4, 4>::TOTAL
                 : DC == 2 ? aa::Cfg<2, 4, 4>::TOTAL : aa::Cfg<4, 4, 4>::TOTAL;
}
// LDS of the plan left free during the broadcast (after the V_A staging rows
// and fragments); it is the same for eight- and four-wave workgroups.
template <int DC>
long bcast_free_for(int ktc) {
  auto f = [](auto c) {
    using C = decltype(c);
    return (long)C::BIG - (C::STAGE_LDS ? C::STAGE_BYTES : 0) - C::VA_BYTES;
  };
  return ktc == 4 ? f(aa::Cfg<DC, 4>{}) : ktc == 8 ? f(aa::Cfg<DC, 8>{}) : f(aa::Cfg<DC, 16>{});
}
long bcast_free_lds(int DC, int nag) {
  const int ktc = mfma_ktc(nag);
  return DC == 1 ? bcast_free_for<1>(ktc) : DC == 2 ? bcast_free_for<2>(ktc) : bcast_free_for<4>(ktc);
}

// Partials of the matrix-core aggregation, in register order: per (head,
// slot, agent tile) the max/sum of 16 agents and 2*DC rows of 64 x 4 floats.
size_t mfma_ml_bytes(const Dims& D, int P, int DC) {
  (void)DC;
  return (size_t)D.BH * P * mfma_ktc(D.nag) * 16 * 2 * sizeof(float);
}
size_t mfma_acc_bytes(const Dims& D, int P, int DC) {
  return (size_t)D.BH * P * mfma_ktc(D.nag) * 2 * DC * 256 * sizeof(float);
}

// Pooling window geometry: the largest window (tokens) and the number of
// token groups per (agent, chunk) item (a power of two, at most 256).
void pool_params(const Dims& D, int& tgp, int& maxcnt) {
  int mr = 0, mc = 0;
  for (int i = 0; i < D.s; ++i) {
    const int r0 = (i * D.h) / D.s, r1 = ((i + 1) * D.h + D.s - 1) / D.s;
    const int c0 = (i * D.w) / D.s, c1 = ((i + 1) * D.w + D.s - 1) / D.s;
    if (r1 - r0 > mr) mr = r1 - r0;
    if (c1 - c0 > mc) mc = c1 - c0;
  }
  maxcnt = mr * mc;
  const int want = (maxcnt + aa::kPoolTok - 1) / aa::kPoolTok;
  tgp = 1;
  while (tgp < want && tgp < 256) tgp *= 2;
}

// Number of compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// One-time check, per device, of the two facts that the one-XCD exchange of
// the fused kernel relies on:
//  1. workgroup b runs on XCD b % 8 (XCC_ID register);
//  2. data stored with sc0 by one workgroup is returned, after a flag
//     barrier, by sc1 loads of another workgroup on the same XCD, even when
//     the reader's CU cache holds an older copy of those lines (the probe
//     plants one by reading the region before it is written).
// 256 workgroups of 256 threads: member m = b / 8 of XCD x = b % 8's group.
constexpr int kProbeWGs = 256, kProbeWords = 1024;

__global__ void __launch_bounds__(256)
xcd_probe_kernel(int* xcc, unsigned* flags, unsigned* data, unsigned* errors) {
  const int b = blockIdx.x, x = b % 8, m = b / 8, members = kProbeWGs / 8;
  const int nb = (m + 1) % members;
  if (threadIdx.x == 0) xcc[b] = aa::xcc_id();
  unsigned* region = data + (long)x * members * kProbeWords;
  const aa::rsrc_t rd = aa::rsrc_of(region, members * kProbeWords * 4);
  const aa::rsrc_t rf = aa::rsrc_of(flags + x * members, members * 4);
  // plant a stale copy of the neighbour's lines in this CU's cache
  unsigned seen = 0;
  for (int i = threadIdx.x; i < kProbeWords; i += 256)
    seen += __builtin_amdgcn_raw_buffer_load_b32(rd, (nb * kProbeWords + i) * 4, 0, aa::kPlain);
  for (int i = threadIdx.x; i < kProbeWords; i += 256)
    __builtin_amdgcn_raw_buffer_store_b32(0x40000000u + (unsigned)(b * kProbeWords + i), rd,
                                          (m * kProbeWords + i) * 4, 0, aa::kL2);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int ok;
  if (threadIdx.x == 0) __builtin_amdgcn_raw_buffer_store_b32(1u, rf, m * 4, 0, aa::kL2);
  if (threadIdx.x < 64) {
    long spins = 0;
    bool good = true;
    while (true) {
      const unsigned f = threadIdx.x < members
                             ? __builtin_amdgcn_raw_buffer_load_b32(rf, threadIdx.x * 4, 0, aa::kCoherent)
                             : 1u;
      if (__all(f == 1u)) break;
      if (++spins > aa::kSpinLimit) { good = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (threadIdx.x == 0) ok = good;
  }
  __syncthreads();
  unsigned bad = ok ? 0u : (1u << 20);
  if (ok) {
    const unsigned base = 0x40000000u + (unsigned)((x + 8 * nb) * kProbeWords);
    for (int i = threadIdx.x; i < kProbeWords; i += 256) {
      const unsigned v = __builtin_amdgcn_raw_buffer_load_b32(rd, (nb * kProbeWords + i) * 4, 0,
                                                              aa::kCoherent);
      bad += v != base + (unsigned)i;
    }
  }
  bad += seen == 0xffffffffu;   // keeps the planting loads
  if (bad) atomicAdd(errors, bad);
}

// Whether the one-XCD exchange may be used on the current device: both facts
// above hold, checked once per device with the probe launch.  The probe
// synchronises, so it is not run while `st` is being captured into a graph
// (the answer is then "no" for that call, and the check waits for a later
// call).  A failed check selects the device-coherent exchange.
bool xcd_round_robin(hipStream_t st) {
  static std::mutex mu;
  static std::vector<int> cache;   // -1 unknown, 0 no, 1 yes
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, -1);
  if (cache[dev] >= 0) return cache[dev] == 1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return false;
  const size_t n_xcc = kProbeWGs, n_flags = kProbeWGs, n_data = (size_t)kProbeWGs * kProbeWords;
  const size_t bytes = (n_xcc + n_flags + n_data + 1) * 4;
  char* buf = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return false;
  int* d_xcc = (int*)buf;
  unsigned* d_flags = (unsigned*)(buf + n_xcc * 4);
  unsigned* d_data = (unsigned*)(buf + (n_xcc + n_flags) * 4);
  unsigned* d_err = (unsigned*)(buf + (n_xcc + n_flags + n_data) * 4);
  std::vector<int> h(n_xcc, -1);
  unsigned errors = 1;
  bool ok = false;
  if (hipMemset(buf, 0, bytes) == hipSuccess) {
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(kProbeWGs), dim3(256), 0, nullptr, d_xcc, d_flags,
                       d_data, d_err);
    if (hipGetLastError() == hipSuccess &&
        hipMemcpy(h.data(), d_xcc, n_xcc * 4, hipMemcpyDeviceToHost) == hipSuccess &&
        hipMemcpy(&errors, d_err, 4, hipMemcpyDeviceToHost) == hipSuccess) {
      ok = errors == 0;
      for (int b = 0; b < kProbeWGs; ++b) ok = ok && h[b] == b % 8;
    }
  }
  (void)hipFree(buf);
  cache[dev] = ok ? 1 : 0;
  return ok;
}

// Split of each head over P workgroups of T tokens (T a multiple of 16):
// P = floor(CUs / BH), so that the P workgroups of every head fit on the
// chip at once (one per compute unit) and can meet at group barriers.
void mfma_split(const Dims& D, int cus, int& P, int& T) {
  long p = (D.BH >= cus || D.BH > kMaxSyncHeads) ? 1 : cus / D.BH;
  if (p > aa::kMaxGroup) p = aa::kMaxGroup;
  const long maxp = (D.N + 15) / 16;
  if (p > maxp) p = maxp;
  if (p < 1) p = 1;
  long t = (D.N + p - 1) / p;
  t = (t + 15) / 16 * 16;
  P = (int)((D.N + t - 1) / t);
  T = (int)t;
}

Plan make_plan(const Dims& D, int cus) {
  Plan P;
  size_t part_bytes;
  if (D.dtype == AGENT_ATTN_F32) {
    aggregate_split(D, P.chunk, P.nchunks);
    part_bytes = (size_t)D.BH * P.nchunks * D.nag * (D.d + 2) * sizeof(float);
  } else {
    P.DC = mfma_dc(D.d);
    mfma_split(D, cus, P.P, P.T);
    P.lds = mfma_lds_bytes(P.DC, D.nag);
    P.fused = 1;  // BH*P <= CUs: the whole grid is co-resident
    P.xcd_heads = (P.P > 1 && D.BH % 8 == 0 && cus % 8 == 0) ? (int)(D.BH / 8) : 0;
    // more heads than CUs, one workgroup per head: with up to 64 agents and
    // two four-wave workgroups' LDS per CU, every head is resident at once
    // instead of the heads running in rounds of one eight-wave workgroup per CU
    if (P.P == 1 && D.BH > cus && mfma_ktc(D.nag) == 4 &&
        2 * (mfma_lds_bytes4(P.DC) + 64) <= 160 * 1024)
      P.waves = 4;
    part_bytes = 0;  // set with the fragment regions below
  }
  // A and V_A regions: fp32 rows, or in the fused path the bf16 MFMA
  // fragment sets that the group exchanges (whichever is larger)
  size_t a_bytes = (size_t)D.BH * D.nag * D.d * sizeof(float), va_bytes = a_bytes;
  if (D.dtype != AGENT_ATTN_F32) {
    const int ktc = mfma_ktc(D.nag);
    a_bytes = std::max(a_bytes, (size_t)D.BH * aa::a_frag_bytes(ktc, P.DC));
    va_bytes = std::max(va_bytes, (size_t)D.BH * aa::va_frag_bytes(ktc, P.DC));
  }
  P.off_sync = 0;
  P.off_status = kSyncRegionBytes;
  P.off_A = P.off_status + 256;
  P.off_VA = align_up(P.off_A + a_bytes, 256);
  P.off_part = align_up(P.off_VA + va_bytes, 256);
  if (D.dtype != AGENT_ATTN_F32) {
    P.off_ml = P.off_part;
    P.off_part = align_up(P.off_ml + mfma_ml_bytes(D, P.P, P.DC), 256);
    part_bytes = mfma_acc_bytes(D, P.P, P.DC);
  }
  P.bytes = align_up(P.off_part + part_bytes, 256);
  return P;
}

// ------------------------------------------------------------- launches
#define AA_LAUNCH_CHECK(what)                      \
  do {                                             \
    hipError_t e_ = hipGetLastError();             \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

template <typename T>
int launch_pool(const Dims& D, const void* q, float* A, hipStream_t st) {
  const long blocks = D.BH * D.nag;
  hipLaunchKernelGGL(aa::pool_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const T*)q, A, D.h, D.w, D.d, D.s, D.strides());
  AA_LAUNCH_CHECK("agent_pool launch");
  return AGENT_ATTN_OK;
}

template <typename T>
int launch_widen(const Dims& D, const void* src, float* dst, hipStream_t st) {
  const long n = D.BH * D.nag * D.d;
  long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(aa::widen_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const T*)src, dst, n);
  AA_LAUNCH_CHECK("agent widen launch");
  return AGENT_ATTN_OK;
}

template <typename T>
int launch_aggregate(const Dims& D, const float* A, const void* k, const void* v, float* VA,
                     float* part, int chunk, int nchunks, float sl2, hipStream_t st,
                     const float* bias1 = nullptr) {
  const long blocks = D.BH * nchunks;
  if (D.d <= 64)
    hipLaunchKernelGGL((aa::aggregate_partial_scalar<T, 64>), dim3((unsigned)blocks), dim3(256), 0,
                       st, A, (const T*)k, (const T*)v, part, (int)D.N, D.d, D.nag, sl2, chunk,
                       nchunks, D.strides(), bias1);
  else
    hipLaunchKernelGGL((aa::aggregate_partial_scalar<T, 128>), dim3((unsigned)blocks), dim3(256),
                       0, st, A, (const T*)k, (const T*)v, part, (int)D.N, D.d, D.nag, sl2, chunk,
                       nchunks, D.strides(), bias1);
  AA_LAUNCH_CHECK("agent_aggregate launch");
  hipLaunchKernelGGL(aa::merge_partials_kernel, dim3((unsigned)(D.BH * D.nag)), dim3(128), 0, st,
                     part, VA, D.d, D.nag, nchunks);
  AA_LAUNCH_CHECK("agent_aggregate merge launch");
  return AGENT_ATTN_OK;
}

template <typename T>
int launch_broadcast(const Dims& D, const void* q, const float* A, const float* VA, void* out,
                     float sl2, hipStream_t st, aa::ScalarMod md = aa::ScalarMod{}) {
  const int nqblk = (int)((D.N + 255) / 256);
  const long blocks = D.BH * nqblk;
  if (D.d <= 64)
    hipLaunchKernelGGL((aa::broadcast_scalar<T, 64>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const T*)q, A, VA, (T*)out, (int)D.N, D.d, D.nag, sl2, nqblk, D.strides(),
                       md);
  else
    hipLaunchKernelGGL((aa::broadcast_scalar<T, 128>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const T*)q, A, VA, (T*)out, (int)D.N, D.d, D.nag, sl2, nqblk, D.strides(),
                       md);
  AA_LAUNCH_CHECK("agent_broadcast launch");
  return AGENT_ATTN_OK;
}

// ------------------------------------------------------ matrix-core path
#ifdef AGENT_ATTN_PHASE_TRACE
long long* g_trace = nullptr;  // profiling builds: per-workgroup phase stamps
#endif
std::atomic<long> g_spin_limit{aa::kSpinLimit};   // polls before a group wait gives up

int launch_mfma(int DC, bool f16, const aa::MfmaParams& mp, long grid, int nag,
                hipStream_t st) {
  // the dense [B, H, N, d] layout has its own kernel instance, and so has
  // the dense layout with the module terms
  const bool strided = !(mp.sn == mp.d && mp.sh == (long)mp.N * mp.d &&
                         mp.sb == (long)mp.H * mp.N * mp.d);
  const bool module = mp.bias_agg || mp.bias_bcast || mp.dwc_w;
  const bool four = mp.waves == 4 && mp.fused && mp.P == 1;
  const int variant = module    ? (four ? aa::kModule4 : aa::kModule)
                      : strided ? aa::kStrided
                                : (four ? aa::kDense4 : aa::kDense);
  const int ktc = mfma_ktc(nag);
  int e;
  if (f16) {
    switch (DC) {
      case 1: e = aa::launch_mfma_dc<1, aa::ElemF16>(mp, ktc, variant, grid, st); break;
      case 2: e = aa::launch_mfma_dc<2, aa::ElemF16>(mp, ktc, variant, grid, st); break;
      default: e = aa::launch_mfma_dc<4, aa::ElemF16>(mp, ktc, variant, grid, st); break;
    }
  } else {
    switch (DC) {
      case 1: e = aa::launch_mfma_dc<1, aa::ElemBF16>(mp, ktc, variant, grid, st); break;
      case 2: e = aa::launch_mfma_dc<2, aa::ElemBF16>(mp, ktc, variant, grid, st); break;
      default: e = aa::launch_mfma_dc<4, aa::ElemBF16>(mp, ktc, variant, grid, st); break;
    }
  }
  if (e != hipSuccess) return hip_fail((hipError_t)e, "agent attention matrix-core kernel launch");
  return AGENT_ATTN_OK;
}

aa::MfmaParams mfma_params(const Dims& D, int P, int T, float scale) {
  aa::MfmaParams mp{};
  mp.spin_limit = g_spin_limit.load();
  mp.BH = (int)D.BH;
  mp.N = (int)D.N;
  mp.h = D.h;
  mp.w = D.w;
  mp.d = D.d;
  mp.s = D.s;
  mp.nag = D.nag;
  mp.H = (int)(D.H > 0 ? D.H : 1);
  mp.sb = D.sb;
  mp.sh = D.sh;
  mp.sn = (int)D.sn;
  mp.P = P;
  mp.T = T;
  mp.sl2 = scale * aa::kLog2e;
  if (D.s > 0) {
    pool_params(D, mp.pool_tgp, mp.pool_maxcnt);
    while ((1 << mp.pool_tgp_log2) < mp.pool_tgp) ++mp.pool_tgp_log2;
  }
  return mp;
}

// Runs `phases` either in one fused launch or as one launch per phase.
int run_mfma_phases(const Dims& D, aa::MfmaParams mp, int DC, int phases, bool fused,
                    hipStream_t st) {
  const bool module = mp.bias_agg || mp.bias_bcast || mp.dwc_w;
  const int lds = mfma_lds_bytes(DC, D.nag) + (module ? 10 * 32 * DC * 4 : 0);
  if (lds > 160 * 1024 - 64)
    return fail(AGENT_ATTN_ERR_UNSUPPORTED, "d=%d with %d agents needs %d bytes of LDS", D.d,
                D.nag, lds);
  // the DWC reads V from LDS when a workgroup's tokens and their 3 x 3
  // neighbourhood (one grid row and one token on either side) fit beside the
  // plan; otherwise each tap is a load from V
  // neighbourhood (one grid row and one token on either side) fit: in the
  // part of the plan the broadcast leaves free, else beside the plan
  mp.dwc_halo_rows = 0;
  mp.dwc_halo_in_plan = 0;
  long halo = 0;
  if (mp.dwc_w) {
    const long rows = std::min<long>(D.N, (long)mp.T + 2L * D.w + 2);
    halo = rows * (32L * DC + 8) * 2;   // dwc_halo_lds_bytes
    if (halo <= bcast_free_lds(DC, D.nag)) {
      mp.dwc_halo_rows = (int)rows;
      mp.dwc_halo_in_plan = 1;
    } else if (lds + halo <= 160 * 1024 - 64) {
      mp.dwc_halo_rows = (int)rows;
    }
  }
  // the four-wave module instance only where two workgroups still share a CU
  if (module && mp.waves == 4) {
    const long l4 = mfma_lds_bytes4(DC) + 10 * 32 * DC * 4 +
                    (mp.dwc_halo_rows > 0 && !mp.dwc_halo_in_plan ? halo : 0);
    if (2 * (l4 + 64) > 160 * 1024) mp.waves = 8;
  }
  if (((D.N - 1) * D.sn + D.d) * 2 >= (long)aa::kOOB)
    return fail(AGENT_ATTN_ERR_SHAPE, "one head spans %ld elements, above the limit of 2^30",
                (D.N - 1) * D.sn + D.d);
  const long grid = D.BH * mp.P;
  if (fused) {
    mp.phases = phases;
    mp.fused = 1;
    return launch_mfma(DC, D.dtype == AGENT_ATTN_F16, mp, grid, D.nag, st);
  }
  mp.fused = 0;
  mp.xcd_heads = 0;
  for (int ph : {aa::PH_POOL, aa::PH_AGG, aa::PH_MERGE, aa::PH_BCAST}) {
    if (!(phases & ph)) continue;
    if (ph == aa::PH_MERGE && mp.P == 1) continue;
    mp.phases = ph;
    const int rc = launch_mfma(DC, D.dtype == AGENT_ATTN_F16, mp, grid, D.nag, st);
    if (rc) return rc;
  }
  return AGENT_ATTN_OK;
}

// Module terms of a forward (agent biases, depth-wise convolution); all
// null for the plain operator.
struct ModTerms {
  const float* bias_agg = nullptr;     // B1 [H, k, N]
  const float* bias_bcast = nullptr;   // B2 [H, N, k]
  const float* dwc_w = nullptr;        // [H*d, 3, 3]
  const float* dwc_b = nullptr;        // [H*d]
};

int run_forward_mfma(const Dims& D, const Plan& P, const void* q, const void* k, const void* v,
                     void* out, const void* agents, float scale, char* ws, hipStream_t st,
                     const ModTerms& mt) {
  aa::MfmaParams mp = mfma_params(D, P.P, P.T, scale);
  mp.bias_agg = mt.bias_agg;
  mp.bias_bcast = mt.bias_bcast;
  mp.dwc_w = mt.dwc_w;
  mp.dwc_b = mt.dwc_w ? mt.dwc_b : nullptr;
  mp.inv_scale = 1.0f / scale;
  mp.q = (const aa::bf16_t*)q;
  mp.k = (const aa::bf16_t*)k;
  mp.v = (const aa::bf16_t*)v;
  mp.out = (aa::bf16_t*)out;
  mp.agents_in = (const aa::bf16_t*)agents;
  mp.agents_f32 = (float*)(ws + P.off_A);
  mp.values_f32 = (float*)(ws + P.off_VA);
  mp.part_ml = (float*)(ws + P.off_ml);
  mp.part_acc = (float*)(ws + P.off_part);
  mp.sync = (unsigned*)(ws + P.off_sync);
  mp.status = (int*)(ws + P.off_status);
  mp.xcd_heads = (P.xcd_heads > 0 && xcd_round_robin(st)) ? P.xcd_heads : 0;
  mp.waves = P.waves;
#ifdef AGENT_ATTN_PHASE_TRACE
  mp.trace = g_trace;
#endif
  const int phases =
      (agents ? 0 : aa::PH_POOL) | aa::PH_AGG | aa::PH_MERGE | aa::PH_BCAST;
  return run_mfma_phases(D, mp, P.DC, phases, P.fused != 0, st);
}

template <typename T>
int run_forward(const Dims& D, const Plan& P, const void* q, const void* k, const void* v,
                void* out, const void* agents, float scale, char* ws, hipStream_t st,
                const ModTerms& mt) {
  float* A = (float*)(ws + P.off_A);
  float* VA = (float*)(ws + P.off_VA);
  float* part = (float*)(ws + P.off_part);
  const float sl2 = scale * aa::kLog2e;
  int rc = agents ? launch_widen<T>(D, agents, A, st) : launch_pool<T>(D, q, A, st);
  if (rc) return rc;
  rc = launch_aggregate<T>(D, A, k, v, VA, part, P.chunk, P.nchunks, sl2, st, mt.bias_agg);
  if (rc) return rc;
  aa::ScalarMod md{};
  md.bias2 = mt.bias_bcast;
  md.v = v;
  md.dwc_w = mt.dwc_w;
  md.dwc_b = mt.dwc_w ? mt.dwc_b : nullptr;
  md.w = D.w;
  return launch_broadcast<T>(D, q, A, VA, out, sl2, st, md);
}

// Element strides (batch, head, token) of q/k/v/out: positive multiples of
// 8 elements (16-byte aligned rows), at least d between tokens, and no two
// (b, h, n, c) positions on the same element: sorted by stride, the
// dimensions of extent > 1 must nest (each stride at least the previous
// stride times its extent, the first at least d).
int set_strides(Dims& D, long long sb, long long sh, long long sn) {
  if (sb < 1 || sh < 1 || sn < 1)
    return fail(AGENT_ATTN_ERR_SHAPE, "strides %lld, %lld, %lld must be >= 1", sb, sh, sn);
  if (sb % 8 || sh % 8 || sn % 8)
    return fail(AGENT_ATTN_ERR_ALIGN, "strides %lld, %lld, %lld must be multiples of 8 elements",
                sb, sh, sn);
  if (sn < D.d)
    return fail(AGENT_ATTN_ERR_SHAPE, "token stride %lld is below the head dim %d", sn, D.d);
  struct Ext {
    long long st, n;
  } e[3] = {{sn, D.N}, {sh, D.H}, {sb, D.B}};
  std::sort(e, e + 3, [](const Ext& a, const Ext& b) { return a.st < b.st; });
  long long need = D.d;
  for (const Ext& x : e) {
    if (x.n <= 1) continue;
    if (x.st < need)
      return fail(AGENT_ATTN_ERR_SHAPE, "strides %lld, %lld, %lld make elements overlap", sb, sh,
                  sn);
    need = x.st * x.n;
  }
  // byte offsets inside one head are 32-bit in the matrix-core kernels
  if (((D.N - 1) * sn + D.d) * (long long)elem_size(D.dtype) >= (long long)aa::kOOB)
    return fail(AGENT_ATTN_ERR_SHAPE, "one head spans more than 2^31 bytes with token stride %lld",
                sn);
  D.sb = (long)sb;
  D.sh = (long)sh;
  D.sn = (long)sn;
  if (D.span() >= (1L << 40))
    return fail(AGENT_ATTN_ERR_SHAPE, "tensors span more than 2^40 elements");
  return AGENT_ATTN_OK;
}

int validate_forward(Dims& D, const void* q, const void* k, const void* v, void* out,
                     const void* agents, int B, int H, int h, int w, int d, int s, float scale,
                     int dtype, const long long* strides = nullptr) {
  int rc = check_grid(D, B, H, h, w, d, s, dtype);
  if (rc) return rc;
  rc = check_scale(scale);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;  // empty batch: tensors may be NULL
  if (strides) {
    rc = set_strides(D, strides[0], strides[1], strides[2]);
    if (rc) return rc;
  }
  if (!q || !k || !v || !out)
    return fail(AGENT_ATTN_ERR_NULL, "q, k, v and out must be non-NULL");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out) || misaligned(agents))
    return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t tb = (size_t)D.span() * elem_size(dtype);
  const size_t ab = (size_t)D.BH * D.nag * D.d * elem_size(dtype);
  if (ranges_overlap(out, tb, q, tb) || ranges_overlap(out, tb, k, tb) ||
      ranges_overlap(out, tb, v, tb) || ranges_overlap(out, tb, agents, ab))
    return fail(AGENT_ATTN_ERR_ALIAS, "out overlaps an input tensor");
  return AGENT_ATTN_OK;
}

int dispatch_forward(const Dims& D, const Plan& P, const void* q, const void* k, const void* v,
                     void* out, const void* agents, float scale, void* ws, hipStream_t st,
                     const ModTerms& mt = ModTerms{}) {
  if (D.dtype == AGENT_ATTN_F32)
    return run_forward<float>(D, P, q, k, v, out, agents, scale, (char*)ws, st, mt);
  return run_forward_mfma(D, P, q, k, v, out, agents, scale, (char*)ws, st, mt);
}

// Per-device grow-only scratch for agent_attn_forward.
std::mutex g_ws_mutex;
std::vector<std::pair<void*, size_t>> g_ws;

int cached_workspace(size_t bytes, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1, {nullptr, 0});
  auto& slot = g_ws[dev];
  if (slot.second < bytes) {
    if (slot.first) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize before workspace growth");
      e = hipFree(slot.first);
      slot = {nullptr, 0};
      if (e != hipSuccess) return hip_fail(e, "hipFree of the old workspace");
    }
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc of the workspace");
    e = hipMemset(p, 0, bytes);  // the sync counters must start at zero
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "hipMemset of the workspace");
    }
    slot = {p, bytes};
  }
  *ptr = slot.first;
  return AGENT_ATTN_OK;
}

size_t aggregate_ws_bytes(const Dims& D) {
  if (D.dtype == AGENT_ATTN_F32) {
    int chunk, nchunks;
    aggregate_split(D, chunk, nchunks);
    return align_up((size_t)D.BH * nchunks * D.nag * (D.d + 2) * sizeof(float), 256);
  }
  int P, T;
  mfma_split(D, device_cus(), P, T);
  const int DC = mfma_dc(D.d);
  return align_up(mfma_ml_bytes(D, P, DC), 256) + align_up(mfma_acc_bytes(D, P, DC), 256);
}

// Checks the module-term buffers of a forward: 4-byte aligned, within the
// kernels' 32-bit offsets, and disjoint from out and the workspace.
int check_module(const Dims& D, const ModTerms& mt, const void* out, const void* ws,
                 size_t ws_bytes) {
  const size_t bias_bytes = (size_t)D.H * D.nag * D.N * 4;
  const size_t w_bytes = (size_t)D.H * D.d * 9 * 4, b_bytes = (size_t)D.H * D.d * 4;
  const void* ptrs[4] = {mt.bias_agg, mt.bias_bcast, mt.dwc_w, mt.dwc_w ? mt.dwc_b : nullptr};
  const size_t sizes[4] = {bias_bytes, bias_bytes, w_bytes, b_bytes};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] && ((uintptr_t)ptrs[i] & 3u))
      return fail(AGENT_ATTN_ERR_ALIGN, "bias and convolution parameters must be 4-byte aligned");
  if ((mt.bias_agg || mt.bias_bcast) && (size_t)D.nag * D.N * 4 >= (size_t)aa::kOOB)
    return fail(AGENT_ATTN_ERR_SHAPE, "an agent bias of one head spans more than 2^31 bytes");
  if (mt.dwc_w && D.N >= (1L << 22))   // grid positions come from a float-reciprocal division
    return fail(AGENT_ATTN_ERR_SHAPE, "the convolution term supports up to 2^22 tokens");
  const size_t tb = (size_t)D.span() * elem_size(D.dtype);
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) continue;
    if (ranges_overlap(out, tb, ptrs[i], sizes[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "out overlaps a bias or convolution parameter");
    if (ws && ranges_overlap(ws, ws_bytes, ptrs[i], sizes[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "the workspace overlaps a bias or convolution parameter");
  }
  return AGENT_ATTN_OK;
}

int forward_ws(const void* q, const void* k, const void* v, void* out, const void* agents, int B,
               int H, int h, int w, int d, int s, float scale, int dtype, void* workspace,
               size_t workspace_bytes, void* stream, const long long* strides,
               const ModTerms& mt = ModTerms{}) {
  Dims D;
  int rc = validate_forward(D, q, k, v, out, agents, B, H, h, w, d, s, scale, dtype, strides);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  rc = check_module(D, mt, out, workspace, workspace_bytes);
  if (rc) return rc;
  const Plan P = make_plan(D, device_cus());
  if (!workspace || workspace_bytes < P.bytes)
    return fail(AGENT_ATTN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, P.bytes);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(AGENT_ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  const size_t tb = (size_t)D.span() * elem_size(dtype);
  const size_t ab = (size_t)D.BH * D.nag * D.d * elem_size(dtype);
  if (ranges_overlap(workspace, P.bytes, q, tb) || ranges_overlap(workspace, P.bytes, k, tb) ||
      ranges_overlap(workspace, P.bytes, v, tb) || ranges_overlap(workspace, P.bytes, out, tb) ||
      ranges_overlap(workspace, P.bytes, agents, ab))
    return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps a tensor argument");
  return dispatch_forward(D, P, q, k, v, out, agents, scale, workspace, (hipStream_t)stream, mt);
}

// ------------------------------------------------------------- backward
// Workspace of the backward pass (float32 regions, 256-byte aligned): A,
// V_A, dV_A, dA [B*H, k, d]; P2 and dS2 [B*H, N, k]; P1 and dS1 [B*H, k, N];
// dQ, dK, dV accumulators [B*H, N, d]; the split-K partial sums of the
// products over the tokens.
constexpr int kBwdSplit = 256;   // tokens per split of the products over N

struct BwdPlan {
  int splits = 1;
  size_t off_A, off_VA, off_dVA, off_dA, off_P2, off_dS2, off_P1, off_dS1, off_dQ, off_dK,
      off_dV, off_part, bytes;
};

BwdPlan make_bwd_plan(const Dims& D) {
  BwdPlan P;
  P.splits = (int)((D.N + kBwdSplit - 1) / kBwdSplit);
  const size_t kd = (size_t)D.BH * D.nag * D.d * 4;
  const size_t nk = (size_t)D.BH * D.N * D.nag * 4, nd = (size_t)D.BH * D.N * D.d * 4;
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o = align_up(o + b, 256);
    return at;
  };
  P.off_A = take(kd);
  P.off_VA = take(kd);
  P.off_dVA = take(kd);
  P.off_dA = take(kd);
  P.off_P2 = take(nk);
  P.off_dS2 = take(nk);
  P.off_P1 = take(nk);
  P.off_dS1 = take(nk);
  P.off_dQ = take(nd);
  P.off_dK = take(nd);
  P.off_dV = take(nd);
  P.off_part = take(kd * P.splits);
  P.bytes = o;
  return P;
}

// part = alpha * A B for every head (M x N results, contraction K), split
// over K in chunks of kchunk (splits = ceil(K / kchunk)).
// With 16-bit tensors (mfma) the products of two float32 operands (dQ, dK,
// dV: contraction over the agents) run on matrix cores with bf16 operand
// pairs (bgemm_mfma, about 2^-16 per term), 1.7x faster at 256 agents; the
// others are bound by the memory traffic of the probability matrices and
// measured no faster there, so they keep the float32 FMA kernel, as do
// float32 tensors.
template <typename TA, typename TB>
int launch_bgemm(const aa::MatRef& A, const aa::MatRef& B, float* part, int M, int N, int K,
                 int kchunk, long batch, float alpha, hipStream_t st, bool mfma) {
  const int splits = (K + kchunk - 1) / kchunk;
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64),
                  (unsigned)(batch * splits));
  if (mfma && std::is_same<TA, float>::value && std::is_same<TB, float>::value)
    hipLaunchKernelGGL((aa::bgemm_mfma<TA, TB>), grid, dim3(256), 0, st, A, B, part, M, N, K,
                       kchunk, splits, batch, alpha);
  else
    hipLaunchKernelGGL((aa::bgemm_f32<TA, TB>), grid, dim3(256), 0, st, A, B, part, M, N, K,
                       kchunk, splits, batch, alpha);
  AA_LAUNCH_CHECK("backward product launch");
  return AGENT_ATTN_OK;
}

int launch_sum_splits(const float* part, float* out, long n, int splits, float factor,
                      int accumulate, hipStream_t st) {
  const unsigned grid = (unsigned)std::min<long>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(aa::sum_splits, dim3(grid), dim3(256), 0, st, part, out, n, splits, factor,
                     accumulate);
  AA_LAUNCH_CHECK("backward split sum launch");
  return AGENT_ATTN_OK;
}

template <typename T>
int run_backward(const Dims& D, const BwdPlan& P, const void* q, const void* k, const void* v,
                 const void* dout, const void* agents, void* dq, void* dk, void* dv,
                 void* dagents, float scale, char* ws, hipStream_t st) {
  float* A = (float*)(ws + P.off_A);
  float* VA = (float*)(ws + P.off_VA);
  float* dVA = (float*)(ws + P.off_dVA);
  float* dA = (float*)(ws + P.off_dA);
  float* P2 = (float*)(ws + P.off_P2);
  float* dS2 = (float*)(ws + P.off_dS2);
  float* P1 = (float*)(ws + P.off_P1);
  float* dS1 = (float*)(ws + P.off_dS1);
  float* dQ = (float*)(ws + P.off_dQ);
  float* dK = (float*)(ws + P.off_dK);
  float* dV = (float*)(ws + P.off_dV);
  float* part = (float*)(ws + P.off_part);
  const float sl2 = scale * aa::kLog2e;
  const long BH = D.BH, N = D.N, kk = D.nag, d = D.d;
  // operands: [N, d] of type T, and float32 [k, d], [N, k], [k, N] per head
  const aa::MatRef Qm{q, N * d, d, 1}, Km{k, N * d, d, 1}, Vm{v, N * d, d, 1},
      dOm{dout, N * d, d, 1};
  const aa::MatRef KmT{k, N * d, 1, d}, VmT{v, N * d, 1, d};
  const aa::MatRef Am{A, kk * d, d, 1}, AmT{A, kk * d, 1, d}, VAmT{VA, kk * d, 1, d},
      dVAm{dVA, kk * d, d, 1};
  const aa::MatRef P2T{P2, N * kk, 1, kk}, dS2m{dS2, N * kk, kk, 1}, dS2T{dS2, N * kk, 1, kk};
  const aa::MatRef dS1m{dS1, kk * N, N, 1}, dS1T{dS1, kk * N, 1, N}, P1m{P1, kk * N, N, 1},
      P1T{P1, kk * N, 1, N};
  const int KN = kBwdSplit, KALL = 1 << 30;   // split over tokens / no split
  const bool mm = !std::is_same<T, float>::value;   // 16-bit tensors: matrix-core products
  const long nkd = BH * kk * d;
  // forward quantities: agents; P1 = softmax(scale A K^T); V_A = P1 V
  int rc = agents ? launch_widen<T>(D, agents, A, st) : launch_pool<T>(D, q, A, st);
  if (rc) return rc;
  if ((rc = launch_bgemm<float, T>(Am, KmT, P1, (int)kk, (int)N, (int)d, KALL, BH, 1.f, st, mm)))
    return rc;
  hipLaunchKernelGGL(aa::row_softmax_log2, dim3((unsigned)(BH * kk)), dim3(256), 0, st, P1,
                     (int)N, sl2);
  AA_LAUNCH_CHECK("backward aggregation probabilities launch");
  if ((rc = launch_bgemm<float, T>(P1m, Vm, part, (int)kk, (int)d, (int)N, KN, BH, 1.f, st, mm)))
    return rc;
  if ((rc = launch_sum_splits(part, VA, nkd, P.splits, 1.f, 0, st))) return rc;
  // P2 = softmax(scale Q A^T)
  if ((rc = launch_bgemm<T, float>(Qm, AmT, P2, (int)N, (int)kk, (int)d, KALL, BH, 1.f, st, mm)))
    return rc;
  hipLaunchKernelGGL(aa::softmax_short, dim3((unsigned)((BH * N + 3) / 4)), dim3(256), 0, st, P2,
                     BH * N, (int)kk, sl2);
  AA_LAUNCH_CHECK("backward broadcast probabilities launch");
  // dV_A = P2^T dO
  if ((rc = launch_bgemm<float, T>(P2T, dOm, part, (int)kk, (int)d, (int)N, KN, BH, 1.f, st, mm)))
    return rc;
  if ((rc = launch_sum_splits(part, dVA, nkd, P.splits, 1.f, 0, st))) return rc;
  // dS2 = P2 (dO V_A^T - rowsum)
  if ((rc = launch_bgemm<T, float>(dOm, VAmT, dS2, (int)N, (int)kk, (int)d, KALL, BH, 1.f, st, mm)))
    return rc;
  hipLaunchKernelGGL(aa::softmax_grad_short, dim3((unsigned)((BH * N + 3) / 4)), dim3(256), 0, st,
                     P2, dS2, BH * N, (int)kk);
  AA_LAUNCH_CHECK("backward broadcast softmax gradient launch");
  // dQ = scale dS2 A;  dA = scale dS2^T Q
  if ((rc = launch_bgemm<float, float>(dS2m, Am, dQ, (int)N, (int)d, (int)kk, KALL, BH, scale, st, mm)))
    return rc;
  if ((rc = launch_bgemm<float, T>(dS2T, Qm, part, (int)kk, (int)d, (int)N, KN, BH, 1.f, st, mm)))
    return rc;
  if ((rc = launch_sum_splits(part, dA, nkd, P.splits, scale, 0, st))) return rc;
  // dS1 = P1 (dV_A V^T - rowsum)
  if ((rc = launch_bgemm<float, T>(dVAm, VmT, dS1, (int)kk, (int)N, (int)d, KALL, BH, 1.f, st, mm)))
    return rc;
  hipLaunchKernelGGL(aa::softmax_grad_rows, dim3((unsigned)(BH * kk)), dim3(256), 0, st, P1, dS1,
                     (int)N);
  AA_LAUNCH_CHECK("backward aggregation softmax gradient launch");
  // dA += scale dS1 K;  dK = scale dS1^T A;  dV = P1^T dV_A
  if ((rc = launch_bgemm<float, T>(dS1m, Km, part, (int)kk, (int)d, (int)N, KN, BH, 1.f, st, mm)))
    return rc;
  if ((rc = launch_sum_splits(part, dA, nkd, P.splits, scale, 1, st))) return rc;
  if ((rc = launch_bgemm<float, float>(dS1T, Am, dK, (int)N, (int)d, (int)kk, KALL, BH, scale, st, mm)))
    return rc;
  if ((rc = launch_bgemm<float, float>(P1T, dVAm, dV, (int)N, (int)d, (int)kk, KALL, BH, 1.f, st, mm)))
    return rc;
  // outputs in the tensors' type; dq with the pooling's share of dA (16-bit
  // tensors: the vectorised finish of the matrix-core path, one thread per
  // 8 channels of a token)
  const long nnd = BH * N * d;
  const unsigned g_nd = (unsigned)std::min<long>((nnd + 255) / 256, 65536);
  const int tiled = (D.h % D.s == 0 && D.w % D.s == 0) ? 1 : 0;
  const unsigned g_fq = (unsigned)((N * (d / 8) + 255) / 256);
  if constexpr (std::is_same<T, aa::bf16_t>::value) {
    if (BH <= 65535)
      hipLaunchKernelGGL(aa::bw::bwd_finish_dq<aa::ElemBF16>, dim3(g_fq, (unsigned)BH), dim3(256),
                         0, st, dQ, agents ? nullptr : dA, (uint16_t*)dq, (int)N, D.h, D.w,
                         (int)d, D.s, tiled);
    else
      hipLaunchKernelGGL(aa::finish_dq<T>, dim3(g_nd), dim3(256), 0, st, dQ,
                         agents ? nullptr : dA, (T*)dq, BH, (int)N, (int)d, (int)kk, D.h, D.w,
                         D.s);
  } else if constexpr (std::is_same<T, aa::half_t>::value) {
    if (BH <= 65535)
      hipLaunchKernelGGL(aa::bw::bwd_finish_dq<aa::ElemF16>, dim3(g_fq, (unsigned)BH), dim3(256),
                         0, st, dQ, agents ? nullptr : dA, (uint16_t*)dq, (int)N, D.h, D.w,
                         (int)d, D.s, tiled);
    else
      hipLaunchKernelGGL(aa::finish_dq<T>, dim3(g_nd), dim3(256), 0, st, dQ,
                         agents ? nullptr : dA, (T*)dq, BH, (int)N, (int)d, (int)kk, D.h, D.w,
                         D.s);
  } else {
    hipLaunchKernelGGL(aa::finish_dq<T>, dim3(g_nd), dim3(256), 0, st, dQ, agents ? nullptr : dA,
                       (T*)dq, BH, (int)N, (int)d, (int)kk, D.h, D.w, D.s);
  }
  hipLaunchKernelGGL(aa::store_as<T>, dim3(g_nd), dim3(256), 0, st, dK, (T*)dk, nnd);
  hipLaunchKernelGGL(aa::store_as<T>, dim3(g_nd), dim3(256), 0, st, dV, (T*)dv, nnd);
  AA_LAUNCH_CHECK("backward output launch");
  if (agents) {
    const unsigned g_kd = (unsigned)std::min<long>((nkd + 255) / 256, 65536);
    hipLaunchKernelGGL(aa::store_as<T>, dim3(g_kd), dim3(256), 0, st, dA, (T*)dagents, nkd);
    AA_LAUNCH_CHECK("backward agent gradient launch");
  }
  return AGENT_ATTN_OK;
}

// Matrix-core backward (16-bit tensors, up to 64 agents): token-tiled
// passes with the k x d operands in LDS (kernels_bwd_mfma.hpp).
struct MfmaBwdPlan {
  bool use = false;
  int KT = 0, DT = 0;
  aa::bw::Pass pp[3];   // stats, bcast, agg
  int nch = 1;           // chunks of 64 agents (more than 64 agents)
  size_t off_A = 0, off_VA = 0, off_dVA = 0, off_dA = 0, off_lse = 0, off_D1 = 0, off_dQ = 0,
         off_part = 0, off_tst = 0, off_dKf = 0, off_dVf = 0, bytes = 0;
};

// Workgroups per CU that the token-tiled passes aim for over the batch
// (stats, and bcast / agg), in whole steps of tokens.
#ifndef AA_BWD_STATS_WPC
#define AA_BWD_STATS_WPC 2
#endif
#ifndef AA_BWD_TILE_WPC
#define AA_BWD_TILE_WPC 2
#endif
aa::bw::Pass bwd_pass(const Dims& D, int cus, int step, int per_cu) {
  const long per_head = std::max<long>(1, (long)per_cu * cus / D.BH);
  long T = (D.N + per_head - 1) / per_head;
  T = (T + step - 1) / step * step;
  return aa::bw::Pass{(int)((D.N + T - 1) / T), (int)T};
}

MfmaBwdPlan make_mfma_bwd_plan(const Dims& D, int cus) {
  MfmaBwdPlan P;
  if (D.dtype == AGENT_ATTN_F32 || D.nag > 256 || D.d > 128) return P;
  if (D.BH * D.N * D.d >= (1L << 31)) return P;   // 32-bit element indices
  if (D.BH > 65535 || D.BH * D.nag * D.d * 8 >= (1L << 31)) return P;   // grid shapes
  P.KT = D.nag <= 32 ? 2 : 4;
  P.DT = D.d <= 32 ? 1 : D.d <= 64 ? 2 : 4;
  P.nch = (D.nag + 63) / 64;
  P.pp[0] = bwd_pass(D, cus, aa::bw::kStatTok, AA_BWD_STATS_WPC);
  P.pp[1] = P.pp[2] = bwd_pass(D, cus, aa::bw::kStep, AA_BWD_TILE_WPC);
  const size_t kd = (size_t)D.BH * D.nag * D.d * 4,
               kp = (size_t)D.BH * P.nch * 16 * P.KT * 4;
  const size_t nd = (size_t)D.BH * D.N * D.d * 4;
  size_t o = 0;
  auto take = [&](size_t b) {
    const size_t at = o;
    o = align_up(o + b, 256);
    return at;
  };
  P.off_A = take(kd);
  P.off_VA = take(kd);
  P.off_dVA = take(kd);
  P.off_dA = take(kd);
  P.off_lse = take(kp);
  P.off_D1 = take(kp);
  P.off_dQ = take(nd);
  P.off_part = take((size_t)aa::bw::part_floats(P.KT, P.DT, D.BH * P.nch, P.pp) * 4);
  if (P.nch > 1) {
    // per-token softmax statistics of every chunk; float32 sums of dk and dv
    P.off_tst = take((size_t)P.nch * D.BH * D.N * 16);
    P.off_dKf = take(nd);
    P.off_dVf = take(nd);
  }
  P.bytes = o;
  P.use = true;
  return P;
}

template <class El>
int run_backward_mfma(const Dims& D, const MfmaBwdPlan& P, const void* q, const void* k,
                      const void* v, const void* dout, const void* agents, void* dq, void* dk,
                      void* dv, void* dagents, float scale, char* ws, hipStream_t st) {
  aa::bw::BwdParams p{};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.dout = (const uint16_t*)dout;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.A = (float*)(ws + P.off_A);
  p.VA = (float*)(ws + P.off_VA);
  p.lse = (float*)(ws + P.off_lse);
  p.dVA = (float*)(ws + P.off_dVA);
  p.dA = (float*)(ws + P.off_dA);
  p.D1 = (float*)(ws + P.off_D1);
  p.dQ = (float*)(ws + P.off_dQ);
  p.part = (float*)(ws + P.off_part);
  p.agents_in = (const uint16_t*)agents;
  p.dq = (uint16_t*)dq;
  p.dagents = (uint16_t*)dagents;
  p.BH = (int)D.BH;
  p.N = (int)D.N;
  p.d = D.d;
  p.nag = D.nag;
  p.h = D.h;
  p.w = D.w;
  p.s = D.s;
  p.sl2 = scale * aa::kLog2e;
  p.scale = scale;
  p.nch = P.nch;
  p.chunk = 0;
  p.a0 = 0;
  p.nagc = D.nag;
  if (P.nch > 1) {
    p.tst = (float*)(ws + P.off_tst);
    p.dKf = (float*)(ws + P.off_dKf);
    p.dVf = (float*)(ws + P.off_dVf);
  }
#ifdef AGENT_ATTN_PHASE_TRACE
  p.trace = g_trace;
#endif
  const int e = aa::bw::run_backward_mfma<El>(p, P.KT, P.DT, P.pp, st);
  if (e) return hip_fail((hipError_t)e, "backward matrix-core launch");
  return AGENT_ATTN_OK;
}

// Workspace of the module with projections: the attention's own workspace
// first (so that the leading synchronisation bytes are the same as
// agent_attn_forward_ws's), then q, k, v [3][B, H, N, d] and o [B, H, N, d]
// in the tensors' format.
struct ModulePlan {
  size_t off_attn = 0, attn_bytes = 0, off_qkv = 0, off_o = 0, bytes = 0;
};

ModulePlan make_module_plan(const Dims& D) {
  ModulePlan P;
  const size_t t = (size_t)D.BH * D.N * D.d * elem_size(D.dtype);
  P.attn_bytes = make_plan(D, device_cus()).bytes;
  P.off_qkv = align_up(P.attn_bytes, 256);
  P.off_o = align_up(P.off_qkv + 3 * t, 256);
  P.bytes = P.off_o + t;
  return P;
}

}  // namespace

extern "C" {

size_t agent_attn_workspace_bytes(int B, int H, int h, int w, int d, int s, int dtype) {
  Dims D;
  if (check_grid(D, B, H, h, w, d, s, dtype)) return 0;
  if (D.BH == 0) return 0;
  return make_plan(D, device_cus()).bytes;
}


int agent_attn_forward_ws(const void* q, const void* k, const void* v, void* out,
                          const void* agents, int B, int H, int h, int w, int d, int s,
                          float scale, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return forward_ws(q, k, v, out, agents, B, H, h, w, d, s, scale, dtype, workspace,
                    workspace_bytes, stream, nullptr);
}

int agent_attn_forward_strided(const void* q, const void* k, const void* v, void* out,
                               const void* agents, int B, int H, int h, int w, int d, int s,
                               long long stride_b, long long stride_h, long long stride_n,
                               float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const long long st[3] = {stride_b, stride_h, stride_n};
  return forward_ws(q, k, v, out, agents, B, H, h, w, d, s, scale, dtype, workspace,
                    workspace_bytes, stream, st);
}

int agent_attn_forward_module(const void* q, const void* k, const void* v, void* out,
                              const void* agents, const float* bias_agg, const float* bias_bcast,
                              const float* dwc_weight, const float* dwc_bias, int B, int H, int h,
                              int w, int d, int s, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  ModTerms mt;
  mt.bias_agg = bias_agg;
  mt.bias_bcast = bias_bcast;
  mt.dwc_w = dwc_weight;
  mt.dwc_b = dwc_bias;
  return forward_ws(q, k, v, out, agents, B, H, h, w, d, s, scale, dtype, workspace,
                    workspace_bytes, stream, nullptr, mt);
}

size_t agent_attn_module_workspace_bytes(int B, int H, int h, int w, int d, int s, int dtype) {
  Dims D;
  if (check_grid(D, B, H, h, w, d, s, dtype)) return 0;
  if (D.BH == 0) return 0;
  return make_module_plan(D).bytes;
}

int agent_attn_module_forward(const void* x, const void* w_qkv, const float* b_qkv,
                              const void* w_out, const float* b_out, const void* agents,
                              const float* bias_agg, const float* bias_bcast,
                              const float* dwc_weight, const float* dwc_bias, void* y, int B,
                              int H, int h, int w, int d, int s, float scale, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Dims D;
  int rc = check_grid(D, B, H, h, w, d, s, dtype);
  if (rc) return rc;
  rc = check_scale(scale);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  if (!x || !w_qkv || !y) return fail(AGENT_ATTN_ERR_NULL, "x, w_qkv and y must be non-NULL");
  const long C = (long)H * d, M = (long)B * D.N;
  if (M * C * 4 >= (1L << 31) || 3 * C * C * 4 >= (1L << 31) || (M + 127) / 128 > 65535)
    return fail(AGENT_ATTN_ERR_UNSUPPORTED,
                "the projections take B*N*C*4 and 3*C*C*4 below 2^31 bytes and B*N below "
                "2^23 tokens (C = H*d = %ld)", C);
  if (misaligned(x) || misaligned(w_qkv) || misaligned(w_out) || misaligned(y) ||
      misaligned(agents))
    return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (((uintptr_t)b_qkv & 3u) || ((uintptr_t)b_out & 3u))
    return fail(AGENT_ATTN_ERR_ALIGN, "biases must be 4-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t xb = (size_t)(M * C) * es, wqb = (size_t)(3 * C * C) * es, wob = (size_t)(C * C) * es;
  const size_t ab = (size_t)D.BH * D.nag * d * es;
  const void* ins[5] = {x, w_qkv, w_out, agents, nullptr};
  const size_t insz[5] = {xb, wqb, wob, ab, 0};
  const void* bs[2] = {b_qkv, b_out};
  const size_t bsz[2] = {(size_t)(3 * C) * 4, (size_t)C * 4};
  for (int i = 0; i < 4; ++i)
    if (ins[i] && ranges_overlap(y, xb, ins[i], insz[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "y overlaps an input");
  for (int i = 0; i < 2; ++i)
    if (bs[i] && ranges_overlap(y, xb, bs[i], bsz[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "y overlaps a bias");
  const ModulePlan P = make_module_plan(D);
  if (!workspace || workspace_bytes < P.bytes)
    return fail(AGENT_ATTN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, P.bytes);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(AGENT_ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (ranges_overlap(workspace, P.bytes, y, xb))
    return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps y");
  for (int i = 0; i < 4; ++i)
    if (ins[i] && ranges_overlap(workspace, P.bytes, ins[i], insz[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps an input");
  for (int i = 0; i < 2; ++i)
    if (bs[i] && ranges_overlap(workspace, P.bytes, bs[i], bsz[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps a bias");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const size_t t = (size_t)D.BH * D.N * d * es;
  char* q = ws + P.off_qkv;
  char* o = ws + P.off_o;
  aa::pj::ProjParams pp{};
  pp.x = x;
  pp.w = w_qkv;
  pp.bias = b_qkv;
  pp.y = q;
  pp.M = (int)M;
  pp.C = (int)C;
  pp.Nout = (int)(3 * C);
  pp.N = (int)D.N;
  pp.H = H;
  pp.d = d;
  int e = aa::pj::launch_proj(pp, 0, dtype, st);
  if (e) return hip_fail((hipError_t)e, "q, k, v projection launch");
  ModTerms mt;
  mt.bias_agg = bias_agg;
  mt.bias_bcast = bias_bcast;
  mt.dwc_w = dwc_weight;
  mt.dwc_b = dwc_bias;
  rc = forward_ws(q, q + t, q + 2 * t, o, agents, B, H, h, w, d, s, scale, dtype,
                  ws + P.off_attn, P.attn_bytes, stream, nullptr, mt);
  if (rc) return rc;
  if (w_out) {
    pp.x = o;
    pp.w = w_out;
    pp.bias = b_out;
    pp.y = y;
    pp.Nout = (int)C;
    e = aa::pj::launch_proj(pp, 1, dtype, st);
    if (e) return hip_fail((hipError_t)e, "output projection launch");
  } else {
    e = aa::pj::launch_heads_concat(o, y, (int)M, (int)D.N, H, d, dtype, st);
    if (e) return hip_fail((hipError_t)e, "head concatenation launch");
  }
  return AGENT_ATTN_OK;
}

int agent_attn_forward(const void* q, const void* k, const void* v, void* out,
                       const void* agents, int B, int H, int h, int w, int d, int s, float scale,
                       int dtype, void* stream) {
  Dims D;
  int rc = validate_forward(D, q, k, v, out, agents, B, H, h, w, d, s, scale, dtype);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  const Plan P = make_plan(D, device_cus());
  void* ws = nullptr;
  rc = cached_workspace(P.bytes, &ws);
  if (rc) return rc;
  return dispatch_forward(D, P, q, k, v, out, agents, scale, ws, (hipStream_t)stream);
}

int agent_attn_pool(const void* q, float* agents_f32, int B, int H, int h, int w, int d, int s,
                    int dtype, void* stream) {
  Dims D;
  int rc = check_grid(D, B, H, h, w, d, s, dtype);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  if (!q || !agents_f32) return fail(AGENT_ATTN_ERR_NULL, "q and agents_f32 must be non-NULL");
  if (misaligned(q) || misaligned(agents_f32))
    return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (ranges_overlap(agents_f32, (size_t)D.BH * D.nag * D.d * 4, q,
                     (size_t)D.BH * D.N * D.d * elem_size(dtype)))
    return fail(AGENT_ATTN_ERR_ALIAS, "agents_f32 overlaps q");
  hipStream_t st = (hipStream_t)stream;
  if (dtype == AGENT_ATTN_F32) return launch_pool<float>(D, q, agents_f32, st);
  aa::MfmaParams mp = mfma_params(D, 1, (int)D.N, 1.0f);
  mp.q = (const aa::bf16_t*)q;
  mp.agents_f32 = agents_f32;
  return run_mfma_phases(D, mp, mfma_dc(D.d), aa::PH_POOL, false, st);
}

size_t agent_attn_aggregate_workspace_bytes(int B, int H, int N, int d, int n_agents, int dtype) {
  Dims D;
  if (check_core(D, B, H, N, d, n_agents, dtype)) return 0;
  if (D.BH == 0) return 0;
  return aggregate_ws_bytes(D);
}

int agent_attn_aggregate(const float* agents_f32, const void* k, const void* v,
                         float* agent_values_f32, int B, int H, int N, int d, int n_agents,
                         float scale, int dtype, void* workspace, size_t workspace_bytes,
                         void* stream) {
  Dims D;
  int rc = check_core(D, B, H, N, d, n_agents, dtype);
  if (rc) return rc;
  rc = check_scale(scale);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  if (!agents_f32 || !k || !v || !agent_values_f32)
    return fail(AGENT_ATTN_ERR_NULL, "agents_f32, k, v and agent_values_f32 must be non-NULL");
  if (misaligned(agents_f32) || misaligned(k) || misaligned(v) || misaligned(agent_values_f32))
    return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = aggregate_ws_bytes(D);
  if (!workspace || workspace_bytes < need)
    return fail(AGENT_ATTN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, need);
  const size_t tb = (size_t)D.BH * D.N * D.d * elem_size(dtype);
  const size_t ab = (size_t)D.BH * D.nag * D.d * 4;
  if (ranges_overlap(agent_values_f32, ab, agents_f32, ab) ||
      ranges_overlap(agent_values_f32, ab, k, tb) || ranges_overlap(agent_values_f32, ab, v, tb) ||
      ranges_overlap(workspace, need, agents_f32, ab) || ranges_overlap(workspace, need, k, tb) ||
      ranges_overlap(workspace, need, v, tb) ||
      ranges_overlap(workspace, need, agent_values_f32, ab))
    return fail(AGENT_ATTN_ERR_ALIAS, "an output or the workspace overlaps an input");
  const float sl2 = scale * aa::kLog2e;
  hipStream_t st = (hipStream_t)stream;
  float* part = (float*)workspace;
  if (dtype == AGENT_ATTN_F32) {
    int chunk, nchunks;
    aggregate_split(D, chunk, nchunks);
    return launch_aggregate<float>(D, agents_f32, k, v, agent_values_f32, part, chunk, nchunks,
                                   sl2, st);
  }
  int P, T;
  mfma_split(D, device_cus(), P, T);
  aa::MfmaParams mp = mfma_params(D, P, T, scale);
  mp.k = (const aa::bf16_t*)k;
  mp.v = (const aa::bf16_t*)v;
  mp.agents_f32_in = agents_f32;
  mp.values_f32 = agent_values_f32;
  mp.part_ml = part;
  mp.part_acc = (float*)((char*)workspace + align_up(mfma_ml_bytes(D, P, mfma_dc(D.d)), 256));
  return run_mfma_phases(D, mp, mfma_dc(D.d), aa::PH_AGG | aa::PH_MERGE, false, st);
}

int agent_attn_broadcast(const void* q, const float* agents_f32, const float* agent_values_f32,
                         void* out, int B, int H, int N, int d, int n_agents, float scale,
                         int dtype, void* stream) {
  Dims D;
  int rc = check_core(D, B, H, N, d, n_agents, dtype);
  if (rc) return rc;
  rc = check_scale(scale);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  if (!q || !agents_f32 || !agent_values_f32 || !out)
    return fail(AGENT_ATTN_ERR_NULL, "q, agents_f32, agent_values_f32 and out must be non-NULL");
  if (misaligned(q) || misaligned(agents_f32) || misaligned(agent_values_f32) || misaligned(out))
    return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t tb = (size_t)D.BH * D.N * D.d * elem_size(dtype);
  const size_t ab = (size_t)D.BH * D.nag * D.d * 4;
  if (ranges_overlap(out, tb, q, tb) || ranges_overlap(out, tb, agents_f32, ab) ||
      ranges_overlap(out, tb, agent_values_f32, ab))
    return fail(AGENT_ATTN_ERR_ALIAS, "out overlaps an input tensor");
  const float sl2 = scale * aa::kLog2e;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == AGENT_ATTN_F32)
    return launch_broadcast<float>(D, q, agents_f32, agent_values_f32, out, sl2, st);
  int P, T;
  mfma_split(D, device_cus(), P, T);
  aa::MfmaParams mp = mfma_params(D, P, T, scale);
  mp.q = (const aa::bf16_t*)q;
  mp.out = (aa::bf16_t*)out;
  mp.agents_f32_in = agents_f32;
  mp.values_f32_in = agent_values_f32;
  return run_mfma_phases(D, mp, mfma_dc(D.d), aa::PH_BCAST, false, st);
}

size_t agent_attn_backward_workspace_bytes(int B, int H, int h, int w, int d, int s, int dtype) {
  Dims D;
  if (check_grid(D, B, H, h, w, d, s, dtype)) return 0;
  if (D.BH == 0) return 0;
  const MfmaBwdPlan M = make_mfma_bwd_plan(D, device_cus());
  return M.use ? M.bytes : make_bwd_plan(D).bytes;
}

int agent_attn_backward(const void* q, const void* k, const void* v, const void* dout,
                        const void* agents, void* dq, void* dk, void* dv, void* dagents, int B,
                        int H, int h, int w, int d, int s, float scale, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Dims D;
  int rc = check_grid(D, B, H, h, w, d, s, dtype);
  if (rc) return rc;
  rc = check_scale(scale);
  if (rc) return rc;
  if (D.BH == 0) return AGENT_ATTN_OK;
  if (!q || !k || !v || !dout || !dq || !dk || !dv)
    return fail(AGENT_ATTN_ERR_NULL, "q, k, v, dout, dq, dk and dv must be non-NULL");
  if (agents && !dagents)
    return fail(AGENT_ATTN_ERR_NULL, "supplied agents need dagents for their gradient");
  const void* all[9] = {q, k, v, dout, agents, dq, dk, dv, agents ? dagents : nullptr};
  for (const void* p : all)
    if (misaligned(p)) return fail(AGENT_ATTN_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t tb = (size_t)D.span() * elem_size(dtype);
  const size_t ab = (size_t)D.BH * D.nag * D.d * elem_size(dtype);
  const size_t sizes[9] = {tb, tb, tb, tb, ab, tb, tb, tb, ab};
  for (int o = 5; o < 9; ++o) {   // outputs against inputs and each other
    if (!all[o]) continue;
    for (int i = 0; i < 9; ++i)
      if (i != o && all[i] && ranges_overlap(all[o], sizes[o], all[i], sizes[i]))
        return fail(AGENT_ATTN_ERR_ALIAS, "a gradient output overlaps another tensor argument");
  }
  const MfmaBwdPlan M = make_mfma_bwd_plan(D, device_cus());
  if (M.use) {
    if (!workspace || workspace_bytes < M.bytes)
      return fail(AGENT_ATTN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                  workspace_bytes, workspace, M.bytes);
    if (((uintptr_t)workspace & 255u) != 0)
      return fail(AGENT_ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
    for (int i = 0; i < 9; ++i)
      if (all[i] && ranges_overlap(workspace, M.bytes, all[i], sizes[i]))
        return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps a tensor argument");
    hipStream_t st = (hipStream_t)stream;
    if (dtype == AGENT_ATTN_BF16)
      return run_backward_mfma<aa::ElemBF16>(D, M, q, k, v, dout, agents, dq, dk, dv,
                                                         dagents, scale, (char*)workspace, st);
    return run_backward_mfma<aa::ElemF16>(D, M, q, k, v, dout, agents, dq, dk, dv,
                                                      dagents, scale, (char*)workspace, st);
  }
  const BwdPlan P = make_bwd_plan(D);
  if (D.BH * P.splits > 65535)   // grid z of the products over the tokens
    return fail(AGENT_ATTN_ERR_UNSUPPORTED,
                "the backward pass takes B*H*ceil(N/%d) <= 65535 (here %ld)", kBwdSplit,
                D.BH * P.splits);
  if (!workspace || workspace_bytes < P.bytes)
    return fail(AGENT_ATTN_ERR_WORKSPACE, "workspace of %zu bytes at %p; %zu bytes needed",
                workspace_bytes, workspace, P.bytes);
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(AGENT_ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
  for (int i = 0; i < 9; ++i)
    if (all[i] && ranges_overlap(workspace, P.bytes, all[i], sizes[i]))
      return fail(AGENT_ATTN_ERR_ALIAS, "workspace overlaps a tensor argument");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  switch (dtype) {
    case AGENT_ATTN_F32:
      return run_backward<float>(D, P, q, k, v, dout, agents, dq, dk, dv, dagents, scale, ws, st);
    case AGENT_ATTN_BF16:
      return run_backward<aa::bf16_t>(D, P, q, k, v, dout, agents, dq, dk, dv, dagents, scale,
                                      ws, st);
    default:
      return run_backward<aa::half_t>(D, P, q, k, v, dout, agents, dq, dk, dv, dagents, scale,
                                      ws, st);
  }
}

long agent_attn_set_wait_limit(long polls) {
  const long prev = g_spin_limit.load();
  if (polls >= 0) g_spin_limit.store(polls);
  return prev;
}

int agent_attn_read_faults(void* workspace, void* stream, int* faults) {
  if (!faults) return fail(AGENT_ATTN_ERR_NULL, "faults must be non-NULL");
  *faults = 0;
  char* ws = (char*)workspace;
  if (!ws) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if ((int)g_ws.size() > dev) ws = (char*)g_ws[dev].first;
  }
  if (!ws) return AGENT_ATTN_OK;   // no fused launch has run on this device
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  unsigned word = 0;
  e = hipMemcpy(&word, ws + kSyncRegionBytes, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy of the fault word");
  if (word) {
    e = hipMemset(ws + kSyncRegionBytes, 0, sizeof(word));
    if (e != hipSuccess) return hip_fail(e, "hipMemset of the fault word");
  }
  *faults = (int)word;
  return AGENT_ATTN_OK;
}

void agent_attn_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  for (size_t dev = 0; dev < g_ws.size(); ++dev) {
    if (!g_ws[dev].first) continue;
    if (hipSetDevice((int)dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws[dev].first);
    }
    g_ws[dev] = {nullptr, 0};
  }
  if (cur >= 0) (void)hipSetDevice(cur);
}

const char* agent_attn_status_string(int status) {
  switch (status) {
    case AGENT_ATTN_OK: return "ok";
    case AGENT_ATTN_ERR_NULL: return "a required pointer is NULL";
    case AGENT_ATTN_ERR_SHAPE: return "a size is out of range";
    case AGENT_ATTN_ERR_DTYPE: return "unknown dtype";
    case AGENT_ATTN_ERR_UNSUPPORTED: return "head dim or agent count outside the supported limits";
    case AGENT_ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case AGENT_ATTN_ERR_ALIAS: return "an output overlaps an input";
    case AGENT_ATTN_ERR_ALIGN: return "a pointer is not sufficiently aligned";
    case AGENT_ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case AGENT_ATTN_ERR_HIP: return "a HIP runtime call failed";
    default: return "unknown status";
  }
}

const char* agent_attn_last_error(void) { return g_last_error.c_str(); }

#ifdef AGENT_ATTN_PHASE_TRACE
// Profiling builds only: device buffer of 16 int64 stamps per workgroup.
void agent_attn_debug_set_trace(void* trace) { g_trace = (long long*)trace; }
#endif

}  // extern "C"
