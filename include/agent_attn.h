/*
 * agent_attn.h -- C ABI of the MI355X (gfx950) Agent Attention forward.
 *
 * The operation (sources: the web pages
 *   "Agent Attention: On the Integration of Softmax and Linear Attention"
 *   (paperlayer.ai summary of arXiv 2312.08874v3), Abstract, §4 Agent
 *   Transformer and §6 Conclusion; and
 *   "Agent Attention：Transformer计算量太大？试试这个'代理令牌'的轻量化方案"
 *   (jsqmd.com), §1 pseudocode and §2):
 *
 *   For every batch b and head h independently, with Q, K, V of shape
 *   [N, d] over a row-major h x w token grid (token n = r*w + c):
 *     1. agents   A   = 2-D average pool of Q down to an s x s grid, k = s*s
 *                       (agent i*s+j averages grid rows
 *                       [floor(i*h/s), ceil((i+1)*h/s)) and columns
 *                       [floor(j*w/s), ceil((j+1)*w/s))), or caller-supplied;
 *     2. aggregation  V_A = softmax(scale * A K^T) V      (softmax over N)
 *     3. broadcast    O   = softmax(scale * Q A^T) V_A    (softmax over k)
 *   Both steps are ordinary Softmax attentions; together they form the
 *   generalised linear attention phi_q(Q) phi_k(K)^T V of §4.
 *
 * Layout: every tensor is dense, row-major, contiguous:
 *   q, k, v, out : [B, H, N, d]      (N = h*w)
 *   agents       : [B, H, k, d]      (k = s*s, or n_agents in the step calls)
 *   agents_f32 / agent_values_f32 in the step calls: float32 [B, H, k, d].
 * Element type of q, k, v, out and caller agents: `dtype` (float32,
 * bfloat16 or float16).  Arithmetic is float32: 16-bit inputs feed the
 * matrix cores in their own format, accumulation is float32, and O is
 * rounded to the I/O format with round-to-nearest-even.  With float16 the
 * pooled agents, the probabilities and V_A are float16 matrix-core operands;
 * the partial aggregation sums exchanged between workgroups stay float32 or
 * bfloat16 (float16 has too little range for unnormalised sums).
 *
 * Pointers: device pointers (hipMalloc/torch CUDA tensors) of the current
 * device, 16-byte aligned.  The library never frees or retains them.
 * `stream` is a hipStream_t (NULL = the default stream); all work is
 * enqueued on it asynchronously and the call returns once it is enqueued.
 *
 * Errors: every argument is validated on the host before any HIP call; a
 * failed check returns a negative status and enqueues nothing.  Kernel
 * launch failures return AGENT_ATTN_ERR_HIP.  Faults inside kernels surface
 * at the caller's next synchronisation.  agent_attn_last_error() gives a
 * message for the calling thread's last failure.  Non-finite inputs are not
 * checked and propagate.  B == 0 or H == 0 is an empty batch: nothing is
 * enqueued and AGENT_ATTN_OK is returned.
 *
 * Limits: 1 <= s <= min(h, w); s*s <= 256 agents; d % 8 == 0, 8 <= d <= 128;
 * B*H*N*d < 2^40 elements; scale finite and > 0.
 *
 * Thread safety: all entry points may be called from several threads.
 * Calls that share a workspace buffer must be ordered on one stream.
 */
#ifndef AGENT_ATTN_H_
#define AGENT_ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AGENT_ATTN_F32 = 0,
  AGENT_ATTN_BF16 = 1,
  AGENT_ATTN_F16 = 2
} agent_attn_dtype_t;

typedef enum {
  AGENT_ATTN_OK = 0,
  AGENT_ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  AGENT_ATTN_ERR_SHAPE = -2,       /* a size is out of range */
  AGENT_ATTN_ERR_DTYPE = -3,       /* unknown dtype */
  AGENT_ATTN_ERR_UNSUPPORTED = -4, /* d or agent count outside the limits */
  AGENT_ATTN_ERR_SCALE = -5,       /* scale not finite or not > 0 */
  AGENT_ATTN_ERR_ALIAS = -6,       /* an output overlaps an input */
  AGENT_ATTN_ERR_ALIGN = -7,       /* a pointer is not 16-byte aligned */
  AGENT_ATTN_ERR_WORKSPACE = -8,   /* workspace NULL or too small */
  AGENT_ATTN_ERR_HIP = -9          /* a HIP call failed */
} agent_attn_status_t;

#define AGENT_ATTN_MAX_AGENTS 256
/* Leading workspace bytes that must be zero before a workspace's first use. */
#define AGENT_ATTN_SYNC_BYTES (512 * 512)
#define AGENT_ATTN_MAX_HEAD_DIM 128

/* Bytes of device scratch the forward needs for these sizes (0 when
 * B*H == 0).  Returns 0 and sets the last error for invalid sizes. */
size_t agent_attn_workspace_bytes(int B, int H, int h, int w, int d, int s,
                                  int dtype);

/* Full forward: pool (when agents == NULL) -> aggregate -> broadcast.
 * agents: NULL, or caller-supplied agents [B, H, s*s, d] of `dtype`.
 * Uses a per-device scratch buffer that the library allocates on first use
 * and grows as needed (hipMalloc; freed by agent_attn_release).  Calls on
 * different streams of one device that overlap in time share that buffer
 * and therefore race: use agent_attn_forward_ws for concurrent streams. */
int agent_attn_forward(const void* q, const void* k, const void* v, void* out,
                       const void* agents, int B, int H, int h, int w, int d,
                       int s, float scale, int dtype, void* stream);

/* Same as agent_attn_forward with caller-owned scratch of at least
 * agent_attn_workspace_bytes(...) bytes, 256-byte aligned, that must not
 * overlap any tensor argument.  Its first AGENT_ATTN_SYNC_BYTES bytes hold
 * the counters of the workgroup barriers: they must be zero before the
 * workspace is first used (zero-fill it once after allocation), and every
 * call leaves them zero again, so one workspace serves any sequence of
 * calls of any shapes that are ordered on one stream.  The rest is
 * overwritten freely.  The call allocates nothing. */
int agent_attn_forward_ws(const void* q, const void* k, const void* v,
                          void* out, const void* agents, int B, int H, int h,
                          int w, int d, int s, float scale, int dtype,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Same as agent_attn_forward_ws with q, k, v and out given by element
 * strides instead of the dense [B, H, N, d] layout: element (b, h, n, c) is
 * at b*stride_b + h*stride_h + n*stride_n + c (channels contiguous), the same
 * strides for all four.  [B, N, H, d] storage, as a projection to H heads
 * produces, has stride_b = N*H*d, stride_h = d, stride_n = H*d.  Strides must
 * be positive multiples of 8 elements, stride_n >= d, and no two positions
 * may share an element (AGENT_ATTN_ERR_SHAPE / AGENT_ATTN_ERR_ALIGN
 * otherwise); one head may span at most 2^31 bytes.  Caller-supplied agents
 * stay dense [B, H, s*s, d].  The range from a tensor's first to its last
 * element must not overlap the workspace, and out's must not overlap those
 * of the inputs. */
int agent_attn_forward_strided(const void* q, const void* k, const void* v,
                               void* out, const void* agents, int B, int H,
                               int h, int w, int d, int s, long long stride_b,
                               long long stride_h, long long stride_n,
                               float scale, int dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* The full module's forward (sources: "Agent Attention: On the Integration
 * of Softmax and Linear Attention", §4 Module Enhancements, Implementation
 * Details and the Efficiency paragraph): the operator above with the agent
 * biases added to the scaled logits of both attentions and the depth-wise
 * convolution of V added to the output,
 *   V_A = softmax(scale A K^T + B1) V,   O = softmax(scale Q A^T + B2) V_A + DWC(V).
 * The page names the biases' construction (column, row and block
 * components) without giving it, so the caller passes the full tensors:
 *   bias_agg   : NULL or B1, float32 [H, k, N] (k = s*s), shared by the batch;
 *   bias_bcast : NULL or B2, float32 [H, N, k], shared by the batch;
 *   dwc_weight : NULL (no convolution term) or float32 [H*d, 3, 3]: channel c
 *                of head h uses row h*d + c; out[n] += sum over the 3 x 3
 *                grid neighbourhood of token n of weight[dy+1][dx+1] *
 *                v[neighbour] (cross-correlation), taps outside the h x w
 *                grid reading zero;
 *   dwc_bias   : NULL (zero) or float32 [H*d]; ignored without dwc_weight.
 * All four are device pointers, 4-byte aligned, read only, and must not
 * overlap out or the workspace (AGENT_ATTN_ERR_ALIGN / _ALIAS otherwise);
 * one head's bias may span at most 2^31 bytes.  With all four NULL this is
 * agent_attn_forward_ws.  Tensors are dense [B, H, N, d]; the other
 * arguments, the workspace (agent_attn_workspace_bytes) and the errors are
 * those of agent_attn_forward_ws.  The call allocates nothing. */
int agent_attn_forward_module(const void* q, const void* k, const void* v,
                              void* out, const void* agents,
                              const float* bias_agg, const float* bias_bcast,
                              const float* dwc_weight, const float* dwc_bias,
                              int B, int H, int h, int w, int d, int s,
                              float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Scratch bytes agent_attn_module_forward needs for these sizes (0 for
 * invalid sizes or an empty batch). */
size_t agent_attn_module_workspace_bytes(int B, int H, int h, int w, int d,
                                         int s, int dtype);

/* The attention module on token features (sources: "Agent Attention: On the
 * Integration of Softmax and Linear Attention", §3 Preliminaries: the
 * projections W_Q, W_K, W_V map channels to per-head queries, keys and
 * values; §4: agent attention with the module terms; "别再死磕Softmax了！…",
 * coreui.cn, §3.1: AgentAttention(dim, num_heads, num_agents) maps
 * [B, N, dim] to [B, N, dim]):
 *   q, k, v = x w_qkv^T + b_qkv   (the 3C outputs in the order q, k, v; each
 *                                  read as H heads of d channels, feature
 *                                  h*d + c = channel c of head h)
 *   o       = agent_attn_forward_module(q, k, v, agents, module terms)
 *   y       = o w_out^T + b_out   (o as [B, N, C], heads side by side)
 * with C = H*d and N = h*w:
 *   x      : [B, N, C] of dtype;
 *   w_qkv  : [3C, C] of dtype (Linear layout [out, in]); b_qkv: NULL or
 *            float32 [3C];
 *   w_out  : NULL (y = o) or [C, C] of dtype; b_out: NULL or float32 [C];
 *   agents, bias_agg, bias_bcast, dwc_weight, dwc_bias: as
 *            agent_attn_forward_module;
 *   y      : [B, N, C] of dtype.
 * q, k, v and o are held in dtype inside the workspace (as the outputs of
 * Linear layers of that format are); products accumulate in float32 and each
 * result is rounded once.  Tensor pointers 16-byte aligned, biases 4-byte
 * aligned (AGENT_ATTN_ERR_ALIGN); y may not overlap an input nor the
 * workspace any argument (AGENT_ATTN_ERR_ALIAS); B*N*C*4 and 3*C*C*4 below
 * 2^31 bytes (AGENT_ATTN_ERR_UNSUPPORTED).  workspace: at least
 * agent_attn_module_workspace_bytes(...) bytes, 256-byte aligned, whose
 * first AGENT_ATTN_SYNC_BYTES bytes must be zero before its first use and
 * are left zero by every call (as for agent_attn_forward_ws).  Other
 * validation and errors as agent_attn_forward_ws; the call allocates
 * nothing. */
int agent_attn_module_forward(const void* x, const void* w_qkv,
                              const float* b_qkv, const void* w_out,
                              const float* b_out, const void* agents,
                              const float* bias_agg, const float* bias_bcast,
                              const float* dwc_weight, const float* dwc_bias,
                              void* y, int B, int H, int h, int w, int d,
                              int s, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Scratch bytes agent_attn_backward needs for these sizes (0 for invalid
 * sizes or an empty batch). */
size_t agent_attn_backward_workspace_bytes(int B, int H, int h, int w, int d,
                                           int s, int dtype);

/* Backward pass of the operator (agent_attn_forward): the gradients of a
 * loss L through O = softmax(scale Q A^T) softmax(scale A K^T) V, given
 * dout = dL/dO (source: "Agent Attention: On the Integration of Softmax and
 * Linear Attention", §4: two Softmax attentions, whose gradients follow
 * by the chain rule; §6: A = f(Q), the pooling, whose gradient spreads each
 * agent's gradient evenly over the tokens of its window).
 *   dq, dk, dv : outputs, [B, H, N, d] of dtype, dense;
 *   agents     : NULL (pooled from q: dq then includes the pooling's share),
 *                or the caller's agents [B, H, s*s, d], whose gradient goes
 *                to dagents [B, H, s*s, d] of dtype (required then, else
 *                ignored).
 * The forward is recomputed inside (nothing is saved between the calls).
 * Arithmetic: float32 for float32 tensors; for 16-bit tensors, matrix-core
 * products accumulating in float32 whose non-exact operands (agents, V_A,
 * dV_A, probabilities, score gradients) enter as pairs of 16-bit values where
 * rounding would cancel.  More than 64 agents run in chunks of 64 whose
 * contributions to dq, dk and dv are summed in float32 in a fixed order (the
 * results are deterministic).
 * workspace: at least
 * agent_attn_backward_workspace_bytes(...) bytes, 256-byte aligned, contents
 * free.  Outputs may not overlap any argument, nor the workspace any tensor
 * (AGENT_ATTN_ERR_ALIAS).  Validation and errors otherwise as
 * agent_attn_forward_ws; the call allocates nothing. */
int agent_attn_backward(const void* q, const void* k, const void* v,
                        const void* dout, const void* agents, void* dq,
                        void* dk, void* dv, void* dagents, int B, int H, int h,
                        int w, int d, int s, float scale, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Step 1 alone: agents_f32 [B, H, s*s, d] (float32) = 2-D average pool of q. */
int agent_attn_pool(const void* q, float* agents_f32, int B, int H, int h,
                    int w, int d, int s, int dtype, void* stream);

/* Scratch bytes that agent_attn_aggregate needs for these sizes. */
size_t agent_attn_aggregate_workspace_bytes(int B, int H, int N, int d,
                                            int n_agents, int dtype);

/* Step 2 alone: agent_values_f32 [B, H, n_agents, d] (float32) =
 * softmax(scale * agents_f32 k^T) v, with k, v [B, H, N, d] of `dtype`.
 * Any 1 <= n_agents <= 256. */
int agent_attn_aggregate(const float* agents_f32, const void* k, const void* v,
                         float* agent_values_f32, int B, int H, int N, int d,
                         int n_agents, float scale, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Step 3 alone: out [B, H, N, d] (`dtype`) =
 * softmax(scale * q agents_f32^T) agent_values_f32. */
int agent_attn_broadcast(const void* q, const float* agents_f32,
                         const float* agent_values_f32, void* out, int B,
                         int H, int N, int d, int n_agents, float scale,
                         int dtype, void* stream);

/* Bits of the fault word that fused launches leave in their workspace. */
#define AGENT_ATTN_FAULT_BARRIER 1 /* a workgroup barrier gave up waiting */
#define AGENT_ATTN_FAULT_XCD 2     /* a workgroup ran off its planned XCD */

/* Waits for the work on `stream`, then reads and clears the fault word of
 * `workspace` (a workspace given to agent_attn_forward_ws), or of the
 * library's scratch of the current device when workspace is NULL.  *faults
 * receives 0 when every forward launched on it since the last read ran
 * normally; otherwise a set of AGENT_ATTN_FAULT_* bits, and the outputs of
 * those launches are not valid.  Device-side waits are bounded, so a fault
 * ends the launch instead of hanging it.  Returns AGENT_ATTN_ERR_NULL when
 * faults is NULL, AGENT_ATTN_ERR_HIP when a HIP call fails. */
int agent_attn_read_faults(void* workspace, void* stream, int* faults);

/* Sets how many times a workgroup polls at a group barrier before it gives
 * up (default 1 << 20 polls, about a second) and returns the previous value;
 * a negative argument only returns it.  Applies to forwards enqueued
 * afterwards by this process.  A launch whose wait gives up sets
 * AGENT_ATTN_FAULT_BARRIER in its fault word and ends normally, so a small
 * value makes that path testable from the host. */
long agent_attn_set_wait_limit(long polls);

/* Frees the library's cached per-device scratch buffers. */
void agent_attn_release(void);

/* Static description of a status code. */
const char* agent_attn_status_string(int status);

/* Message describing the calling thread's last failed call ("" if none). */
const char* agent_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AGENT_ATTN_H_ */
