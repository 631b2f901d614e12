/*
 * loglinear.h — C ABI of the MI355X (gfx950) log-linear attention library.
 *
 * The operator (page "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性
 * 复杂度注意力机制", sections 并行形式 and 与已有模型的组合):
 *
 *     O = (Q K^T ⊙ M^S ⊙ M^H) V,
 *     M^H[t,s] = lambda[t, level(t,s)],   M^S[t,s] = exp(cum[t] - cum[s]),  s <= t,
 *
 * where level(t,s) is the Fenwick-bucket level of key s seen from query t
 * (section 层级判定算法; 0 for s == t) and cum is the inclusive prefix sum of
 * log_a (the Mamba-2 scalar decay).  No softmax and no 1/sqrt(dk) scale.
 *
 * Common conventions
 *   - Every tensor pointer is a DEVICE pointer to row-major, contiguous memory
 *     owned by the caller.  Nothing is retained after a call returns.
 *   - q, k, v, lambda, out and the gradient buffers of the forward, prefill
 *     and backward calls, and the decode step's states and out, must be
 *     16-byte aligned (the kernels move them in 16-byte vectors; device
 *     allocations are), else LL_ERR_SHAPE.  log_a, t and the decode step's
 *     q, k, v, log_a and lambda (read one element at a time) may sit anywhere.
 *   - Calls are asynchronous on `stream` (a hipStream_t, NULL = the null stream)
 *     and return once the work is enqueued.  No host/device synchronisation.
 *   - Return value: LL_OK (0) or a negative status; loglinear_strerror() gives
 *     its text.  Argument errors are detected on the host before any HIP call,
 *     leave all buffers untouched, and need no GPU.
 *   - Results are deterministic: no atomics, fixed reduction order.
 *   - `out` must not alias any input.
 *   - L = loglinear_num_levels(T) = bit_length(T-1) + 1 lambda levels.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16_t storage).
 */
#ifndef LOGLINEAR_H
#define LOGLINEAR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum loglinear_status {
  LL_OK = 0,
  LL_ERR_NULL = -1,        /* a required pointer is NULL                       */
  LL_ERR_SHAPE = -2,       /* a size is negative, inconsistent or out of range */
  LL_ERR_UNSUPPORTED = -3, /* valid sizes that this build has no kernel for    */
  LL_ERR_HIP = -4,         /* a HIP runtime call (launch / allocation) failed  */
  LL_ERR_WORKSPACE = -5    /* caller workspace too small                       */
};

enum loglinear_dtype { LL_BF16 = 0, LL_F32 = 1 };

/* Sweep kernel selection (loglinear_fwd_opts.kernel). */
enum loglinear_kernel {
  LL_KERNEL_AUTO = 0,           /* register-state kernel where it applies, else LDS-state */
  LL_KERNEL_LDS_STATE = 1,      /* bucket states in LDS, 16 dv columns per workgroup; all shapes */
  LL_KERNEL_REGISTER_STATE = 2, /* bucket states in registers, 64 dv columns per workgroup;
                                   bf16, C = 64, 64 < dk <= 128, dv % 64 == 0,
                                   ceil(T / 64) <= 1024 */
  LL_KERNEL_WIDE = 3            /* bucket states in registers, all dv columns of a segment in
                                   one workgroup, each wave over the whole of dk; bf16,
                                   C = 64, 64 < dk <= 128, dv = 128, ceil(T / 64) <= 256 */
};

/* Number of lambda levels for sequence length T >= 1: bit_length(T-1) + 1
 * (T = 64 -> 7, 2048 -> 12, 16384 -> 15, 65536 -> 17).  Returns 0 for T < 1. */
int loglinear_num_levels(int T);

/*
 * Forward, bf16 inputs (the performance path).
 *   q, k   : [B, H, T, dk]  bf16
 *   v      : [B, H, T, dv]  bf16
 *   log_a  : [B, H, T]      fp32, per-token log decay (0 = no decay)
 *   lambda : [B, H, T, L]   fp32, level weights lambda[t, l]
 *   out    : [B, H, T, dv]  fp32, written completely
 *   C      : chunk size of the chunkwise algorithm (page above, section
 *            训练：分块并行扫描算法): pairs inside one C-token chunk (levels
 *            <= log2 C) are computed densely, all other levels through
 *            chunk states.  C in {16, 32, 64}.
 * Sizes: B, H, T >= 0 (any zero -> nothing to do, LL_OK, pointers unchecked);
 * T need not be a multiple of C (the last chunk is ragged);
 * dk a multiple of 16 in [16, 128]; dv a multiple of 16 in [16, 1024].
 * Scratch: allocated stream-ordered (hipMallocAsync) on `stream` and freed
 * the same way; allocation failure returns LL_ERR_HIP.
 */
int loglinear_fwd(const void* q, const void* k, const void* v, const float* log_a,
                  const float* lambda, float* out, int B, int H, int T, int dk, int dv,
                  int C, void* stream);

/* Forward with fp32 q, k, v (fp32 matrix-core arithmetic throughout).  Same
 * contract as loglinear_fwd otherwise. */
int loglinear_fwd_f32(const float* q, const float* k, const float* v, const float* log_a,
                      const float* lambda, float* out, int B, int H, int T, int dk, int dv,
                      int C, void* stream);

/*
 * Decode states: a HOST struct describing a caller-owned DEVICE buffer
 *   data : [N, H, L, dk, dv] fp32, row-major (dv fastest).
 * Slot l holds the level-l state S^(l) = sum over the level-l bucket of
 * decay * k v^T, stored k-major (dk x dv) — the transpose of the pages' v k^T.
 */
typedef struct {
  float* data;
  int N, H, L, dk, dv;
} loglinear_states;

/*
 * Options for loglinear_fwd_ex.
 *   dtype        : LL_BF16 or LL_F32 (type of q, k, v).
 *   seg_log2     : -1 = automatic.  Otherwise the sequence is processed in
 *                  segments of 2^seg_log2 chunks (0..12); states of levels that
 *                  span whole segments are built by a separate segment pass.
 *                  Changes only the rounding order, never the result's
 *                  definition; exposed so every path can be exercised at small T.
 *   kernel       : a loglinear_kernel value; an explicit choice that does not
 *                  apply to the sizes returns LL_ERR_UNSUPPORTED.
 *   workspace    : NULL = allocate stream-ordered on `stream`; otherwise a
 *                  device buffer of at least loglinear_fwd_workspace_size()
 *                  bytes, 256-byte aligned (else LL_ERR_WORKSPACE), owned by
 *                  the caller, not used by any concurrent call.
 *   workspace_bytes : size of `workspace`.
 *   phase_events : NULL, or 4 caller-created hipEvent_t recorded on `stream`
 *                  before the segment-state kernel, before the node kernel,
 *                  before the sweep kernel and after it (kernels that a plan
 *                  does not need are skipped, their events still recorded), so
 *                  a caller can time each kernel of one call.
 *   final_states : NULL, or a states buffer (see loglinear_states) that
 *                  receives the per-level decode states at position T-1, as
 *                  loglinear_prefill describes.
 *   qk_heads     : 0 (or H) = every head has its own q and k.  Otherwise the
 *                  number Hk of q/k heads, a divisor of H: q and k are
 *                  [B, Hk, T, dk] and head h uses q/k head h / (H / Hk) — the
 *                  multi-value layout (MVA) of log-linear Mamba-2, where the
 *                  pages' kernel benchmark shares q and k across heads ("Log-
 *                  Linear Attention" article, experiment setup).  v, log_a,
 *                  lambda and out stay per head.  A value that does not divide
 *                  H gives LL_ERR_SHAPE.
 */
typedef struct {
  int dtype;
  int seg_log2;
  int kernel;
  void* workspace;
  size_t workspace_bytes;
  void* const* phase_events;
  const loglinear_states* final_states;
  int qk_heads;
} loglinear_fwd_opts;

int loglinear_fwd_ex(const void* q, const void* k, const void* v, const float* log_a,
                     const float* lambda, float* out, int B, int H, int T, int dk, int dv,
                     int C, const loglinear_fwd_opts* opts, void* stream);

/*
 * Prefill: the forward of loglinear_fwd, plus the decode states that continue
 * the sequence (page above, sections 循环形式与输出计算 and 解码：基于 lssb 的状态更新).
 *   states : a states buffer with N = B, the same H, dk, dv, and
 *            L >= loglinear_num_levels(T) (more levels are allowed, so decoding
 *            can run past 2^(L_T - 1) tokens).  On return level l holds
 *            S^(l) = sum over the level-l Fenwick bucket of query T-1 of
 *            exp(cum[T-1] - cum[s]) k_s v_s^T, and levels with no bucket at
 *            T-1 hold 0: exactly the states a loglinear_decode_step at t = T
 *            expects on entry.  Every element of the buffer is written.
 * Other arguments, sizes and errors as loglinear_fwd; a states buffer whose
 * N, H, dk or dv differ from the forward's, or whose L is too small, gives
 * LL_ERR_SHAPE.  The bf16 register-state path keeps the inter-chunk bucket
 * states in fp16 with power-of-two scales, so its states carry the forward's
 * rounding (about 1e-3 of their RMS).
 */
int loglinear_prefill(const void* q, const void* k, const void* v, const float* log_a,
                      const float* lambda, float* out, const loglinear_states* states, int B,
                      int H, int T, int dk, int dv, int C, void* stream);

/* Same as loglinear_prefill with fp32 q, k, v. */
int loglinear_prefill_f32(const float* q, const float* k, const float* v, const float* log_a,
                          const float* lambda, float* out, const loglinear_states* states,
                          int B, int H, int T, int dk, int dv, int C, void* stream);

/*
 * Backward: gradients of sum(out * dout) with respect to every input of
 * loglinear_fwd (page above, sections 并行形式 and 与已有模型的组合 define the
 * operator being differentiated; 训练：分块并行扫描算法 the chunking reused here).
 *   q, k, v, log_a, lambda : the forward's inputs (bf16 q, k, v)
 *   out    : [B, H, T, dv] fp32, the forward's output for these inputs, or
 *            NULL: the gradients do not read it (d log_a takes dO_t . O_t as
 *            sum_l lambda[t,l] grad_lambda[t,l], the same sum); kept in the
 *            signature so a caller may pass what it has
 *   dout   : [B, H, T, dv] fp32, gradient with respect to out
 *   grad_q, grad_k : [B, H, T, dk] fp32;  grad_v : [B, H, T, dv] fp32
 *   grad_log_a : [B, H, T] fp32;  grad_lambda : [B, H, T, L] fp32
 * All outputs are written completely (grad_lambda is 0 for levels a row never
 * reaches).  Sizes and C as loglinear_fwd; additionally at most 4096 chunks,
 * and the staging and per-level states of one workgroup must fit in LDS (bf16
 * with C = 64 and dk = dv = 128: up to 1024 chunks), else LL_ERR_UNSUPPORTED.
 * Scratch (per-slice partial sums of grad_lambda, (dk/16) * B * H * T *
 * bit_length(N-1) floats, and B * H * T doubles) is allocated stream-ordered
 * on `stream`.
 * Arithmetic: with bf16 inputs and C = 64 (dk, dv multiples of 32 up to 128,
 * at most 256 chunks) bf16 matrix cores with the fp32 operands (dO, masked
 * scores, level states) split into bf16 hi + lo, ~1e-3 of each gradient's RMS
 * at worst; otherwise fp32 matrix-core instructions.  No atomics, so the
 * results are deterministic.
 */
int loglinear_bwd(const void* q, const void* k, const void* v, const float* log_a,
                  const float* lambda, const float* out, const float* dout, float* grad_q,
                  float* grad_k, float* grad_v, float* grad_log_a, float* grad_lambda, int B,
                  int H, int T, int dk, int dv, int C, void* stream);

/* Same as loglinear_bwd with fp32 q, k, v. */
int loglinear_bwd_f32(const float* q, const float* k, const float* v, const float* log_a,
                      const float* lambda, const float* out, const float* dout, float* grad_q,
                      float* grad_k, float* grad_v, float* grad_log_a, float* grad_lambda, int B,
                      int H, int T, int dk, int dv, int C, void* stream);

/*
 * loglinear_bwd with the element type as an argument (dtype: LL_BF16 or LL_F32)
 * and q / k shared by groups of heads (qk_heads as in loglinear_fwd_opts):
 * q, k, grad_q and grad_k are then [B, Hk, T, dk], and grad_q / grad_k hold
 * the sum over the H / Hk heads of each group (summed in head order after
 * per-head gradients in stream-ordered scratch of 2 * B * H * T * dk floats).
 * qk_heads = 0 is exactly loglinear_bwd / _f32.
 */
int loglinear_bwd_ex(const void* q, const void* k, const void* v, const float* log_a,
                     const float* lambda, const float* out, const float* dout, float* grad_q,
                     float* grad_k, float* grad_v, float* grad_log_a, float* grad_lambda, int B,
                     int H, int T, int dk, int dv, int C, int dtype, int qk_heads, void* stream);

/*
 * Level weights from the hidden state (page above, section 循环形式与输出计算:
 * a per-head linear projection of the token's hidden representation, made
 * non-negative; the map is read as softplus):
 *   lambda[b, h, t, l] = softplus(sum_d x[b, t, d] * W[h*L + l, d] + bias[h*L + l])
 * with softplus(z) = log(1 + exp(z)), fused into one kernel (matrix cores,
 * fp32 accumulation; bias, softplus and the [B, H, T, L] layout applied before
 * the only store).
 *   x      : [B, T, D] DEVICE, LL_BF16 (bf16 bits) or LL_F32 per `dtype`
 *   W      : [H*L, D] DEVICE, same type as x; row h*L + l is head h, level l
 *   bias   : [H*L] fp32 DEVICE, or NULL for none
 *   lambda : [B, H, T, L] fp32 DEVICE output (L = loglinear_num_levels(T)
 *            for use with loglinear_fwd; any 1 <= L <= 31 is accepted)
 * D must be a multiple of 8 (bf16) or 4 (fp32) and x, W 16-byte aligned, else
 * LL_ERR_SHAPE; D or H*L above 2^20 give LL_ERR_UNSUPPORTED.  B = 0 or T = 0
 * is a no-op.  Asynchronous on `stream`; allocates nothing.
 */
int loglinear_lambda_proj(const void* x, const void* W, const float* bias, float* lambda, int B,
                          int T, int D, int H, int L, int dtype, void* stream);

/*
 * Gradient of loglinear_lambda_proj (same page and section) for a training
 * step: with z = x W^T + bias, m = b*T + t and n = h*L + l,
 *   dz[m, n]     = grad_lambda[b, h, t, l] * sigmoid(z[m, n])
 *   grad_x       = dz W            [B, T, D]  fp32
 *   grad_W       = dz^T x          [H*L, D]   fp32
 *   grad_bias[n] = sum_m dz[m, n]  [H*L]      fp32 (NULL: not computed)
 * sigmoid(z) is recovered from the forward's output as 1 - exp(-lambda), so
 * the bias is not needed.
 *   x, W        : as for loglinear_lambda_proj (dtype LL_BF16 or LL_F32)
 *   lambda      : [B, H, T, L] fp32, the forward's output
 *   grad_lambda : [B, H, T, L] fp32
 * All DEVICE pointers; outputs are overwritten.  Arithmetic: fp32 inputs on
 * fp32 matrix cores; bf16 inputs on bf16 matrix cores with dz split into bf16
 * hi + lo (each product term within 2^-16 of the fp32 one); fp32
 * accumulation, no atomics (bitwise repeatable).  Stream-ordered scratch
 * (allocated and released on `stream`): for bf16 inputs with D % 8 == 0 and
 * 16-byte aligned x, W, dz as two bf16 arrays of B*T rows of H*L rounded up to
 * 128, per-64-token column sums and the dW split partials; otherwise B*T*H*L
 * floats for dz plus the dW split partials.  B*T = 0 writes zeros
 * to grad_W and grad_bias.  Errors: bad dtype or sizes (L outside 1..31)
 * LL_ERR_SHAPE; D > 2^20, H*L > 2^16 or B*T >= 2^31 LL_ERR_UNSUPPORTED; a NULL
 * required pointer LL_ERR_NULL.
 */
int loglinear_lambda_proj_bwd(const void* x, const void* W, const float* lambda,
                              const float* grad_lambda, float* grad_x, float* grad_W,
                              float* grad_bias, int B, int T, int D, int H, int L, int dtype,
                              void* stream);

/* Workspace bytes loglinear_fwd_ex needs for these sizes (0 if none); seg_log2
 * as in loglinear_fwd_opts.  Returns (size_t)-1 for invalid sizes. */
size_t loglinear_fwd_workspace_size(int B, int H, int T, int dk, int dv, int C, int seg_log2);

/*
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, arithmetic and result as loglinear_fwd (bf16
 * q, k, v; the same kernels and launch plan, so the output is bitwise equal),
 * but the workspace lives in a static device array of
 * LOGLINEAR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends, and the call allocates and frees nothing.
 *   - Sizes whose workspace (loglinear_fwd_workspace_size with seg_log2 = -1)
 *     exceeds LOGLINEAR_NOALLOC_SCRATCH_BYTES give LL_ERR_WORKSPACE, checked on
 *     the host before any HIP call.  The automatic plans at dk = dv = 128
 *     need at most ~37 MiB (B=2, H=16, T=16384: 34 MiB; B=1, H=16, T=65536:
 *     37 MiB); wide dv with small C can need more.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on a
 *     GPU (other streams, other host threads) race and must be serialised by
 *     the caller; calls on one stream are ordered and safe.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current; a failure is LL_ERR_HIP.
 * Other errors as loglinear_fwd.
 */
#define LOGLINEAR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int loglinear_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_a,
                          const float* lambda, float* out, int B, int H, int T, int dk, int dv,
                          int C, void* stream);

/*
 * One O(log T) decode step for N sequences x H heads (page above, section
 * 解码：基于 lssb 的状态更新; slide 21 of "論文紹介：Log Linear Attention").
 *   states : on entry S_{t-1} of every (sequence, head), levels dead at t-1
 *            equal to 0; on return S_t, updated in place.  With m = lssb(t)
 *            (index of the lowest set bit): level m+1 <- a_t * sum_{l<=m} S^l,
 *            levels 1..m <- 0, levels > m+1 that are live <- a_t * S^l, level
 *            0 <- k_t v_t^T; a_t = exp(log_a).  At t = 0 all levels are
 *            cleared before level 0 is written.  Levels above m+1 that are
 *            dead at t are neither read nor written.
 *   q, k   : [N, H, dk] bf16;  v : [N, H, dv] bf16
 *   log_a  : [N, H] fp32;  lambda : [N, H, L] fp32
 *   t      : [N] int32 DEVICE array, position of the incoming token
 *   out    : [N, H, dv] fp32, o = sum_l lambda[l] q^T S_t^l
 * Valid t: 0 <= t < 2^(L-1).  A t outside that range cannot be checked on the
 * host: that sequence's out rows are set to NaN and its states left unchanged.
 * Sizes: dk, dv multiples of 4 in [4, 1024]; 1 <= L <= 31; N, H >= 0.
 */
int loglinear_decode_step(const loglinear_states* states, const void* q, const void* k,
                          const void* v, const float* log_a, const float* lambda,
                          const int* t, float* out, void* stream);

/* Same as loglinear_decode_step with fp32 q, k, v. */
int loglinear_decode_step_f32(const loglinear_states* states, const float* q,
                              const float* k, const float* v, const float* log_a,
                              const float* lambda, const int* t, float* out, void* stream);

/*
 * loglinear_decode_step with the element type as an argument (dtype: LL_BF16
 * or LL_F32) and q / k shared by groups of heads (qk_heads as in
 * loglinear_fwd_opts): q and k are [N, Hk, dk]; states, v, log_a, lambda and
 * out stay per head.  qk_heads = 0 is exactly loglinear_decode_step / _f32.
 */
int loglinear_decode_step_ex(const loglinear_states* states, const void* q, const void* k,
                             const void* v, const float* log_a, const float* lambda,
                             const int* t, float* out, int dtype, int qk_heads, void* stream);

/*
 * Log-linear Gated DeltaNet forward.  The pages lift Gated DeltaNet with the
 * same Fenwick hierarchy as Mamba-2 (page "论文阅读：Log-Linear Attention — 基于
 * Fenwick 树与层次矩阵的对数线性复杂度注意力机制", section 与已有模型的组合; page
 * "算力终结者来了！华人天团「降维打击」注意力瓶颈，AI狂飙进对数时代", section
 * 对Mamba-2和门控DeltaNet的对数线性推广) but print no delta rule; this call
 * takes the published gated delta rule, with k-major states,
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 * and weights each pair of its unrolled form by the level weight:
 *     o_t = sum_{s<=t} lambda[t, level(t,s)] beta_s q_t^T A_t...A_{s+1} k_s v_s,
 *     A_r = alpha_r (I - beta_r k_r k_r^T),  alpha_r = exp(log_alpha[r]).
 * With lambda = 1 on every level this is Gated DeltaNet itself.
 *   q, k      : [B, H, T, dk]  bf16 (dtype LL_BF16) or fp32 (LL_F32); the
 *               delta rule expects unit-norm keys (not checked)
 *   v         : [B, H, T, dv]  same dtype as q
 *   log_alpha : [B, H, T] fp32 (<= 0),  beta : [B, H, T] fp32 (in [0, 1])
 *   lambda    : [B, H, T, L] fp32,  out : [B, H, T, dv] fp32, written completely
 * Chunks of 64 tokens; arithmetic in fp32 (matrix cores).  dk in {64, 128},
 * dv a multiple of 16, ceil(T / 64) <= 8192 chunks at dk = 128 (else
 * LL_ERR_UNSUPPORTED; the bucket states of a 16-column slice live in LDS).
 * workspace: NULL (the call allocates and frees it on `stream`) or at least
 * loglinear_gdn_workspace_size() bytes of device memory, 256-byte aligned,
 * else LL_ERR_WORKSPACE; its contents on entry do not matter.  It holds
 * 4 (3 dk + 128) * 64 bytes per chunk (~128 KiB at dk = 128).
 */
int loglinear_gdn_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* lambda, float* out, int B, int H, int T, int dk,
                      int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One O(log T) decode step of log-linear Gated DeltaNet (the delta rule as in
 * loglinear_gdn_fwd; the decode rule of the page above, section 解码：基于
 * lssb 的状态更新, with the transition in place of the scalar decay) for N
 * sequences x H heads.
 *   states : as loglinear_decode_step (k-major [N, H, L, dk, dv] fp32, levels
 *            dead at t-1 equal to 0), updated in place: with m = lssb(t),
 *            level m+1 <- A_t sum_{l<=m} S^l, live levels above m+1 <- A_t S^l,
 *            levels 1..m <- 0, level 0 <- beta k v^T, where A_t = alpha
 *            (I - beta k k^T), alpha = exp(log_alpha).  At t = 0 every level
 *            is cleared before level 0 is written.  Levels above m+1 that are
 *            dead at t are neither read nor written.
 *   q, k   : [N, H, dk], v : [N, H, dv]  (dtype LL_BF16 or LL_F32)
 *   log_alpha, beta : [N, H] fp32;  lambda : [N, H, L] fp32
 *   t      : [N] int32 DEVICE array, position of the incoming token
 *   out    : [N, H, dv] fp32, o = sum_l lambda[l] q^T S_t^l
 * Valid t: 0 <= t < 2^(L-1); other t give NaN output rows and leave that
 * sequence's states unchanged.  Sizes: dk in {64, 128}, dv a multiple of 4 in
 * [4, 1024] (else LL_ERR_UNSUPPORTED / LL_ERR_SHAPE); 1 <= L <= 31.
 */
int loglinear_gdn_decode_step(const loglinear_states* states, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* beta,
                              const float* lambda, const int* t, float* out, int dtype, void* stream);

/*
 * loglinear_gdn_fwd plus the decode states at position T-1 (prefill ->
 * decode hand-off, page above, section 解码：基于 lssb 的状态更新):
 *   states   : [B, H, states_L, dk, dv] fp32 DEVICE, 16-byte aligned, written
 *              completely: level l holds sum over the level-l Fenwick bucket of
 *              T-1 of A_{T-1}...A_{s+1} beta_s k_s v_s^T (k-major); levels with
 *              no bucket at T-1 hold 0.  These are exactly the states a
 *              loglinear_gdn_decode_step at t = T continues from.
 *   states_L : levels of the states tensor, L <= states_L <= 31 (else
 *              LL_ERR_SHAPE); NULL states with non-empty sizes: LL_ERR_NULL.
 * Other arguments, sizes and errors as loglinear_gdn_fwd.
 */
int loglinear_gdn_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* lambda, float* out, float* states,
                          int states_L, int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes of loglinear_gdn_fwd for these sizes; (size_t)-1 if the
 * sizes are invalid or unsupported. */
size_t loglinear_gdn_workspace_size(int B, int H, int T, int dk, int dv);

/*
 * Test export: lev[t*T + s] = level(t, s) for s <= t and -1 for s > t (int8,
 * DEVICE buffer of T*T bytes), computed on the GPU with the same device
 * helper the kernels use (section 层级判定算法).  1 <= T <= 8192.
 */
int loglinear_level_table(signed char* lev, int T, void* stream);

/* Static text for a status code. */
const char* loglinear_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LOGLINEAR_H */
