/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The operation (from the "K3 notes" pages, section "KDA 递归核心", subsection
 * "逐步公式"): for every sequence b and value head hv, with state
 * S[K][V] (key rows, value columns), for each token t in order
 *
 *     S_dec = exp(g_t) (.) S_{t-1}            per-key-channel decay of row kappa
 *     r_t   = v_t - k_t . S_dec               delta-rule residual
 *     S_t   = S_dec + (beta_t k_t) outer r_t  rank-1 write
 *     o_t   = (1/sqrt(K)) q_t . S_t           read (includes token t's own write)
 *
 * g_t is the gate ("K3 notes", section "Gate 激活"): with
 * input = g_raw + dt_bias[hv][kappa] and rate = exp(A_log[hv]),
 *     KDA_GATE_SAFE     : g = lower_bound * sigmoid(rate * input)   in [lower_bound, 0]
 *     KDA_GATE_STANDARD : g = -rate * softplus(input)               in (-inf, 0]
 *     KDA_GATE_NONE     : g = g_raw  (the caller passes the log-decay itself)
 * GVA: value head hv reads query/key head h = hv / (HV / H) (q and k are
 * shared by HV/H consecutive value heads, as repeat_interleave would do).
 *
 * Per-head gates: KDA_GATE_PER_HEAD may be OR-ed into any gate kind.  The gate
 * is then one scalar per (token, value head), shared by all key channels: the
 * scalar retain gate of Gated DeltaNet ("DeltaNet family" page, "Gated
 * DeltaNet"), of which KDA's channel-wise gate is the generalisation.  g_raw
 * loses its K axis ([..., HV] instead of [..., HV, K]) and dt_bias is [HV];
 * the same activation formulas apply.  DeltaNet itself is KDA_GATE_NONE with
 * g_raw = 0.
 *
 * Two schedules of the same recurrence ("DeltaNet family" page, sections on
 * the fused recurrent kernel and on chunkwise KDA): kda_chunk_fwd processes a
 * whole sequence chunk by chunk (intra-chunk dependencies resolved by a
 * lower-triangular solve, the state carried between chunks); kda_recurrent_fwd
 * runs the tokens of a call one by one with the state kept on chip, and
 * kda_recurrent_step advances a state held in HBM by one token.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major memory
 *    with the shapes given below, aligned to 16 bytes (4 bytes suffice for
 *    g_raw and dt_bias with KDA_GATE_PER_HEAD).  The caller owns every
 *    buffer; the library allocates nothing and keeps no global state; every
 *    entry point may be called from several host threads and streams.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 *    default stream).  Nothing synchronises the host.  Input buffers must stay
 *    valid, and outputs unread, until the stream reaches the enqueued work.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-KDA_OK status means nothing was enqueued (except KDA_ERR_HIP, which
 *    reports a failed launch).  No entry point aborts or throws.
 *  - The read scale is fixed at 1/sqrt(K).
 *  - Outputs must not overlap inputs, except where stated.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, HV % H != 0, ... */
  KDA_ERR_UNSUPPORTED = 2, /* valid but not built: head size, chunk size */
  KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KDA_ERR_HIP = 4,         /* a kernel launch failed */
  KDA_ERR_SCRATCH = 5      /* kda_chunk_fwd_split_noalloc: the workspace this call needs
                              exceeds the library's fixed scratch */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

typedef enum {
  KDA_GATE_STANDARD = 0,
  KDA_GATE_SAFE = 1,
  KDA_GATE_NONE = 2,
  KDA_GATE_PER_HEAD = 16 /* flag, OR-ed into one of the three kinds above */
} kda_gate_kind;

typedef struct ihipStream_t* kda_stream_t; /* the same type as hipStream_t */

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status s);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

/*
 * kda_gate -- gate activation ("K3 notes", "Gate 激活": two-gate table and the
 * kda_gate_reference panel), optionally followed by the chunk-local inclusive
 * prefix sum of the log-decay ("DeltaNet family" page, chunkwise pipeline:
 * the cumulative log-decay whose differences give D_{j+1:i}).
 *
 *   g_raw   [B, T, HV, K] float32 ([B, T, HV] with KDA_GATE_PER_HEAD)
 *   A_log   [HV] float32                 rate = exp(A_log[hv])
 *   dt_bias [HV, K] float32 or NULL      NULL means zero bias ([HV] per head)
 *   gate, lower_bound                    lower_bound < 0 required for KDA_GATE_SAFE
 *   chunk_size  0: g_out = g;  C > 0: g_out[t] = sum of g over the tokens of
 *               t's chunk up to and including t (chunks of C tokens from t = 0)
 *   g_out   the shape of g_raw, float32 (may alias g_raw)
 * Any K >= 1 is accepted (K is ignored with KDA_GATE_PER_HEAD).  B or T equal
 * to 0 is a no-op.
 */
kda_status kda_gate(const float* g_raw, const float* A_log, const float* dt_bias,
                    kda_gate_kind gate, float lower_bound, int B, int T, int HV, int K,
                    int chunk_size, float* g_out, kda_stream_t stream);

/*
 * kda_chunk_fwd -- chunkwise-parallel forward over whole sequences ("DeltaNet
 * family" page, "Chunkwise KDA": temporary errors, causal triangular solve,
 * chunk-end state, chunk outputs), gate computed in-kernel from g_raw.
 *
 *   q, k          [B, T, H, K]   float32 or bfloat16 (qkv_dtype)
 *   v             [B, T, HV, V]  same dtype as q and k
 *   g_raw         [B, T, HV, K]  float32 ([B, T, HV] with KDA_GATE_PER_HEAD)
 *   beta          [B, T, HV]     float32
 *   A_log         [HV]           float32
 *   dt_bias       [HV, K]        float32 or NULL ([HV] with KDA_GATE_PER_HEAD)
 *   initial_state [B, HV, K, V]  float32, or NULL for zeros
 *   o             [B, T, HV, V]  float32 output
 *   final_state   [B, HV, K, V]  float32 output, or NULL; may alias initial_state
 *   chunk_size    16, 32 or 64, validated and otherwise unused: the kernel always
 *                 solves the chunk's lower-triangular system in its 16-token diagonal
 *                 blocks, carrying the coupling between blocks through the on-chip
 *                 state (block forward substitution, the "Chunkwise Triton pipeline"
 *                 section's 16-token diagonal blocks), so any accepted chunk size
 *                 gives the same result, bit for bit
 *   workspace     device scratch of kda_chunk_fwd_workspace_bytes(...) bytes, or
 *                 NULL when that size is 0
 * Supported head sizes: K == V in {16, 32, 64, 128}; HV % H == 0; HV * K <=
 * 2^24 (KDA_ERR_UNSUPPORTED beyond; the kernel addresses 16 tokens of one
 * tensor with 32-bit offsets).  T may be any length >= 0 (a ragged last chunk is
 * handled in-kernel); T == 0 copies the initial state (or zeros) to final_state.
 * Arithmetic: fp32 inputs run fp32 matrix products; bf16 inputs run bf16 MFMA
 * products with fp32 accumulation and split (hi + lo) operands where precision
 * needs them; the state is fp32 throughout.
 */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int chunk_size,
                                     kda_dtype qkv_dtype);

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                         const float* g_raw, const float* beta, const float* A_log,
                         const float* dt_bias, kda_gate_kind gate, float lower_bound,
                         const float* initial_state, float* o, float* final_state, int B, int T,
                         int H, int HV, int K, int V, int chunk_size, void* workspace,
                         size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_recurrent_step -- one decode token for every sequence ("DeltaNet family"
 * page, fused recurrent mode: decay, key prediction, residual, rank-1 write,
 * query read), the state updated in place in HBM.
 *
 *   q, k    [B, H, K]        float32 or bfloat16 (qkv_dtype)
 *   v       [B, HV, V]       same dtype
 *   g_raw   [B, HV, K]       float32 ([B, HV] with KDA_GATE_PER_HEAD)
 *   beta    [B, HV]          float32
 *   A_log   [HV], dt_bias [HV, K] or NULL, gate, lower_bound: as kda_gate
 *   state   [B, HV, K, V]    float32, read and overwritten with the new state
 *   o       [B, HV, V]       float32 output
 * Supported: K, V in {16, 32, 64, 128}; HV % H == 0.
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                              const float* g_raw, const float* beta, const float* A_log,
                              const float* dt_bias, kda_gate_kind gate, float lower_bound,
                              float* state, float* o, int B, int H, int HV, int K, int V,
                              kda_stream_t stream);

/*
 * kda_recurrent_fwd -- the fused recurrent schedule over T tokens per call
 * ("DeltaNet family" page, fused recurrent mode, which loops over time with the
 * state on chip): per (sequence, value head, value tile) the state tile is read
 * from initial_state once, advanced through the T tokens in registers, and
 * written to final_state once.  Meant for short prefills and multi-token
 * (speculative) decode, where the chunked path's fixed cost does not pay off;
 * the result equals T calls of kda_recurrent_step up to rounding.
 *
 *   q, k          [B, T, H, K]   float32 or bfloat16 (qkv_dtype)
 *   v             [B, T, HV, V]  same dtype
 *   g_raw         [B, T, HV, K]  float32 ([B, T, HV] with KDA_GATE_PER_HEAD)
 *   beta          [B, T, HV]     float32
 *   A_log, dt_bias, gate, lower_bound: as kda_gate
 *   initial_state [B, HV, K, V]  float32, or NULL for zeros
 *   o             [B, T, HV, V]  float32 output
 *   final_state   [B, HV, K, V]  float32 output, or NULL; may alias initial_state
 * Supported: K, V in {16, 32, 64, 128} (independently); HV % H == 0; any
 * T >= 0 (T == 0 copies the initial state, or zeros, to final_state).
 * Arithmetic is fp32 throughout (bf16 inputs are widened exactly).
 */
kda_status kda_recurrent_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const float* g_raw, const float* beta, const float* A_log,
                             const float* dt_bias, kda_gate_kind gate, float lower_bound,
                             const float* initial_state, float* o, float* final_state, int B,
                             int T, int H, int HV, int K, int V, kda_stream_t stream);

/*
 * kda_chunk_fwd_split -- the chunkwise forward as three stages with the entry
 * state of every chunk materialised ("DeltaNet family" page, "Chunkwise Triton
 * pipeline": an intra-chunk stage, one pass across chunks producing the
 * chunk-entry states h and the resolved values, and an output stage parallel
 * over chunks).  Only the middle stage is sequential over a sequence, and it
 * carries just two K x V products per chunk, so this schedule fills the GPU
 * where B * HV is too small for kda_chunk_fwd (one long sequence, few heads);
 * it also hands the caller the state at every chunk boundary.
 *
 *   arguments as kda_chunk_fwd, plus
 *   h             [B, HV, NC, K, V] float32 output, NC = ceil(T / chunk_size):
 *                 h[b, hv, c] is the state entering chunk c (h[.., 0] is the
 *                 initial state); NULL keeps h inside the workspace
 *   o             as kda_chunk_fwd, or NULL when h is given: then only the
 *                 states are produced (h and final_state) and the output
 *                 stage is skipped, as a training forward that keeps the
 *                 states for the backward would do
 *   workspace     device scratch of at least
 *                 kda_chunk_fwd_split_workspace_bytes(...) bytes, 16-byte aligned,
 *                 owned by the caller; its contents need not be initialised and
 *                 are meaningless afterwards
 * Supported: K == V in {16, 32, 64, 128}; chunk_size 16, 32 or 64; HV % H == 0;
 * T >= 0.  Arithmetic: fp32 matrix products with fp32 accumulation, except
 * that with bf16 inputs (and K, chunk_size >= 32) the state pass runs bf16 MFMA
 * products on split (hi + lo) operands; the state is fp32 throughout.  Three
 * kernels run in order on `stream`.  Returns KDA_ERR_WORKSPACE if the
 * workspace is missing or too small.
 */
size_t kda_chunk_fwd_split_workspace_bytes(int B, int T, int H, int HV, int K, int V,
                                           int chunk_size);

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* g_raw, const float* beta, const float* A_log,
                               const float* dt_bias, kda_gate_kind gate, float lower_bound,
                               const float* initial_state, float* o, float* final_state, float* h,
                               int B, int T, int H, int HV, int K, int V, int chunk_size,
                               void* workspace, size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_chunk_fwd_split_noalloc -- kda_chunk_fwd_split for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and arguments, minus
 * the workspace, which instead lives in a scratch array inside the library.
 *
 *   limit   the workspace kda_chunk_fwd_split_workspace_bytes(...) gives for
 *           the call must not exceed 64 MiB (67,108,864 bytes), else
 *           KDA_ERR_SCRATCH and nothing is enqueued.  For K = V = 128 and
 *           chunk 64 a (sequence, value head, chunk) triple takes 164 KiB, so
 *           e.g. 8 value heads x 3,136 tokens (49 chunks) fit, 3,200 do not.
 *   memory  the call allocates nothing and calls no allocating routine.  Each
 *           GPU the library runs on holds its own 64 MiB copy of the scratch
 *           from the first use until the process ends; its address is looked
 *           up once per device, on the first call made with that device
 *           current.  Nothing in it needs to start at zero.
 *   races   every call on one GPU shares that GPU's scratch: calls that may
 *           overlap in time on one device (different streams, or host threads
 *           enqueueing concurrently) must be ordered by the caller.  Calls on
 *           one stream are ordered by it.
 * Everything else as kda_chunk_fwd_split.
 */
kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v,
                                       kda_dtype qkv_dtype, const float* g_raw, const float* beta,
                                       const float* A_log, const float* dt_bias,
                                       kda_gate_kind gate, float lower_bound,
                                       const float* initial_state, float* o, float* final_state,
                                       float* h, int B, int T, int H, int HV, int K, int V,
                                       int chunk_size, kda_stream_t stream);

/*
 * kda_bwd -- gradients of the KDA forward (kda_chunk_fwd and its siblings
 * compute the same function) for a loss L(o, S_T), given dL/do and dL/dS_T.
 * The "K3 notes" ledger lists a backward derivation ("反向传播推导") whose
 * text the pages do not keep; these are the reverse-mode gradients of the
 * four-step update of section "KDA 递归核心" and of the gate of section
 * "Gate 激活", for one (sequence, value head) with dS the running dL/dS_t,
 * token by token from the last (s = 1/sqrt(K), alpha = exp(g)):
 *     dS += s q_t do_t^T,  dq_t = s S_t do_t,  a = dS^T k_t,  dr = beta_t a,
 *     dv_t = dr,  dbeta_t = a . r_t,  dk_t = beta_t dS r_t - Sd_t dr,
 *     dSd = dS - k_t dr^T,  dg_t = rowsum(dSd (.) Sd_t),  dS <- diag(alpha_t) dSd
 * then the gate's chain rule: dg_raw = dg dg/dx with x = g_raw + dt_bias, and
 * the sums of dg dg/dx (dt_bias) and dg dg/dA_log (A_log) over sequences and
 * tokens.  Under the none gate dt_bias and A_log do not enter the forward and
 * their gradients are zero.  Under GVA, dq and dk sum over the value heads
 * that read the same query/key head.
 *
 *   q, k, v, qkv_dtype, g_raw, beta, A_log, dt_bias, gate, lower_bound,
 *   initial_state        the forward's inputs, as kda_chunk_fwd (a per-channel
 *                        or, with KDA_GATE_PER_HEAD, a per-head gate)
 *   dout                 [B, T, HV, V]  float32, dL/do
 *   dfinal_state         [B, HV, K, V]  float32, dL/dS_T, or NULL for zero
 *   dq, dk               [B, T, H, K]   float32 outputs
 *   dv                   [B, T, HV, V]  float32 output
 *   dbeta                [B, T, HV]     float32 output
 *   dg_raw               [B, T, HV, K]  float32 output ([B, T, HV] with a
 *                                       per-head gate: the sum over the key
 *                                       channels the value is broadcast to)
 *   dA_log               [HV]           float32 output, or NULL to skip
 *   ddt_bias             [HV, K]        float32 output ([HV] with a per-head
 *                                       gate), or NULL to skip (with dt_bias
 *                                       NULL it is the gradient at a zero bias)
 *   dinitial_state       [B, HV, K, V]  float32 output (dL/dS_0), or NULL
 *   workspace            device scratch of at least kda_bwd_workspace_bytes(...)
 *                        bytes, 16-byte aligned, owned by the caller; per
 *                        16-token segment it holds the entering K x V state,
 *                        U = beta r, the segment's cumulative decays, three
 *                        16 x 16 matrices and a range flag, all written by
 *                        the forward pass the call runs first; its contents
 *                        are meaningless afterwards
 * Every output is overwritten (none needs initialising).  dq, dk, dg_raw,
 * dbeta, dA_log and ddt_bias are sums accumulated with fp32 atomics, so their
 * last bits can differ from run to run; dv and dinitial_state are written
 * once.  All pointers are device pointers; outputs must not alias inputs or
 * each other.
 * Supported: K == V in {32, 64, 128}; HV % H == 0; T >= 0; either gate
 * layout.  Arithmetic is fp32 throughout
 * (bf16 inputs widened exactly; the forward pass that writes the segment
 * states is kda_chunk_fwd's kernel on its fp32 products).  Several kernels
 * run in order on `stream`.  Returns KDA_ERR_WORKSPACE if the workspace is missing
 * or too small.
 */
size_t kda_bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V);

kda_status kda_bwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                   const float* g_raw, const float* beta, const float* A_log, const float* dt_bias,
                   kda_gate_kind gate, float lower_bound, const float* initial_state,
                   const float* dout, const float* dfinal_state, float* dq, float* dk, float* dv,
                   float* dbeta, float* dg_raw, float* dA_log, float* ddt_bias,
                   float* dinitial_state, int B, int T, int H, int HV, int K, int V,
                   void* workspace, size_t workspace_bytes, kda_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
