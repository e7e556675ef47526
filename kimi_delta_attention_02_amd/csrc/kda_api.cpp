// Host side of the C ABI declared in include/kda.h: argument validation,
// then one asynchronous kernel launch on the caller's stream.  Validation runs
// entirely on the host and returns before anything is enqueued.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kda.h"

namespace kda {
hipError_t launch_gate(const float* g_raw, const float* A_log, const float* dt_bias, int kind,
                       float lower_bound, int B, int T, int HV, int K, int chunk, float* g_out,
                       hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k, const void* v, int bf16,
                         const float* g_raw, const float* beta, const float* A_log,
                         const float* dt_bias, int kind, int per_head, float lower_bound,
                         float* state, float* o, int B, int H, int HV, int K, int V,
                         hipStream_t stream);
hipError_t launch_recurrent(const void* q, const void* k, const void* v, int bf16,
                            const float* g_raw, const float* beta, const float* A_log,
                            const float* dt_bias, int kind, int per_head, float lower_bound,
                            const float* S0, float* o, float* S_out, int B, int T, int H, int HV,
                            int K, int V, hipStream_t stream);
hipError_t launch_chunk(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        int per_head, float lower_bound, const float* S0, float* o, float* S_out,
                        int B, int T, int H, int HV, int K, hipStream_t stream);
size_t split_workspace_bytes_per_chunk(int K, int V, int C);
hipError_t launch_split(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        int per_head, float lower_bound, const float* S0, float* o, float* S_out,
                        float* h, void* workspace, int B, int T, int H, int HV, int K, int C,
                        hipStream_t stream);
size_t bwd_workspace_bytes(int B, int T, int HV, int K, int V);
hipError_t launch_bwd(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                      const float* beta, const float* A_log, const float* dt_bias, int kind,
                      int per_head, float lower_bound, const float* S0, const float* dout, const float* dST,
                      float* dq, float* dk, float* dv, float* dbeta, float* dg_raw, float* dA_log,
                      float* ddt_bias, float* dS0, void* workspace, int B, int T, int H, int HV,
                      int K, hipStream_t stream);
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
}  // namespace kda

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool head_size_ok(int n) { return n == 16 || n == 32 || n == 64 || n == 128; }

// The gate kind without the per-head flag, and the flag.
int gate_base(kda_gate_kind gate) { return (int)gate & ~(int)KDA_GATE_PER_HEAD; }
int gate_per_head(kda_gate_kind gate) { return ((int)gate & (int)KDA_GATE_PER_HEAD) ? 1 : 0; }

// Gate arguments shared by every entry point.
kda_status check_gate(kda_gate_kind gate, float lower_bound, const float* A_log) {
  const int kind = gate_base(gate);
  if (kind != KDA_GATE_STANDARD && kind != KDA_GATE_SAFE && kind != KDA_GATE_NONE)
    return KDA_ERR_INVALID_ARG;
  if (kind != KDA_GATE_NONE && !A_log) return KDA_ERR_INVALID_ARG;
  if (kind == KDA_GATE_SAFE && !(lower_bound < 0.0f && isfinite(lower_bound)))
    return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Gate inputs: per-channel rows are read as 16-byte vectors; a per-head gate
// is read one float at a time.
bool gate_inputs_aligned(kda_gate_kind gate, const float* g_raw, const float* dt_bias) {
  if (gate_per_head(gate)) return (!g_raw || aligned4(g_raw)) && (!dt_bias || aligned4(dt_bias));
  return (!g_raw || aligned16(g_raw)) && (!dt_bias || aligned16(dt_bias));
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head or chunk size not built";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
    case KDA_ERR_SCRATCH:
      return "KDA_ERR_SCRATCH: workspace larger than the allocation-free entry point's fixed scratch";
  }
  return "unknown kda_status";
}

int kda_version(void) { return 10000; }

kda_status kda_gate(const float* g_raw, const float* A_log, const float* dt_bias,
                    kda_gate_kind gate, float lower_bound, int B, int T, int HV, int K,
                    int chunk_size, float* g_out, kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (B < 0 || T < 0 || HV < 1 || K < 1 || chunk_size < 0) return KDA_ERR_INVALID_ARG;
  if (B == 0 || T == 0) return KDA_OK;
  if (!g_raw || !g_out) return KDA_ERR_INVALID_ARG;
  // a per-head gate is the per-channel layout with K = 1
  return from_hip(kda::launch_gate(g_raw, A_log, dt_bias, gate_base(gate), lower_bound, B, T, HV,
                                   gate_per_head(gate) ? 1 : K, chunk_size, g_out,
                                   reinterpret_cast<hipStream_t>(stream)));
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int HV, int K, int V, int chunk_size,
                                     kda_dtype qkv_dtype) {
  (void)B, (void)T, (void)H, (void)HV, (void)K, (void)V, (void)chunk_size, (void)qkv_dtype;
  return 0;  // the fused kernel keeps every intermediate on chip
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                         const float* g_raw, const float* beta, const float* A_log,
                         const float* dt_bias, kda_gate_kind gate, float lower_bound,
                         const float* initial_state, float* o, float* final_state, int B, int T,
                         int H, int HV, int K, int V, int chunk_size, void* workspace,
                         size_t workspace_bytes, kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 28)) return KDA_ERR_INVALID_ARG;
  if (!head_size_ok(K) || V != K) return KDA_ERR_UNSUPPORTED;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  // 16 tokens of g_raw (the widest per-token row) must span less than 2^31 bytes
  if ((long)HV * K > (1L << 24)) return KDA_ERR_UNSUPPORTED;
  // empty tensors may come with null data pointers: required only when there are tokens
  if (B > 0 && T > 0 && (!q || !k || !v || !g_raw || !beta || !o)) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, initial_state, final_state};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  size_t need = kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, chunk_size, qkv_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (B == 0) return KDA_OK;
  return from_hip(kda::launch_chunk(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log, dt_bias,
                                    gate_base(gate), gate_per_head(gate), lower_bound,
                                    initial_state, o, final_state, B, T, H, HV, K,
                                    reinterpret_cast<hipStream_t>(stream)));
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                              const float* g_raw, const float* beta, const float* A_log,
                              const float* dt_bias, kda_gate_kind gate, float lower_bound,
                              float* state, float* o, int B, int H, int HV, int K, int V,
                              kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 28)) return KDA_ERR_INVALID_ARG;
  if (!head_size_ok(K) || !head_size_ok(V)) return KDA_ERR_UNSUPPORTED;
  if (B > 0 && (!q || !k || !v || !g_raw || !beta || !state || !o)) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, state, o};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  if (B == 0) return KDA_OK;
  return from_hip(kda::launch_decode(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log, dt_bias,
                                     gate_base(gate), gate_per_head(gate), lower_bound, state, o,
                                     B, H, HV, K, V, reinterpret_cast<hipStream_t>(stream)));
}

kda_status kda_recurrent_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const float* g_raw, const float* beta, const float* A_log,
                             const float* dt_bias, kda_gate_kind gate, float lower_bound,
                             const float* initial_state, float* o, float* final_state, int B,
                             int T, int H, int HV, int K, int V, kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 28)) return KDA_ERR_INVALID_ARG;
  if (!head_size_ok(K) || !head_size_ok(V)) return KDA_ERR_UNSUPPORTED;
  if (B > 0 && T > 0 && (!q || !k || !v || !g_raw || !beta || !o)) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, initial_state, final_state};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  if (B == 0) return KDA_OK;
  return from_hip(kda::launch_recurrent(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log,
                                        dt_bias, gate_base(gate), gate_per_head(gate),
                                        lower_bound, initial_state, o, final_state, B, T, H, HV,
                                        K, V, reinterpret_cast<hipStream_t>(stream)));
}

size_t kda_chunk_fwd_split_workspace_bytes(int B, int T, int H, int HV, int K, int V,
                                           int chunk_size) {
  (void)H;
  if (B <= 0 || T <= 0 || HV < 1 || K < 1 || V < 1 || chunk_size < 1) return 0;
  const size_t nc = ((size_t)T + chunk_size - 1) / chunk_size;
  return (size_t)B * HV * nc * kda::split_workspace_bytes_per_chunk(K, V, chunk_size);
}

}  // extern "C"

namespace {

// Argument checks of the split schedule, workspace aside.
kda_status check_split(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                       const float* g_raw, const float* beta, const float* A_log,
                       const float* dt_bias, kda_gate_kind gate, float lower_bound,
                       const float* initial_state, const float* o, const float* final_state,
                       const float* h, int B, int T, int H, int HV, int K, int V,
                       int chunk_size) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 28)) return KDA_ERR_INVALID_ARG;
  if (!head_size_ok(K) || V != K) return KDA_ERR_UNSUPPORTED;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  const long nc = ((long)T + chunk_size - 1) / chunk_size;
  if ((long)B * HV * nc > 0x7fffffffL) return KDA_ERR_INVALID_ARG;  // one workgroup per chunk
  // o may be NULL when h is wanted: the states only, without the output stage
  if (B > 0 && T > 0 && (!q || !k || !v || !g_raw || !beta || (!o && !h)))
    return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, initial_state, final_state, h};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v,
                                       kda_dtype qkv_dtype, const float* g_raw, const float* beta,
                                       const float* A_log, const float* dt_bias,
                                       kda_gate_kind gate, float lower_bound,
                                       const float* initial_state, float* o, float* final_state,
                                       float* h, int B, int T, int H, int HV, int K, int V,
                                       int chunk_size, kda_stream_t stream) {
  kda_status st = check_split(q, k, v, qkv_dtype, g_raw, beta, A_log, dt_bias, gate, lower_bound,
                              initial_state, o, final_state, h, B, T, H, HV, K, V, chunk_size);
  if (st != KDA_OK) return st;
  const size_t need = kda_chunk_fwd_split_workspace_bytes(B, T, H, HV, K, V, chunk_size);
  if (need > kda::noalloc_scratch_bytes()) return KDA_ERR_SCRATCH;
  if (B == 0) return KDA_OK;
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = kda::noalloc_scratch(&scratch);
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  return from_hip(kda::launch_split(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log, dt_bias,
                                    gate_base(gate), gate_per_head(gate), lower_bound,
                                    initial_state, o, final_state, h, scratch, B, T, H, HV, K,
                                    chunk_size, reinterpret_cast<hipStream_t>(stream)));
}

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* g_raw, const float* beta, const float* A_log,
                               const float* dt_bias, kda_gate_kind gate, float lower_bound,
                               const float* initial_state, float* o, float* final_state, float* h,
                               int B, int T, int H, int HV, int K, int V, int chunk_size,
                               void* workspace, size_t workspace_bytes, kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 28)) return KDA_ERR_INVALID_ARG;
  if (!head_size_ok(K) || V != K) return KDA_ERR_UNSUPPORTED;
  if (chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return KDA_ERR_UNSUPPORTED;
  const long nc = ((long)T + chunk_size - 1) / chunk_size;
  if ((long)B * HV * nc > 0x7fffffffL) return KDA_ERR_INVALID_ARG;  // one workgroup per chunk
  // o may be NULL when h is wanted: the states only, without the output stage
  if (B > 0 && T > 0 && (!q || !k || !v || !g_raw || !beta || (!o && !h)))
    return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, initial_state, final_state, h, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  const size_t need = kda_chunk_fwd_split_workspace_bytes(B, T, H, HV, K, V, chunk_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (B == 0) return KDA_OK;
  return from_hip(kda::launch_split(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log, dt_bias,
                                    gate_base(gate), gate_per_head(gate), lower_bound,
                                    initial_state, o, final_state, h, workspace, B, T, H, HV, K,
                                    chunk_size, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

size_t kda_bwd_workspace_bytes(int B, int T, int H, int HV, int K, int V) {
  (void)H;
  if (B <= 0 || T <= 0 || HV <= 0 || K != V || (K != 32 && K != 64 && K != 128)) return 0;
  return kda::bwd_workspace_bytes(B, T, HV, K, V);
}

kda_status kda_bwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                   const float* g_raw, const float* beta, const float* A_log, const float* dt_bias,
                   kda_gate_kind gate, float lower_bound, const float* initial_state,
                   const float* dout, const float* dfinal_state, float* dq, float* dk, float* dv,
                   float* dbeta, float* dg_raw, float* dA_log, float* ddt_bias,
                   float* dinitial_state, int B, int T, int H, int HV, int K, int V,
                   void* workspace, size_t workspace_bytes, kda_stream_t stream) {
  kda_status st = check_gate(gate, lower_bound, A_log);
  if (st != KDA_OK) return st;
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0) return KDA_ERR_INVALID_ARG;
  if ((long)B * HV > (1L << 26) || HV > 65535) return KDA_ERR_INVALID_ARG;
  if ((K != 32 && K != 64 && K != 128) || V != K) return KDA_ERR_UNSUPPORTED;
  const long nc = ((long)T + 15) / 16;
  if ((long)B * HV * nc > 0x7fffffffL || (long)B * T > 0x7fffffffL) return KDA_ERR_INVALID_ARG;
  if (B > 0 && T > 0 &&
      (!q || !k || !v || !g_raw || !beta || !dout || !dq || !dk || !dv || !dbeta || !dg_raw))
    return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, dv, initial_state, dinitial_state, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
  const void* ptrs4[] = {dout, dfinal_state, dq, dk, dbeta, dg_raw, dA_log, ddt_bias};
  for (const void* ptr : ptrs4)
    if (ptr && !aligned4(ptr)) return KDA_ERR_INVALID_ARG;
  if (!gate_inputs_aligned(gate, g_raw, dt_bias)) return KDA_ERR_INVALID_ARG;
  const size_t need = kda_bwd_workspace_bytes(B, T, H, HV, K, V);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  if (B == 0 && !dA_log && !ddt_bias) return KDA_OK;  // else those two sums are zero-filled
  return from_hip(kda::launch_bwd(q, k, v, qkv_dtype == KDA_BF16, g_raw, beta, A_log, dt_bias,
                                  gate_base(gate), gate_per_head(gate), lower_bound, initial_state, dout, dfinal_state,
                                  dq, dk, dv, dbeta, dg_raw, dA_log, ddt_bias, dinitial_state,
                                  workspace, B, T, H, HV, K, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
