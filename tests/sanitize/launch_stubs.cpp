// Stand-ins for the kernel launchers of libkda.so, for the host sanitizer
// build of the C ABI's argument validation (test infrastructure): each records
// that it was called and with which sizes, and launches nothing.
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "launch_stubs.h"

StubCall g_last;

static void record(const char* name, int B, int T, int H, int HV, int K, int V, const void* ws) {
  g_last.name = name;
  g_last.B = B, g_last.T = T, g_last.H = H, g_last.HV = HV, g_last.K = K, g_last.V = V;
  g_last.workspace = ws;
  ++g_last.count;
}

namespace kda {
hipError_t launch_gate(const float*, const float*, const float*, int, float, int B, int T, int HV,
                       int K, int, float*, hipStream_t) {
  record("gate", B, T, 0, HV, K, 0, nullptr);
  return hipSuccess;
}
hipError_t launch_decode(const void*, const void*, const void*, int, const float*, const float*,
                         const float*, const float*, int, int, float, float*, float*, int B, int H,
                         int HV, int K, int V, hipStream_t) {
  record("decode", B, 1, H, HV, K, V, nullptr);
  return hipSuccess;
}
hipError_t launch_recurrent(const void*, const void*, const void*, int, const float*, const float*,
                            const float*, const float*, int, int, float, const float*, float*,
                            float*, int B, int T, int H, int HV, int K, int V, hipStream_t) {
  record("recurrent", B, T, H, HV, K, V, nullptr);
  return hipSuccess;
}
hipError_t launch_chunk(const void*, const void*, const void*, int, const float*, const float*,
                        const float*, const float*, int, int, float, const float*, float*, float*,
                        int B, int T, int H, int HV, int K, hipStream_t) {
  record("chunk", B, T, H, HV, K, K, nullptr);
  return hipSuccess;
}
// a stand-in per-chunk size (the real one depends on the kernels' layouts)
size_t split_workspace_bytes_per_chunk(int K, int V, int C) {
  return (size_t)C * K * 8 + ((size_t)C * V + (size_t)K * V) * sizeof(float);
}
hipError_t launch_split(const void*, const void*, const void*, int, const float*, const float*,
                        const float*, const float*, int, int, float, const float*, float*, float*,
                        float*, void* workspace, int B, int T, int H, int HV, int K, int,
                        hipStream_t) {
  record("split", B, T, H, HV, K, K, workspace);
  return hipSuccess;
}
size_t bwd_workspace_bytes(int B, int T, int HV, int K, int V) {
  return (size_t)B * HV * (((size_t)T + 15) / 16) * K * V * sizeof(float) + 256;
}
hipError_t launch_bwd(const void*, const void*, const void*, int, const float*, const float*,
                      const float*, const float*, int, int, float, const float*, const float*,
                      const float*, float*, float*, float*, float*, float*, float*, float*, float*,
                      void* workspace, int B, int T, int H, int HV, int K, hipStream_t) {
  record("bwd", B, T, H, HV, K, K, workspace);
  return hipSuccess;
}
static char fake_scratch[16];
size_t noalloc_scratch_bytes() { return (size_t)64 << 20; }
hipError_t noalloc_scratch(void** out) {
  *out = fake_scratch;
  return hipSuccess;
}
}  // namespace kda
