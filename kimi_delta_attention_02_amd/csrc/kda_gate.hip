// Gate activation + chunk-local cumulative log-decay.
//
// The gate is the elementwise map of the "K3 notes" section "Gate 激活" (two-gate
// table, kda_gate_reference panel).  With chunk_size C > 0 the kernel also forms
// the chunk-local inclusive prefix sum of g along time -- the cumulative
// log-decay of the "DeltaNet family" page's chunkwise pipeline, whose
// differences give D_{j+1:i} -- restarting at every chunk boundary.
//
// One thread per (b, hv, kappa, chunk); it walks the chunk's tokens in order.
// Consecutive threads take consecutive key channels, so every token's row of
// K values is read and written as one coalesced segment.  The work is a single
// pass over g_raw: HBM-bound at 8 bytes per element.
#include "kda_device.h"

namespace kda {

struct GateParams {
  const float* g_raw;
  const float* A_log;
  const float* dt_bias;
  float* g_out;
  int B, T, HV, K, chunk, kind;
  float lower_bound;
};

__global__ __launch_bounds__(256) void gate_cumsum_kernel(GateParams p) {
  const long K = p.K, HV = p.HV, T = p.T;
  const long C = p.chunk > 0 ? p.chunk : 1;
  const long nchunks = (T + C - 1) / C;
  const long total = (long)p.B * HV * K * nchunks;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    long kap = idx % K;
    long r = idx / K;
    long hv = r % HV;
    r /= HV;
    long c = r % nchunks;
    long b = r / nchunks;
    float rate = p.kind != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
    float bias = (p.dt_bias && p.kind != KDA_GATE_NONE) ? p.dt_bias[hv * K + kap] : 0.0f;
    long t0 = c * C, t1 = t0 + C < T ? t0 + C : T;
    float acc = 0.0f;
    for (long t = t0; t < t1; ++t) {
      long off = ((b * T + t) * HV + hv) * K + kap;
      float g = gate_log_decay(p.g_raw[off], bias, rate, p.kind, p.lower_bound);
      if (p.chunk > 0) {
        acc += g;
        g = acc;
      }
      p.g_out[off] = g;
    }
  }
}

hipError_t launch_gate(const float* g_raw, const float* A_log, const float* dt_bias, int kind,
                       float lower_bound, int B, int T, int HV, int K, int chunk, float* g_out,
                       hipStream_t stream) {
  GateParams p{g_raw, A_log, dt_bias, g_out, B, T, HV, K, chunk, kind, lower_bound};
  long C = chunk > 0 ? chunk : 1;
  long total = (long)B * HV * K * ((T + C - 1) / C);
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gate_cumsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
