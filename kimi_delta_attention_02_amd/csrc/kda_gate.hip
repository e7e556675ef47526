// Gate activation + chunk-local cumulative log-decay.
//
// The gate is the elementwise map of the "K3 notes" section "Gate 激活" (two-gate
// table, kda_gate_reference panel).  With chunk_size C > 0 the kernel also forms
// the chunk-local inclusive prefix sum of g along time -- the cumulative
// log-decay of the "DeltaNet family" page's chunkwise pipeline, whose
// differences give D_{j+1:i} -- restarting at every chunk boundary.
//
// One thread per (b, hv, key channel or quad of channels, chunk); it walks the
// chunk's tokens in order, in batches whose loads all go out before the first
// is used.  Consecutive threads take consecutive channels, so every token's
// row of K values is read and written as one coalesced segment.  The work is
// a single pass over g_raw: HBM-bound at 8 bytes per element.
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

// General layout (any K, any alignment): one thread per (b, hv, kappa, chunk).
// Each batch of kBatch tokens is loaded before any of it is used or stored, so
// a thread keeps kBatch loads in flight instead of one (g_out may alias g_raw:
// a thread reads each of its elements before it writes it, and no other
// thread touches them).
constexpr int kBatch = 16;

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
    const long stride = HV * K;
    float acc = 0.0f;
    for (long tb = t0; tb < t1; tb += kBatch) {
      const float* src = p.g_raw + ((b * T + tb) * HV + hv) * K + kap;
      float x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) x[j] = tb + j < t1 ? src[j * stride] : 0.0f;
      float* dst = p.g_out + ((b * T + tb) * HV + hv) * K + kap;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float g = gate_log_decay(x[j], bias, rate, p.kind, p.lower_bound);
        if (p.chunk > 0) {
          acc += g;
          g = acc;
        }
        if (tb + j < t1) dst[j * stride] = g;
      }
    }
  }
}

// K a multiple of 4, 16-byte aligned rows, and g_raw and g_out each under
// 4 GiB: one thread per (b, hv, key quad, chunk), the gate kind a template
// parameter.  Rows are read and written with 16-byte non-temporal buffer
// loads and stores on a descriptor of the whole tensor at 32-bit byte
// offsets, so no 64-bit address is formed per load.  Tokens go in
// batches of kBatch4; the next batch's loads are issued before the current
// one is computed and stored (two register sets, alternating), so every
// thread always has a batch in flight.  Rows past a chunk's end are loaded
// as its last row again and never stored, so no load leaves the tensor.
constexpr int kBatch4 = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNT = 2;  // cache policy bit: non-temporal

template <int GK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void gate_cumsum_kernel4(GateParams p) {
  const long K4 = p.K / 4, HV = p.HV, T = p.T;
  const long C = p.chunk > 0 ? p.chunk : 1;
  const long nchunks = (T + C - 1) / C;
  const long total = (long)p.B * HV * K4 * nchunks;
  const uint32_t bytes = (uint32_t)((long)p.B * T * HV * K4 * 16);
  const auto rin = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.g_raw), (short)0, (int)bytes, 0x00020000);
  const auto rout = __builtin_amdgcn_make_buffer_rsrc(p.g_out, (short)0, (int)bytes, 0x00020000);
  const uint32_t sbytes = (uint32_t)(HV * K4 * 16);  // one token row of all value heads
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const long kq = idx % K4;
    long r = idx / K4;
    const long hv = r % HV;
    r /= HV;
    const long c = r % nchunks;
    const long b = r / nchunks;
    const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.dt_bias && GK != KDA_GATE_NONE) {
      const float4 b4 = reinterpret_cast<const float4*>(p.dt_bias + hv * 4 * K4)[kq];
      bias[0] = b4.x; bias[1] = b4.y; bias[2] = b4.z; bias[3] = b4.w;
    }
    const long t0 = c * C, t1 = t0 + C < T ? t0 + C : T;
    const uint32_t off = (uint32_t)((((b * T + t0) * HV + hv) * K4 + kq) * 16);
    const long n = t1 - t0;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // rows past the chunk's end re-read its last row (never past the tensor)
    const int last = (int)(n - 1);
    auto fetch = [&](long tb, f32x4 x[kBatch4]) {
#pragma unroll
      for (int j = 0; j < kBatch4; ++j) {
        const uint32_t row = (uint32_t)min((int)tb + j, last);
        x[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rin, off + row * sbytes, 0, kNT));
      }
    };
    auto finish = [&](long tb, const f32x4 x[kBatch4]) {
#pragma unroll
      for (int j = 0; j < kBatch4; ++j) {
        float g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[e] = gate_log_decay_k<GK>(x[j][e], bias[e], rate, p.lower_bound);
          if (p.chunk > 0) {
            acc[e] += g[e];
            g[e] = acc[e];
          }
        }
        if (tb + j < n)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{g[0], g[1], g[2], g[3]}),
                                                 rout, off + (uint32_t)(tb + j) * sbytes, 0, kNT);
      }
    };
    f32x4 xa[kBatch4], xb[kBatch4];
    fetch(0, xa);
    long tb = 0;
    for (; tb + kBatch4 < n; tb += 2 * kBatch4) {
      fetch(tb + kBatch4, xb);
      finish(tb, xa);
      if (tb + 2 * kBatch4 < n) fetch(tb + 2 * kBatch4, xa);
      finish(tb + kBatch4, xb);
    }
    if (tb < n) finish(tb, xa);
  }
}

hipError_t launch_gate(const float* g_raw, const float* A_log, const float* dt_bias, int kind,
                       float lower_bound, int B, int T, int HV, int K, int chunk, float* g_out,
                       hipStream_t stream) {
  GateParams p{g_raw, A_log, dt_bias, g_out, B, T, HV, K, chunk, kind, lower_bound};
  const bool vec = K % 4 == 0 && (reinterpret_cast<uintptr_t>(g_raw) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(g_out) & 15) == 0 &&
                   (!dt_bias || (reinterpret_cast<uintptr_t>(dt_bias) & 15) == 0) &&
                   (long)B * T * HV * K * 4 <= 0xFFFFFFFFL;
  long C = chunk > 0 ? chunk : 1;
  long total = (long)B * HV * (vec ? K / 4 : K) * ((T + C - 1) / C);
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (vec && kind == KDA_GATE_SAFE)
    hipLaunchKernelGGL(gate_cumsum_kernel4<KDA_GATE_SAFE>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else if (vec && kind == KDA_GATE_STANDARD)
    hipLaunchKernelGGL(gate_cumsum_kernel4<KDA_GATE_STANDARD>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else if (vec)
    hipLaunchKernelGGL(gate_cumsum_kernel4<KDA_GATE_NONE>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(gate_cumsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
