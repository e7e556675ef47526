// One recurrent (decode) step of KDA for every sequence, state updated in place.
//
// Per (b, hv) the step applies the four-step update of the "K3 notes" section
// "KDA 递归核心" (decay, key prediction and residual, rank-1 write, query read
// with 1/sqrt(K)), the schedule of the "DeltaNet family" page's fused recurrent
// mode: independent programs per (sequence, value head, value tile), each
// owning a tile of the state for the whole step.
//
// The step is bound by HBM: the fp32 state [K, V] of every (b, hv) is read once
// and written once.  One wavefront owns a K x TV column tile (TV = min(V, 32)):
// lane l holds column quad cq = l % NQ (16-byte loads, NQ lanes cover one
// 128-byte row segment) and rows kappa = rg + RG * i of row group rg = l / NQ,
// so every load instruction reads RG full row segments.  All RPL row loads are
// issued before any arithmetic.  The two reductions over kappa (prediction
// k.S_dec and read q.S_new) stay inside the wavefront: lanes of one column quad
// differ only in the rg bits, so log2(RG) butterfly shuffles finish each sum;
// no LDS and no barrier.
#include "kda_device.h"

namespace kda {

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g_raw;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  float* state;
  float* o;
  int B, H, HV, kind;
  float lower_bound;
};

template <int K, int V, typename T>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeParams p) {
  constexpr int TV = V < 32 ? V : 32;  // columns per wavefront
  constexpr int NQ = TV / 4;           // column quads per row segment
  constexpr int RG = 64 / NQ;          // row groups
  constexpr int RPL = K / RG;          // rows per lane
  static_assert(RPL >= 1 && K % RG == 0, "head size too small for this tiling");
  constexpr int NVT = V / TV;

  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const long nwaves = (long)p.B * p.HV * NVT;
  if (wave >= nwaves) return;
  const int vt = (int)(wave % NVT);
  const long bh = wave / NVT;  // b * HV + hv
  const int hv = (int)(bh % p.HV);
  const long b = bh / p.HV;
  const int h = hv / (p.HV / p.H);

  const int cq = lane % NQ;
  const int rg = lane / NQ;
  const int col = vt * TV + cq * 4;

  float* S = p.state + bh * (long)K * V;
  f32x4 s[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (long)(rg + RG * i) * V + col));

  const T* q = static_cast<const T*>(p.q) + (b * p.H + h) * K;
  const T* kk = static_cast<const T*>(p.k) + (b * p.H + h) * K;
  const float* gr = p.g_raw + bh * K;
  const float rate = p.kind != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const float* bias = (p.dt_bias && p.kind != KDA_GATE_NONE) ? p.dt_bias + (long)hv * K : nullptr;
  float kr[RPL], qr[RPL], al[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int r = rg + RG * i;
    kr[i] = In<T>::at(kk, r);
    qr[i] = In<T>::at(q, r);
    al[i] = exp_f(gate_log_decay(gr[r], bias ? bias[r] : 0.0f, rate, p.kind, p.lower_bound));
  }
  float vv[4];
  In<T>::load4(static_cast<const T*>(p.v), bh * V + col, vv);
  const float bt = p.beta[bh];

  // decay, then prediction p = k . S_dec
  f32x4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    s[i] *= al[i];
    pr += kr[i] * s[i];
  }
#pragma unroll
  for (int m = NQ; m < 64; m <<= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) pr[c] += __shfl_xor(pr[c], m);

  // residual, rank-1 write, read q . S_new
  f32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = bt * (vv[c] - pr[c]);
  f32x4 ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    s[i] += kr[i] * r;
    ov += qr[i] * s[i];
  }
#pragma unroll
  for (int m = NQ; m < 64; m <<= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] += __shfl_xor(ov[c], m);

#pragma unroll
  for (int i = 0; i < RPL; ++i)
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (long)(rg + RG * i) * V + col));
  if (rg == 0) {
    const float scale = 1.0f / __builtin_sqrtf((float)K);
    *reinterpret_cast<f32x4*>(p.o + bh * V + col) = ov * scale;
  }
}

template <int K, int V, typename T>
static hipError_t launch_decode_kv(const DecodeParams& p, hipStream_t stream) {
  constexpr int TV = V < 32 ? V : 32;
  long waves = (long)p.B * p.HV * (V / TV);
  long blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((decode_step_kernel<K, V, T>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_t(const DecodeParams& p, int K, int V, hipStream_t stream) {
#define KDA_DEC_CASE(KK, VV) \
  if (K == KK && V == VV) return launch_decode_kv<KK, VV, T>(p, stream);
#define KDA_DEC_ROW(KK) KDA_DEC_CASE(KK, 16) KDA_DEC_CASE(KK, 32) KDA_DEC_CASE(KK, 64) KDA_DEC_CASE(KK, 128)
  KDA_DEC_ROW(16) KDA_DEC_ROW(32) KDA_DEC_ROW(64) KDA_DEC_ROW(128)
#undef KDA_DEC_ROW
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const void* q, const void* k, const void* v, int bf16,
                         const float* g_raw, const float* beta, const float* A_log,
                         const float* dt_bias, int kind, float lower_bound, float* state,
                         float* o, int B, int H, int HV, int K, int V, hipStream_t stream) {
  DecodeParams p{q, k, v, g_raw, beta, A_log, dt_bias, state, o, B, H, HV, kind, lower_bound};
  return bf16 ? launch_decode_t<uint16_t>(p, K, V, stream) : launch_decode_t<float>(p, K, V, stream);
}

}  // namespace kda
