// Chunk-parallel KDA forward with materialised chunk-entry states: the
// chunkwise form split into three launches, so that only the state pass runs
// sequentially over a sequence ("DeltaNet family" page, sections "Chunkwise
// KDA" and "Chunkwise Triton pipeline": an intra-chunk stage, one traversal
// across chunks that materialises the entry state h of every chunk, and an
// output stage that is parallel over chunks).
//
// For chunk c (tokens t0 .. t0 + C - 1) with G_i the inclusive sum of the
// log-decay from the chunk start (per key channel), s = 1/sqrt(K):
//
//   R_ij  = beta_i sum_k k_ik k_jk exp(G_ik - G_jk)             (j < i)
//   W     = (I + R)^{-1} diag(beta) (k * exp(G))                C x K
//   u     = (I + R)^{-1} diag(beta) v                           C x V
//   Kt    = k * exp(G_{C-1} - G),  gamma = exp(G_{C-1})
//   U     = u - W h_c,   h_{c+1} = diag(gamma) h_c + Kt^T U     (state pass)
//   O     = s (q * exp(G)) h_c + A U,
//   A_ij  = s sum_k q_ik k_jk exp(G_ik - G_jk)                  (j <= i)
//
// Every factor is bounded by |k| or |q| for a non-positive log-decay: the
// terms of R and A between different 16-token sub-blocks I > J are split at
// the end of sub-block J, exp(G_i - G_Jend) exp(G_Jend - G_j), both factors
// at most 1, and run on MFMA; the terms inside one 16-token sub-block are
// summed directly, exp(G_i - G_j) per channel, which is exact for any decay.
//
//   split_intra_kernel   one workgroup per (b, hv, chunk): gate, cumulative
//                        sums, R, the blocked triangular solve for W and u,
//                        Kt and gamma into the workspace
//   split_state_kernel   one workgroup per (b, hv), one wavefront per 16-wide
//                        value column block holding that block of the fp32
//                        state in registers; per chunk: h_c out, U = u - W h_c
//                        (written over u), h_{c+1}
//   split_output_kernel  one workgroup per (b, hv, chunk): gate and sums
//                        again, A, O = s (q * exp(G)) h_c + A U
//
// All products use the fp32 MFMA (16x16x4) with fp32 accumulation; bf16
// inputs are widened on load.
#include "kda_device.h"

namespace kda {

struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g_raw;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  const float* S0;
  float* o;
  float* S_out;
  float* h;    // [B, HV, NC, K, V] entry state of every chunk
  float* w;    // workspace: W      [B, HV, NC, C, K]
  float* kt;   //            Kt^T   [B, HV, NC, K, C]
  float* u;    //            u -> U [B, HV, NC, C, V]
  float* gam;  //            gamma  [B, HV, NC, K]
  int B, T, H, HV, NC, kind, per_head;
  float lower_bound;
};

constexpr int kSplitThreads = 256;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Shared memory of a chunk: the log2 cumulative decay inside each 16-token
// sub-block, and the k (and q) rows in fp32, row stride K + 4 (16-byte rows,
// spread over the banks).  The exponent of every decay factor is formed from
// these local sums and whole sub-block totals, never as the difference of two
// long prefix sums, so its rounding error scales with the factor's own
// exponent (terms of one sign add without cancellation).
template <int K, int C>
struct alignas(16) ChunkRows {
  static constexpr int LD = K + 4;
  alignas(16) float G2[C * LD];  // G2[i] = sum of log2 alpha over the sub-block of i, up to i
  alignas(16) float k[C * LD];
  alignas(16) float beta[C];
};

// log2 decay of whole sub-blocks J0 .. J1 - 1 in channel c
template <int K, int C>
__device__ __forceinline__ float blocks_log2(const ChunkRows<K, C>& L, int J0, int J1, int c) {
  float s = 0.0f;
  for (int J = J0; J < J1; ++J) s += L.G2[(J * 16 + 15) * ChunkRows<K, C>::LD + c];
  return s;
}

// Loads chunk c of head (b, hv): G2 (see ChunkRows), k (and q when qrows is
// given) widened to fp32, beta.  Tokens at or past T read as g = 0,
// k = q = 0, beta = 0, which leave the state unchanged.  Ends with a barrier.
template <int K, int C, typename T>
__device__ void load_chunk(const SplitParams& p, long bh, int c, ChunkRows<K, C>& L, float* qrows) {
  constexpr int LD = ChunkRows<K, C>::LD, NB = C / 16;
  const int tid = threadIdx.x;
  const int HV = p.HV, T_ = p.T;
  const int hv = (int)(bh % HV);
  const long b = bh / HV;
  const int hq = hv / (HV / p.H);
  const int t0 = c * C;
  const int gK = p.per_head ? 1 : K;
  const float rate = p.kind != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;

  // gate and the cumulative sum inside each sub-block: one (channel,
  // sub-block) pair per thread and pass
  for (int pr = tid; pr < K * NB; pr += kSplitThreads) {
    const int kap = pr % K, J = pr / K;
    const int gc = p.per_head ? 0 : kap;
    const float bias =
        (p.dt_bias && p.kind != KDA_GATE_NONE) ? p.dt_bias[(long)hv * gK + gc] : 0.0f;
    float run = 0.0f;
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const int i = J * 16 + j;
      const int t = t0 + i;
      float g = 0.0f;
      if (t < T_)
        g = gate_log_decay(p.g_raw[((b * T_ + t) * HV + hv) * (long)gK + gc], bias, rate, p.kind,
                           p.lower_bound);
      run += g * kLog2e;
      L.G2[i * LD + kap] = run;
    }
  }

  // k (and q) rows, four elements per load
  const T* kp = static_cast<const T*>(p.k);
  const T* qp = static_cast<const T*>(p.q);
  for (int e = tid; e < C * K / 4; e += kSplitThreads) {
    const int i = e / (K / 4), c4 = (e % (K / 4)) * 4;
    const int t = t0 + i;
    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < T_) {
      const long off = ((b * T_ + t) * p.H + hq) * (long)K + c4;
      In<T>::load4(kp, off, x);
      if (qrows) In<T>::load4(qp, off, y);
    }
    *reinterpret_cast<float4*>(L.k + i * LD + c4) = make_float4(x[0], x[1], x[2], x[3]);
    if (qrows) *reinterpret_cast<float4*>(qrows + i * LD + c4) = make_float4(y[0], y[1], y[2], y[3]);
  }
  for (int i = tid; i < C; i += kSplitThreads)
    L.beta[i] = t0 + i < T_ ? p.beta[(b * T_ + t0 + i) * HV + hv] : 0.0f;
  __syncthreads();
}

// sum_k a_ik k_jk 2^(G2_ik - G2_jk) for rows i, j of one sub-block (direct form).
template <int K, int C>
__device__ __forceinline__ float decayed_dot(const ChunkRows<K, C>& L, const float* arows, int i,
                                             int j) {
  constexpr int LD = ChunkRows<K, C>::LD;
  float acc = 0.0f;
#pragma unroll 4
  for (int c4 = 0; c4 < K; c4 += 4) {
    const float4 a = *reinterpret_cast<const float4*>(arows + i * LD + c4);
    const float4 bb = *reinterpret_cast<const float4*>(L.k + j * LD + c4);
    const float4 gi = *reinterpret_cast<const float4*>(L.G2 + i * LD + c4);
    const float4 gj = *reinterpret_cast<const float4*>(L.G2 + j * LD + c4);
    acc += a.x * bb.x * __builtin_amdgcn_exp2f(gi.x - gj.x);
    acc += a.y * bb.y * __builtin_amdgcn_exp2f(gi.y - gj.y);
    acc += a.z * bb.z * __builtin_amdgcn_exp2f(gi.z - gj.z);
    acc += a.w * bb.w * __builtin_amdgcn_exp2f(gi.w - gj.w);
  }
  return acc;
}

// The 16 x 16 block (I, J), I > J, of  sum_k a_ik k_jk 2^(G_ik - G_jk) (G the
// log2 cumulative decay over the chunk), split at the last token of sub-block
// J; result in the accumulator layout.
template <int K, int C>
__device__ __forceinline__ f32x4 decayed_block(const ChunkRows<K, C>& L, const float* arows, int I,
                                               int J, int lane) {
  constexpr int LD = ChunkRows<K, C>::LD;
  const int ai = I * 16 + (lane & 15), bj = J * 16 + (lane & 15), je = J * 16 + 15;
  const int kk = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < K; s += 4) {
    const int c = s + kk;
    const float mid = blocks_log2(L, J + 1, I, c);  // whole sub-blocks between J and I
    const float a = arows[ai * LD + c] * __builtin_amdgcn_exp2f(L.G2[ai * LD + c] + mid);
    const float bb = L.k[bj * LD + c] * __builtin_amdgcn_exp2f(L.G2[je * LD + c] - L.G2[bj * LD + c]);
    acc = mfma4(a, bb, acc);
  }
  return acc;
}

// pair index -> (i, j), j < i < 16 (strict) or j <= i < 16
__device__ __forceinline__ void tri_pair(int pr, bool strict, int& i, int& j) {
  int r = strict ? 1 : 0;
  while (true) {
    const int n = strict ? r : r + 1;  // pairs in row r
    if (pr < n) break;
    pr -= n;
    ++r;
  }
  i = r;
  j = pr;
}

// ----------------------------------------------------------------- intra
template <int K, int C, typename T>
__global__ __launch_bounds__(kSplitThreads) void split_intra_kernel(SplitParams p) {
  constexpr int NB = C / 16, LD = ChunkRows<K, C>::LD, LR = C + 4, LX = 20;
  __shared__ ChunkRows<K, C> L;
  __shared__ alignas(16) float R[C * LR];
  __shared__ alignas(16) float Xd[NB * 16 * LX];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  const long ch = blockIdx.x;
  const long bh = ch / p.NC;
  const int c = (int)(ch % p.NC);
  load_chunk<K, C, T>(p, bh, c, L, nullptr);

  // R inside the 16-token sub-blocks, direct
  for (int e = tid; e < NB * 120; e += kSplitThreads) {
    const int J = e / 120;
    int i, j;
    tri_pair(e % 120, true, i, j);
    i += J * 16;
    j += J * 16;
    R[i * LR + j] = L.beta[i] * decayed_dot<K, C>(L, L.k, i, j);
  }
  // R between sub-blocks I > J, on MFMA
  constexpr int NP = NB * (NB - 1) / 2;
  for (int pi = w; pi < NP; pi += kSplitThreads / 64) {
    int I, J;
    tri_pair(pi, true, I, J);
    const f32x4 acc = decayed_block<K, C>(L, L.k, I, J, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = I * 16 + 4 * g4 + r;
      R[i * LR + J * 16 + (lane & 15)] = L.beta[i] * acc[r];
    }
  }
  __syncthreads();

  // (I + R_JJ)^{-1} of each diagonal 16 x 16 block: lane j of group J
  // substitutes down column j
  if (tid < NB * 16) {
    const int J = tid >> 4, j = tid & 15;
    const float* Rj = R + (J * 16) * LR + J * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = i == j ? 1.0f : 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) a -= Rj[i * LR + m] * x[m];
      x[i] = a;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Xd[(J * 16 + i) * LX + j] = x[i];
  }
  __syncthreads();

  // [W | u] = (I + R)^{-1} diag(beta) [k exp(G) | v], by blocks of 16 rows:
  // Y_I = X_II (B_I - sum_{J<I} R_IJ Y_J), one 16-wide column block per pass
  const T* vp = static_cast<const T*>(p.v);
  const int hv = (int)(bh % p.HV);
  const long b = bh / p.HV;
  const int t0 = c * C;
  float* Wout = p.w + ch * (long)C * K;
  float* Uout = p.u + ch * (long)C * K;
  for (int cb = w; cb < 2 * (K / 16); cb += kSplitThreads / 64) {
    const bool isw = cb < K / 16;
    const int col = (isw ? cb : cb - K / 16) * 16 + (lane & 15);
    f32x4 y[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = I * 16 + 4 * g4 + r;
        float x;
        if (isw) {
          x = L.k[i * LD + col] *
              __builtin_amdgcn_exp2f(L.G2[i * LD + col] + blocks_log2(L, 0, I, col));
        } else {
          x = t0 + i < p.T ? In<T>::at(vp, ((b * p.T + t0 + i) * p.HV + hv) * (long)K + col) : 0.0f;
        }
        t[r] = L.beta[i] * x;
      }
#pragma unroll
      for (int J = 0; J < I; ++J) {
        const float4 a = *reinterpret_cast<const float4*>(R + (I * 16 + (lane & 15)) * LR + J * 16 + 4 * g4);
        t = mfma4(-a.x, y[J][0], t);
        t = mfma4(-a.y, y[J][1], t);
        t = mfma4(-a.z, y[J][2], t);
        t = mfma4(-a.w, y[J][3], t);
      }
      const float4 a = *reinterpret_cast<const float4*>(Xd + (I * 16 + (lane & 15)) * LX + 4 * g4);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      z = mfma4(a.x, t[0], z);
      z = mfma4(a.y, t[1], z);
      z = mfma4(a.z, t[2], z);
      z = mfma4(a.w, t[3], z);
      y[I] = z;
    }
    float* out = isw ? Wout : Uout;
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(I * 16 + 4 * g4 + r) * K + col] = y[I][r];
  }

  // Kt^T [K][C] and gamma
  float* kt = p.kt + ch * (long)K * C;
  for (int e = tid; e < K * C; e += kSplitThreads) {
    const int kap = e / C, i = e % C;
    const int I = i >> 4;
    const float rest = (L.G2[(I * 16 + 15) * LD + kap] - L.G2[i * LD + kap]) + blocks_log2(L, I + 1, NB, kap);
    kt[e] = L.k[i * LD + kap] * __builtin_amdgcn_exp2f(rest);
  }
  for (int kap = tid; kap < K; kap += kSplitThreads)
    p.gam[ch * K + kap] = __builtin_amdgcn_exp2f(blocks_log2(L, 0, NB, kap));
}

// ----------------------------------------------------------------- states
// One wavefront per 16-wide column block of the state; lane l holds rows
// 16 kb + 4 (l / 16) + r of column l % 16 (the MFMA accumulator layout), which
// is also the layout of the B operand the two products below take.
template <int K, int C>
__global__ __launch_bounds__(K * 4) void split_state_kernel(SplitParams p) {
  constexpr int NB = C / 16, NKB = K / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4;
  const long bh = blockIdx.x;
  const int col = w * 16 + (lane & 15);
  f32x4 s[NKB];
  const float* S0 = p.S0 ? p.S0 + bh * (long)K * K : nullptr;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[kb][r] = S0 ? S0[(kb * 16 + 4 * g4 + r) * K + col] : 0.0f;

  for (int c = 0; c < p.NC; ++c) {
    const long ch = bh * p.NC + c;
    float* hc = p.h + ch * (long)K * K;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) hc[(kb * 16 + 4 * g4 + r) * K + col] = s[kb][r];

    // X = W h_c, then U = u - X (over u)
    const float* W = p.w + ch * (long)C * K;
    float* U = p.u + ch * (long)C * K;
    f32x4 x[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const float4 a = *reinterpret_cast<const float4*>(W + (I * 16 + (lane & 15)) * K + kb * 16 + 4 * g4);
        acc = mfma4(a.x, s[kb][0], acc);
        acc = mfma4(a.y, s[kb][1], acc);
        acc = mfma4(a.z, s[kb][2], acc);
        acc = mfma4(a.w, s[kb][3], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int idx = (I * 16 + 4 * g4 + r) * K + col;
        const float uu = U[idx] - acc[r];
        U[idx] = uu;
        x[I][r] = uu;
      }
    }

    // h_{c+1} = diag(gamma) h_c + Kt^T U
    const float* Kt = p.kt + ch * (long)K * C;
    const float* gm = p.gam + ch * K;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float4 gg = *reinterpret_cast<const float4*>(gm + kb * 16 + 4 * g4);
      f32x4 acc = {gg.x * s[kb][0], gg.y * s[kb][1], gg.z * s[kb][2], gg.w * s[kb][3]};
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const float4 a = *reinterpret_cast<const float4*>(Kt + (kb * 16 + (lane & 15)) * C + I * 16 + 4 * g4);
        acc = mfma4(a.x, x[I][0], acc);
        acc = mfma4(a.y, x[I][1], acc);
        acc = mfma4(a.z, x[I][2], acc);
        acc = mfma4(a.w, x[I][3], acc);
      }
      s[kb] = acc;
    }
  }
  if (p.S_out) {
    float* So = p.S_out + bh * (long)K * K;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) So[(kb * 16 + 4 * g4 + r) * K + col] = s[kb][r];
  }
}

// ----------------------------------------------------------------- output
template <int K, int C, typename T>
__global__ __launch_bounds__(kSplitThreads) void split_output_kernel(SplitParams p) {
  constexpr int NB = C / 16, LD = ChunkRows<K, C>::LD, LR = C + 4;
  __shared__ ChunkRows<K, C> L;
  __shared__ alignas(16) float Q[C * LD];
  __shared__ alignas(16) float A[C * LR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  const long ch = blockIdx.x;
  const long bh = ch / p.NC;
  const int c = (int)(ch % p.NC);
  load_chunk<K, C, T>(p, bh, c, L, Q);
  const float scale = 1.0f / __builtin_sqrtf((float)K);

  // A inside the sub-blocks (j <= i), direct
  for (int e = tid; e < NB * 136; e += kSplitThreads) {
    const int J = e / 136;
    int i, j;
    tri_pair(e % 136, false, i, j);
    i += J * 16;
    j += J * 16;
    A[i * LR + j] = scale * decayed_dot<K, C>(L, Q, i, j);
  }
  for (int e = tid; e < NB * 120; e += kSplitThreads) {  // zeros above the diagonal
    const int J = e / 120;
    int i, j;
    tri_pair(e % 120, true, i, j);
    A[(J * 16 + j) * LR + J * 16 + i] = 0.0f;
  }
  constexpr int NP = NB * (NB - 1) / 2;
  for (int pi = w; pi < NP; pi += kSplitThreads / 64) {
    int I, J;
    tri_pair(pi, true, I, J);
    const f32x4 acc = decayed_block<K, C>(L, Q, I, J, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) A[(I * 16 + 4 * g4 + r) * LR + J * 16 + (lane & 15)] = scale * acc[r];
  }
  __syncthreads();
  // Q <- s q exp(G)
  for (int e = tid; e < C * K; e += kSplitThreads) {
    const int i = e / K, kap = e % K;
    Q[i * LD + kap] *= scale * __builtin_amdgcn_exp2f(L.G2[i * LD + kap] + blocks_log2(L, 0, i >> 4, kap));
  }
  __syncthreads();

  const int hv = (int)(bh % p.HV);
  const long b = bh / p.HV;
  const int t0 = c * C;
  const float* hc = p.h + ch * (long)K * K;
  const float* U = p.u + ch * (long)C * K;
  constexpr int KQ = K / 4;  // key channels per lane group: channel = g4 * KQ + s
  for (int cb = w; cb < K / 16; cb += kSplitThreads / 64) {
    const int col = cb * 16 + (lane & 15);
    float hf[KQ];
#pragma unroll
    for (int s = 0; s < KQ; ++s) hf[s] = hc[(g4 * KQ + s) * K + col];
    f32x4 uf[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J)
#pragma unroll
      for (int r = 0; r < 4; ++r) uf[J][r] = U[(J * 16 + 4 * g4 + r) * K + col];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* qrow = Q + (I * 16 + (lane & 15)) * LD + g4 * KQ;
#pragma unroll
      for (int s = 0; s < KQ; s += 4) {
        const float4 a = *reinterpret_cast<const float4*>(qrow + s);
        acc = mfma4(a.x, hf[s], acc);
        acc = mfma4(a.y, hf[s + 1], acc);
        acc = mfma4(a.z, hf[s + 2], acc);
        acc = mfma4(a.w, hf[s + 3], acc);
      }
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const float4 a = *reinterpret_cast<const float4*>(A + (I * 16 + (lane & 15)) * LR + J * 16 + 4 * g4);
        acc = mfma4(a.x, uf[J][0], acc);
        acc = mfma4(a.y, uf[J][1], acc);
        acc = mfma4(a.z, uf[J][2], acc);
        acc = mfma4(a.w, uf[J][3], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + I * 16 + 4 * g4 + r;
        if (t < p.T) p.o[((b * p.T + t) * p.HV + hv) * (long)K + col] = acc[r];
      }
    }
  }
}

// ----------------------------------------------------------------- launch
template <int K, int C, typename T>
static hipError_t launch_split_kc(const SplitParams& p, hipStream_t stream) {
  const long heads = (long)p.B * p.HV;
  const long chunks = heads * p.NC;
  if (chunks > 0) {
    hipLaunchKernelGGL((split_intra_kernel<K, C, T>), dim3((unsigned)chunks), dim3(kSplitThreads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((split_state_kernel<K, C>), dim3((unsigned)heads), dim3(K * 4), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 0) return e;
  hipLaunchKernelGGL((split_output_kernel<K, C, T>), dim3((unsigned)chunks), dim3(kSplitThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_split_t(const SplitParams& p, int K, int C, hipStream_t stream) {
#define KDA_SPLIT_CASE(KK, CC) \
  if (K == KK && C == CC) return launch_split_kc<KK, CC, T>(p, stream);
#define KDA_SPLIT_ROW(KK) KDA_SPLIT_CASE(KK, 16) KDA_SPLIT_CASE(KK, 32) KDA_SPLIT_CASE(KK, 64)
  KDA_SPLIT_ROW(16) KDA_SPLIT_ROW(32) KDA_SPLIT_ROW(64) KDA_SPLIT_ROW(128)
#undef KDA_SPLIT_ROW
#undef KDA_SPLIT_CASE
  return hipErrorInvalidValue;
}

// Workspace floats per (b, hv, chunk): W, Kt^T, u / U, gamma and the entry state.
size_t split_workspace_floats(int K, int V, int C) {
  return (size_t)C * K + (size_t)K * C + (size_t)C * V + (size_t)K + (size_t)K * V;
}

hipError_t launch_split(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        int per_head, float lower_bound, const float* S0, float* o, float* S_out,
                        float* h, void* workspace, int B, int T, int H, int HV, int K, int C,
                        hipStream_t stream) {
  const int NC = (T + C - 1) / C;
  const size_t n = (size_t)B * HV * NC;
  float* ws = static_cast<float*>(workspace);
  SplitParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g_raw = g_raw;
  p.beta = beta;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.S0 = S0;
  p.o = o;
  p.S_out = S_out;
  p.w = ws;
  p.kt = p.w + n * C * K;
  p.u = p.kt + n * K * C;
  p.gam = p.u + n * C * K;
  p.h = h ? h : p.gam + n * K;
  p.B = B;
  p.T = T;
  p.H = H;
  p.HV = HV;
  p.NC = NC;
  p.kind = kind;
  p.per_head = per_head;
  p.lower_bound = lower_bound;
  return bf16 ? launch_split_t<uint16_t>(p, K, C, stream) : launch_split_t<float>(p, K, C, stream);
}

}  // namespace kda
