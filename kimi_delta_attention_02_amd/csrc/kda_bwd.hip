// Backward pass of the KDA forward: the gradients of a loss L(o, S_T) with
// respect to q, k, v, g_raw, beta, A_log, dt_bias and the initial state,
// given dL/do and dL/dS_T.
//
// The pages list a backward derivation without printing it, so the gradients
// are those of the four-step update of the "K3 notes" (section "KDA 递归核心")
// and the gate of section "Gate 激活", in reverse mode.  For one (sequence,
// value head), S[K][V], alpha_t = exp(g_t), s = 1/sqrt(K), and dS the running
// dL/dS_t, token by token from the last:
//
//   Sd_t = diag(alpha_t) S_{t-1},  r_t = v_t - Sd_t^T k_t,  S_t = Sd_t + beta_t k_t r_t^T
//   dS     += s q_t do_t^T              dq_t = s S_t do_t
//   a_t     = dS^T k_t                  dbeta_t = a_t . r_t,  dv_t = dr_t = beta_t a_t
//   dk_t    = beta_t dS r_t - Sd_t dr_t
//   dSd     = dS - k_t dr_t^T           dg_t = rowsum(dSd (.) Sd_t)
//   dS_{t-1} = diag(alpha_t) dSd,       dS0 = dS_{-1}
//
// then the gate's chain rule into g_raw, dt_bias and A_log (sums over the
// sequence for the last two), and under GVA sums of dq, dk over the value
// heads that share a query/key head.
//
// Schedule.  The states S_{t-1} the reverse pass needs come from checkpoints:
// the split schedule (kda_split.hip) writes the state entering every 16-token
// segment; then one workgroup per (sequence, value head, 16-wide value tile)
// walks the segments from the last, recomputes a segment's sixteen states from
// its checkpoint into LDS (128 KiB for K = 128) and runs the reverse recurrence
// over them with its tile of dS in registers.  Thread 2 kappa + c holds key row
// kappa, value columns 8 c .. 8 c + 7 of the tile: sums over the columns are
// in-thread plus one lane exchange, sums over the keys are DPP row rotations,
// row swaps and one LDS exchange across the wavefronts.  The per-key results
// (dq, dk, dg) and dbeta, summed over the value tiles (and the value heads of a
// GVA group), are accumulated with fp32 atomics into zeroed outputs, so their
// last bits depend on the order the tiles finish in.  A last kernel applies
// the gate's chain rule and sums dt_bias and A_log over the sequences.
// Arithmetic is fp32 throughout (bf16 inputs widened exactly).
#include <type_traits>

#include "kda_device.h"

namespace kda {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g_raw;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  const float* dout;
  const float* dST;   // dL/dS_T or null
  const float* ckpt;  // [B, HV, NC, K, V]: the state entering each 16-token segment
  float* dq;
  float* dk;
  float* dv;
  float* dbeta;
  float* dg;  // dL/dg, turned into dL/dg_raw by the gate kernel
  float* dS0;
  float* dA_log;
  float* ddt_bias;
  int B, T, H, HV, NC;
  float lower_bound;
};

constexpr int kSeg = 16;  // tokens per segment (the checkpoint spacing)
constexpr int kBV = 16;   // value columns per workgroup

__global__ void bwd_zero_kernel(float* p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// x + the value N lanes further round its 16-lane row (DPP row rotation)
template <int N>
__device__ __forceinline__ float ror_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, false));
}
// x + the value of the neighbouring lane (quad permutation [1, 0, 3, 2])
__device__ __forceinline__ float pair_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   0xB1, 0xF, 0xF, false));
}

template <int K>
struct BwdSmem {
  float st[kSeg][K][kBV];  // S_{t-1} of the segment's tokens, this tile's columns
  float r[kSeg][kBV];      // residuals
  float v[kSeg][kBV];
  float dout[kSeg][kBV];
  float beta[kSeg];
  float red[2][K / 32][kBV];  // per-wavefront partial sums over the keys (two buffers)
};

template <int K, int V, typename T, int GK>
__global__ __launch_bounds__(2 * K) void bwd_segment_kernel(BwdParams p) {
  constexpr int NW = 2 * K / 64;  // wavefronts
  constexpr int NVT = V / kBV;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  BwdSmem<K>& sm = *reinterpret_cast<BwdSmem<K>*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kap = tid >> 1, ch = tid & 1, c8 = 8 * ch;
  const int vt = blockIdx.x % NVT, hd = blockIdx.x / NVT;
  const int HV = p.HV, H = p.H, T_ = p.T;
  const long b = hd / HV;
  const int hv = hd % HV, h = hv / (HV / H), v0 = vt * kBV;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const GateConsts gc = gate_consts(rate, p.lower_bound);
  const float bias = gate_bias_pre<GK>((p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[hv * K + kap] : 0.0f, gc);
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);

  // sum over the keys of each of this thread's 8 columns: rows of 16 lanes
  // hold 8 keys x 2 column halves, so rotations by 2, 4, 8 keep the half;
  // then the four rows of the wavefront; then the wavefronts, through LDS
  int rb = 0;
  auto key_sum = [&](float x[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = ror_add<2>(x[i]);
      x[i] = ror_add<4>(x[i]);
      x[i] = ror_add<8>(x[i]);
      x[i] = xor_sum<16>(x[i]);
      x[i] = xor_sum<32>(x[i]);
    }
    if (lane < 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.red[rb][w][c8 + i] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) s += sm.red[rb][ww][c8 + i];
      x[i] = s;
    }
    rb ^= 1;
  };

  float dS[8];
  {
    const long o = ((long)hd * K + kap) * V + v0 + c8;
#pragma unroll
    for (int i = 0; i < 8; ++i) dS[i] = p.dST ? p.dST[o + i] : 0.0f;
  }
  for (int seg = p.NC - 1; seg >= 0; --seg) {
    const int t0 = seg * kSeg;
    const int n = min(kSeg, T_ - t0);
    // this key's retain factor, k and q for the segment's tokens
    float al[kSeg], kk[kSeg], qq[kSeg];
#pragma unroll
    for (int tt = 0; tt < kSeg; ++tt) {
      al[tt] = 1.0f;
      kk[tt] = 0.0f;
      qq[tt] = 0.0f;
      if (tt < n) {
        const long row = b * T_ + t0 + tt;
        al[tt] = gate_alpha_pre<GK>(p.g_raw[(row * HV + hv) * K + kap], bias, gc);
        kk[tt] = In<T>::at(kg, (row * H + h) * K + kap);
        qq[tt] = In<T>::at(qg, (row * H + h) * K + kap);
      }
    }
    for (int e = tid; e < kSeg * kBV; e += 2 * K) {
      const int tt = e / kBV, j = e % kBV;
      const long row = b * T_ + t0 + tt;
      sm.v[tt][j] = tt < n ? In<T>::at(vg, (row * HV + hv) * V + v0 + j) : 0.0f;
      sm.dout[tt][j] = tt < n ? p.dout[(row * HV + hv) * V + v0 + j] : 0.0f;
    }
    if (tid < kSeg) sm.beta[tid] = tid < n ? p.beta[(b * T_ + t0 + tid) * HV + hv] : 0.0f;
    float S[8];
    {
      const float* c = p.ckpt + (((long)hd * p.NC + seg) * K + kap) * V + v0 + c8;
      const float4 a = *reinterpret_cast<const float4*>(c);
      const float4 z = *reinterpret_cast<const float4*>(c + 4);
      S[0] = a.x; S[1] = a.y; S[2] = a.z; S[3] = a.w;
      S[4] = z.x; S[5] = z.y; S[6] = z.z; S[7] = z.w;
    }
    __syncthreads();
    // forward through the segment: keep S_{t-1} and the residual of every token
#pragma unroll
    for (int tt = 0; tt < kSeg; ++tt) {
      if (tt < n) {
        float* dst = &sm.st[tt][kap][c8];
        *reinterpret_cast<float4*>(dst) = float4{S[0], S[1], S[2], S[3]};
        *reinterpret_cast<float4*>(dst + 4) = float4{S[4], S[5], S[6], S[7]};
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          S[i] *= al[tt];
          x[i] = kk[tt] * S[i];
        }
        key_sum(x);  // prediction Sd^T k
        const float bk = sm.beta[tt] * kk[tt];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float r = sm.v[tt][c8 + i] - x[i];
          S[i] += bk * r;
          x[i] = r;
        }
        if (kap == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sm.r[tt][c8 + i] = x[i];
        }
      }
    }
    __syncthreads();
    // reverse through the segment
#pragma unroll
    for (int tt = kSeg - 1; tt >= 0; --tt) {
      if (tt < n) {
        const long row = b * T_ + t0 + tt;
        const float bt = sm.beta[tt];
        float Sd[8], r[8], a[8], St, dq = 0.0f, dkr = 0.0f, dg = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          Sd[i] = al[tt] * sm.st[tt][kap][c8 + i];
          r[i] = sm.r[tt][c8 + i];
          const float d = sm.dout[tt][c8 + i];
          St = Sd[i] + bt * kk[tt] * r[i];
          dq += St * d;
          dS[i] += scale * qq[tt] * d;
          a[i] = kk[tt] * dS[i];
        }
        dq = pair_add(dq) * scale;
        key_sum(a);  // a_t = dS^T k_t, per column
        float db = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float dr = bt * a[i];
          db += a[i] * r[i];
          dkr += bt * dS[i] * r[i] - Sd[i] * dr;
          const float dsd = dS[i] - kk[tt] * dr;
          dg += dsd * Sd[i];
          dS[i] = al[tt] * dsd;
          a[i] = dr;
        }
        dkr = pair_add(dkr);
        dg = pair_add(dg);
        db = pair_add(db);
        if (ch == 0) {
          atomicAdd(p.dq + (row * H + h) * K + kap, dq);
          atomicAdd(p.dk + (row * H + h) * K + kap, dkr);
          atomicAdd(p.dg + (row * HV + hv) * K + kap, dg);
        }
        if (kap == 0) {
          float* dvp = p.dv + (row * HV + hv) * V + v0 + c8;
          *reinterpret_cast<float4*>(dvp) = float4{a[0], a[1], a[2], a[3]};
          *reinterpret_cast<float4*>(dvp + 4) = float4{a[4], a[5], a[6], a[7]};
          if (ch == 0) atomicAdd(p.dbeta + row * HV + hv, db);
        }
      }
    }
    __syncthreads();  // the next segment rewrites the LDS
  }
  if (p.dS0) {
    float* o = p.dS0 + ((long)hd * K + kap) * V + v0 + c8;
    *reinterpret_cast<float4*>(o) = float4{dS[0], dS[1], dS[2], dS[3]};
    *reinterpret_cast<float4*>(o + 4) = float4{dS[4], dS[5], dS[6], dS[7]};
  }
}

// dg -> dg_raw in place (chain rule through the gate), and the sums of the
// dt_bias and A_log gradients over the rows (sequence, token) of a block.
// One workgroup per (64 rows, value head), one thread per key channel.
template <int GK>
__global__ void bwd_gate_kernel(BwdParams p, int K, long rows) {
  const int hv = blockIdx.y, c = threadIdx.x;
  const long r0 = (long)blockIdx.x * 64, r1 = r0 + 64 < rows ? r0 + 64 : rows;
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const float bias = (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[hv * K + c] : 0.0f;
  float sb = 0.0f, sa = 0.0f;
  for (long r = r0; r < r1; ++r) {
    const long i = (r * p.HV + hv) * K + c;
    const float dg = p.dg[i], x = p.g_raw[i] + bias;
    float dx = dg, da = 0.0f;
    if constexpr (GK == KDA_GATE_SAFE) {  // g = L sigma(rate x)
      const float z = rate * x;
      const float sg = __builtin_amdgcn_rcpf(1.0f + exp_f(-z));
      const float d = p.lower_bound * sg * (1.0f - sg);
      dx = dg * d * rate;
      da = dg * d * z;
    } else if constexpr (GK == KDA_GATE_STANDARD) {  // g = -rate softplus(x)
      const float sg = __builtin_amdgcn_rcpf(1.0f + exp_f(-x));
      dx = -dg * rate * sg;
      da = -dg * rate * softplus_f(x);
    }
    p.dg[i] = dx;
    sb += dx;
    sa += da;
  }
  if (GK == KDA_GATE_NONE) return;  // neither dt_bias nor A_log enters this gate
  if (p.ddt_bias) atomicAdd(p.ddt_bias + hv * K + c, sb);
  if (!p.dA_log) return;
  __shared__ float red[128];
  red[c] = sa;
  __syncthreads();
  if (c == 0) {
    float s = 0.0f;
    for (int i = 0; i < K; ++i) s += red[i];
    atomicAdd(p.dA_log + hv, s);
  }
}

hipError_t launch_split(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        int per_head, float lower_bound, const float* S0, float* o, float* S_out,
                        float* h, void* workspace, int B, int T, int H, int HV, int K, int C,
                        hipStream_t stream);
size_t split_workspace_bytes_per_chunk(int K, int V, int C);

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace: checkpoints [B, HV, NC, K, V], the forward outputs the split
// schedule writes on the way, its own workspace.
size_t bwd_workspace_bytes(int B, int T, int HV, int K, int V) {
  const size_t nc = ((size_t)T + kSeg - 1) / kSeg;
  return align256((size_t)B * HV * nc * K * V * sizeof(float)) +
         align256((size_t)B * T * HV * V * sizeof(float)) +
         (size_t)B * HV * nc * split_workspace_bytes_per_chunk(K, V, kSeg);
}

static hipError_t zero(float* p, long n, hipStream_t stream) {
  if (!p || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <int K, typename T, int GK>
static hipError_t launch_bwd_kt(BwdParams p, hipStream_t stream) {
  const size_t lds = sizeof(BwdSmem<K>);
  const long nblk = (long)p.B * p.HV * (K / kBV);
  if (nblk > 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bwd_segment_kernel<K, K, T, GK>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_segment_kernel<K, K, T, GK>), dim3((unsigned)nblk), dim3(2 * K), lds,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long rows = (long)p.B * p.T;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_gate_kernel<GK>), dim3((unsigned)((rows + 63) / 64), (unsigned)p.HV),
                     dim3(K), 0, stream, p, K, rows);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                      const float* beta, const float* A_log, const float* dt_bias, int kind,
                      float lower_bound, const float* S0, const float* dout, const float* dST,
                      float* dq, float* dk, float* dv, float* dbeta, float* dg_raw, float* dA_log,
                      float* ddt_bias, float* dS0, void* workspace, int B, int T, int H, int HV,
                      int K, hipStream_t stream) {
  const int NC = (T + kSeg - 1) / kSeg;
  char* ws = static_cast<char*>(workspace);
  float* ckpt = reinterpret_cast<float*>(ws);
  float* o = reinterpret_cast<float*>(ws + align256((size_t)B * HV * NC * K * K * sizeof(float)));
  void* split_ws = reinterpret_cast<char*>(o) + align256((size_t)B * T * HV * K * sizeof(float));
  hipError_t e;
  const long nq = (long)B * T * H * K, ng = (long)B * T * HV * K;
  if ((e = zero(dq, nq, stream)) != hipSuccess || (e = zero(dk, nq, stream)) != hipSuccess ||
      (e = zero(dbeta, (long)B * T * HV, stream)) != hipSuccess ||
      (e = zero(dg_raw, ng, stream)) != hipSuccess || (e = zero(dA_log, HV, stream)) != hipSuccess ||
      (e = zero(ddt_bias, (long)HV * K, stream)) != hipSuccess)
    return e;
  if (T > 0) {
    e = launch_split(q, k, v, bf16, g_raw, beta, A_log, dt_bias, kind, 0, lower_bound, S0, o,
                     nullptr, ckpt, split_ws, B, T, H, HV, K, kSeg, stream);
    if (e != hipSuccess) return e;
  }
  BwdParams p{q, k, v, g_raw, beta, A_log, dt_bias, dout, dST, ckpt, dq, dk, dv, dbeta, dg_raw,
              dS0, dA_log, ddt_bias, B, T, H, HV, NC, lower_bound};
#define KDA_BWD_GATE(KK, TT)                                                       \
  switch (kind) {                                                                  \
    case KDA_GATE_SAFE: return launch_bwd_kt<KK, TT, KDA_GATE_SAFE>(p, stream);    \
    case KDA_GATE_STANDARD: return launch_bwd_kt<KK, TT, KDA_GATE_STANDARD>(p, stream); \
    default: return launch_bwd_kt<KK, TT, KDA_GATE_NONE>(p, stream);               \
  }
#define KDA_BWD_CASE(KK)                      \
  if (K == KK) {                              \
    if (bf16) { KDA_BWD_GATE(KK, uint16_t) }  \
    else { KDA_BWD_GATE(KK, float) }          \
  }
  KDA_BWD_CASE(32) KDA_BWD_CASE(64) KDA_BWD_CASE(128)
#undef KDA_BWD_CASE
#undef KDA_BWD_GATE
  return hipErrorInvalidValue;
}

}  // namespace kda
