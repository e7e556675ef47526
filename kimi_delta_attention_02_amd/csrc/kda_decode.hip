// One recurrent (decode) step of KDA for every sequence, state updated in place.
//
// Per (b, hv) the step applies the four-step update of the "K3 notes" section
// "KDA 递归核心" (decay, key prediction and residual, rank-1 write, query read
// with 1/sqrt(K)), the schedule of the "DeltaNet family" page's fused recurrent
// mode: independent programs per (sequence, value head, value tile), each
// owning a tile of the state for the whole step.
//
// The step is bound by HBM: the fp32 state [K, V] of every (b, hv) is read once
// and written once.  A K x TV column tile (TV = V, at most 128) is split by
// rows over WT wavefronts (four for K = 128), so each lane keeps RPL 16-byte
// rows in flight.  In a wavefront, lane l holds column quad cq = l % NQ (NQ
// lanes cover one row segment of the tile) and rows row0 + RG i of row group
// rg = l / NQ, so every load instruction reads RG full row segments; the whole
// tile is loaded before any arithmetic.  The two reductions over kappa
// (prediction k.S_dec and read q.S_new) run as log2(RG) butterfly steps inside
// each wavefront (row swaps for the 16- and 32-lane distances), then one LDS
// exchange across the WT wavefronts of the tile.  The decay factors exp(g) and
// the key and query rows are computed once per workgroup into LDS.  Measured on
// the decode workload, whole-head tiles (TV = 128) beat 64- and 32-wide ones:
// one workgroup per (b, hv) computes exp(g) once and leaves fewer, longer
// workgroups, which shortens the end-of-launch tail.
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
  int per_head;  // g_raw [B, HV] and dt_bias [HV]: one gate per (b, hv)
  float lower_bound;
};

// Sum over the lanes of a wavefront that share l % NQ (the row groups), for
// the four components at once.
template <int NQ>
__device__ __forceinline__ f32x4 sum_row_groups(f32x4 v) {
  if constexpr (NQ < 64) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = xor_sum<NQ>(v[c]);
    return sum_row_groups<2 * NQ>(v);
  } else {
    return v;
  }
}

// State loads: a state of at most kCachedStateBytes is read with ordinary
// loads, which let the last-level cache keep part of it from one call to the
// next; a larger one is read non-temporally, which streams better once the
// cache can hold no useful part of it.  Stores are always non-temporal.
// Measured with a read-modify-write sweep on MI355X: ordinary loads with
// non-temporal stores win by 22-31% up to 512 MiB and 3% at 768 MiB, and lose
// by 4-7% from 1 GiB on.
constexpr size_t kCachedStateBytes = 768ull << 20;

template <bool NTL>
__device__ __forceinline__ f32x4 load_state(const float* p) {
  if constexpr (NTL) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else return *reinterpret_cast<const f32x4*>(p);
}

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = 64 * kDecodeWaves;

template <int K, int V>
struct DecodeTiling {
  static constexpr int TV = V < 128 ? V : 128;   // columns of a tile
  static constexpr int NQ = TV / 4;              // column quads per row segment
  static constexpr int RG = 64 / NQ;             // row groups per wavefront
  static constexpr int NW = kDecodeWaves;             // wavefronts per workgroup
  static constexpr int WT = K / RG < NW ? K / RG : NW;  // wavefronts splitting a tile's rows
  static constexpr int RPL = K / (WT * RG);      // rows per lane
  static constexpr int NVT = V / TV;             // tiles per (b, hv)
  static constexpr int TPW = NW / WT;            // tiles per workgroup
  static_assert(RPL >= 1 && K % (WT * RG) == 0, "head size too small for this tiling");
};

template <int K, int V, typename T, int GK, bool NTL>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(DecodeParams p) {
  using D = DecodeTiling<K, V>;
  constexpr int TV = D::TV, NQ = D::NQ, RG = D::RG, WT = D::WT, RPL = D::RPL, NVT = D::NVT,
                TPW = D::TPW;
  __shared__ float s_al[TPW][K], s_k[TPW][K], s_q[TPW][K];
  __shared__ f32x4 s_red[2][kDecodeWaves][NQ];  // per wavefront partials of the two reductions

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long nheads = (long)p.B * p.HV;
  const long tile0 = (long)blockIdx.x * TPW;
  const long ntiles = nheads * NVT;

  const int ts = w / WT, rq = w % WT;  // tile slot, row quarter
  const long tile = tile0 + ts;
  const bool active = tile < ntiles;
  const long bh = tile / NVT;          // b * HV + hv
  const int vt = (int)(tile % NVT);
  const int cq = lane % NQ, rg = lane / NQ;
  const int col = vt * TV + cq * 4;
  const int row0 = rq * (K / WT) + rg;
  float* S = p.state + bh * (long)K * V;
  f32x4 s[RPL];
  float vv[4] = {0.f, 0.f, 0.f, 0.f};
  float bt = 0.0f;
  // the state tile's loads go out first: the decay/key/query loop below waits
  // on its own (small) loads, and the two latencies overlap
  if (active) {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      s[i] = load_state<NTL>(S + (long)(row0 + RG * i) * V + col);
    In<T>::load4(static_cast<const T*>(p.v), bh * V + col, vv);
    bt = p.beta[bh];
  }

  // decay factors and key/query rows of each tile's (b, hv), once per workgroup
  for (int e = tid; e < TPW * K; e += kDecodeThreads) {
    const int ts = e / K, r = e % K;
    const long tile = tile0 + ts;
    if (tile < ntiles) {
      const long bh = tile / NVT;
      const int hv = (int)(bh % p.HV);
      const long b = bh / p.HV;
      const int h = hv / (p.HV / p.H);
      const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
      const long gi = p.per_head ? bh : bh * K + r, bi = p.per_head ? hv : (long)hv * K + r;
      const float bias = (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[bi] : 0.0f;
      s_al[ts][r] = exp_f(gate_log_decay_k<GK>(p.g_raw[gi], bias, rate, p.lower_bound));
      s_k[ts][r] = In<T>::at(static_cast<const T*>(p.k), (b * p.H + h) * K + r);
      s_q[ts][r] = In<T>::at(static_cast<const T*>(p.q), (b * p.H + h) * K + r);
    }
  }

  __syncthreads();

  // decay, then prediction p = k . S_dec: in-wave butterfly, then across the WT waves
  f32x4 pr = {0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = row0 + RG * i;
      s[i] *= s_al[ts][r];
      pr += s_k[ts][r] * s[i];
    }
  }
  pr = sum_row_groups<NQ>(pr);
  if (rg == 0) s_red[0][w][cq] = pr;
  __syncthreads();
  pr = s_red[0][ts * WT][cq];
#pragma unroll
  for (int j = 1; j < WT; ++j) pr += s_red[0][ts * WT + j][cq];

  // residual, rank-1 write, read q . S_new
  f32x4 rv;
#pragma unroll
  for (int c = 0; c < 4; ++c) rv[c] = bt * (vv[c] - pr[c]);
  f32x4 ov = {0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = row0 + RG * i;
      s[i] += s_k[ts][r] * rv;
      ov += s_q[ts][r] * s[i];
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (long)(row0 + RG * i) * V + col));
  }
  ov = sum_row_groups<NQ>(ov);
  if (rg == 0) s_red[1][w][cq] = ov;
  __syncthreads();
  if (active && rq == 0 && rg == 0) {
    f32x4 o = s_red[1][ts * WT][cq];
#pragma unroll
    for (int j = 1; j < WT; ++j) o += s_red[1][ts * WT + j][cq];
    const float scale = 1.0f / __builtin_sqrtf((float)K);
    *reinterpret_cast<f32x4*>(p.o + bh * V + col) = o * scale;
  }
}

// ---------------------------------------------------------------------------
// Fused recurrent forward over T tokens per call: the same per-token step with
// the state tile held in registers across all tokens, read from the initial
// state once and written to the final state once ("DeltaNet family" page, the
// fused recurrent kernel: one program per (sequence, head, value tile) looping
// over time).  Per token: the row factors of the next token are formed in a
// second LDS buffer while the current token runs, so each token costs two
// barriers (after the prediction partials and after the read partials); the
// HBM inputs of a token are loaded one token ahead.
//
// The tile is kept as S_hat = S / D, with D the running product of exp(g) per
// key row since the last renormalisation.  The decay then costs no
// multiplication of the tile: the prediction uses k D, the write k / D and the
// read q D (three factors per row, formed once per row), so each state element
// takes three fused multiply-adds per token instead of four operations.  A row
// whose D leaves [2^-64, 2^64] (or is NaN) makes the workgroup fold D into
// S_hat before that token (S_hat *= D, D = 1; the factor is 1 for the other
// rows), and D is folded in once more before the final state is stored.

struct RecurrentParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g_raw;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  const float* S0;
  float* S_out;
  float* o;
  int B, T, H, HV, kind;
  int per_head;  // g_raw [B, T, HV] and dt_bias [HV]: one gate per (token, value head)
  float lower_bound;
};

template <int K, int V, typename T, int GK, bool NTL>
__global__ __launch_bounds__(kDecodeThreads) void recurrent_fwd_kernel(RecurrentParams p) {
  using D = DecodeTiling<K, V>;
  constexpr int TV = D::TV, NQ = D::NQ, RG = D::RG, WT = D::WT, RPL = D::RPL, NVT = D::NVT,
                TPW = D::TPW;
  static_assert(TPW * K <= kDecodeThreads, "one decay/key/query element per thread");
  // per token buffer: renormalisation factor, k D, k / D, q D of every row
  __shared__ float s_f[2][TPW][K], s_k1[2][TPW][K], s_k2[2][TPW][K], s_q1[2][TPW][K];
  __shared__ int s_rn[2][kDecodeWaves];  // per wavefront: some row renormalises
  __shared__ float s_D[TPW][K];
  __shared__ f32x4 s_red[2][kDecodeWaves][NQ];
  constexpr float kDLo = 5.421010862427522e-20f, kDHi = 1.8446744073709552e19f;  // 2^-64, 2^64

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T_ = p.T, HV = p.HV, H = p.H;
  const long nheads = (long)p.B * HV;
  const long tile0 = (long)blockIdx.x * TPW;
  const long ntiles = nheads * NVT;

  // ---- the decay / key / query element of this thread: tile slot gts, row gr
  const bool gthread = tid < TPW * K;
  const int gts = tid / K, gr = tid % K;
  const bool gactive = gthread && tile0 + gts < ntiles;
  const long gbh = gactive ? (tile0 + gts) / NVT : 0;  // b * HV + hv
  const int ghv = (int)(gbh % HV);
  const long gb = gbh / HV;
  const int gh = ghv / (HV / H);
  const GateConsts gc = gate_consts(GK != KDA_GATE_NONE ? exp_f(p.A_log[ghv]) : 1.0f, p.lower_bound);
  const int gK = p.per_head ? 1 : K;  // gate elements per (token, value head)
  const float gbias = (p.dt_bias && GK != KDA_GATE_NONE && gactive)
                          ? p.dt_bias[(long)ghv * gK + (p.per_head ? 0 : gr)] : 0.0f;
  const float* g_ptr = p.g_raw + (gb * T_ * HV + ghv) * (long)gK + (p.per_head ? 0 : gr);
  const T* k_ptr = static_cast<const T*>(p.k) + (gb * T_ * H + gh) * (long)K + gr;
  const T* q_ptr = static_cast<const T*>(p.q) + (gb * T_ * H + gh) * (long)K + gr;
  float pg = 0.0f;
  typename In<T>::Raw1 pk = In<T>::zero1(), pq = In<T>::zero1();
  auto fetch_g = [&](int t) {
    if (gactive) {
      pg = g_ptr[(long)t * HV * gK];
      pk = k_ptr[(long)t * H * K];
      pq = q_ptr[(long)t * H * K];
    }
  };
  float gD = 1.0f;  // running decay of this thread's row
  auto put_g = [&](int buf) {  // called by every thread of the workgroup
    bool rn = false;
    if (gthread) {
      float f = 1.0f, k1 = 0.0f, k2 = 0.0f, q1 = 0.0f;
      if (gactive) {
        const float kk = In<T>::widen(pk), qq = In<T>::widen(pq);
        const float dn = gD * gate_alpha<GK>(pg, gbias, gc);
        rn = !(dn >= kDLo && dn <= kDHi);
        if (rn) {  // fold this token's decayed state into S_hat
          f = dn;
          gD = 1.0f;
          k1 = kk;
          k2 = kk;
          q1 = qq;
        } else {
          gD = dn;
          k1 = kk * dn;
          k2 = kk * __builtin_amdgcn_rcpf(dn);
          q1 = qq * dn;
        }
      }
      s_f[buf][gts][gr] = f;
      s_k1[buf][gts][gr] = k1;
      s_k2[buf][gts][gr] = k2;
      s_q1[buf][gts][gr] = q1;
    }
    const bool any = __any(rn);
    if (lane == 0) s_rn[buf][w] = any ? 1 : 0;
  };

  // ---- the state tile of this thread (layout of the decode step)
  const int ts = w / WT, rq = w % WT;
  const long tile = tile0 + ts;
  const bool active = tile < ntiles;
  const long bh = active ? tile / NVT : 0;
  const int vt = (int)(tile % NVT);
  const int cq = lane % NQ, rg = lane / NQ;
  const int col = vt * TV + cq * 4;
  const int row0 = rq * (K / WT) + rg;
  const long b = bh / HV;
  const int hv = (int)(bh % HV);
  f32x4 s[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active && p.S0) {
    const float* S = p.S0 + bh * (long)K * V;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      s[i] = load_state<NTL>(S + (long)(row0 + RG * i) * V + col);
  }
  const T* v_ptr = static_cast<const T*>(p.v) + (b * T_ * HV + hv) * (long)V + col;
  const float* beta_ptr = p.beta + b * T_ * HV + hv;
  float* o_ptr = p.o + (b * T_ * HV + hv) * (long)V + col;
  float pv[4] = {0.f, 0.f, 0.f, 0.f}, pb = 0.0f;
  auto fetch_v = [&](int t) {
    if (active) {
      In<T>::load4(v_ptr, (long)t * HV * V, pv);
      pb = beta_ptr[(long)t * HV];
    }
  };
  const float scale = 1.0f / __builtin_sqrtf((float)K);

  if (T_ > 0) {
    fetch_g(0);
    fetch_v(0);
    put_g(0);
    if (T_ > 1) fetch_g(1);
  }
  __syncthreads();
  for (int t = 0; t < T_; ++t) {
    const int buf = t & 1;
    const float vv[4] = {pv[0], pv[1], pv[2], pv[3]};
    const float bt = pb;
    if (t + 1 < T_) fetch_v(t + 1);

    // the prediction k . S_dec = (k D) . S_hat (after a renormalisation where
    // some row needs one): in-wave butterfly, then across the WT waves
    int rn = 0;
#pragma unroll
    for (int j = 0; j < kDecodeWaves; ++j) rn |= s_rn[buf][j];
    if (rn) {
#pragma unroll
      for (int i = 0; i < RPL; ++i) s[i] *= s_f[buf][ts][row0 + RG * i];
    }
    f32x4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPL; ++i) pr += s_k1[buf][ts][row0 + RG * i] * s[i];
    pr = sum_row_groups<NQ>(pr);
    if (rg == 0) s_red[0][w][cq] = pr;
    __syncthreads();

    // residual, rank-1 write, read q . S_new
    pr = s_red[0][ts * WT][cq];
#pragma unroll
    for (int j = 1; j < WT; ++j) pr += s_red[0][ts * WT + j][cq];
    f32x4 rv;
#pragma unroll
    for (int c = 0; c < 4; ++c) rv[c] = bt * (vv[c] - pr[c]);
    f32x4 ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = row0 + RG * i;
      s[i] += s_k2[buf][ts][r] * rv;  // S_hat += (k / D) r^T
      ov += s_q1[buf][ts][r] * s[i];  // q . S_new = (q D) . S_hat
    }
    ov = sum_row_groups<NQ>(ov);
    if (rg == 0) s_red[1][w][cq] = ov;
    if (t + 1 < T_) {  // the next token's rows; that buffer was last read before the last barrier
      put_g(buf ^ 1);
      if (t + 2 < T_) fetch_g(t + 2);
    }
    __syncthreads();
    if (active && rq == 0 && rg == 0) {
      f32x4 o = s_red[1][ts * WT][cq];
#pragma unroll
      for (int j = 1; j < WT; ++j) o += s_red[1][ts * WT + j][cq];
      *reinterpret_cast<f32x4*>(o_ptr + (long)t * HV * V) = o * scale;
    }
  }
  // S = diag(D) S_hat
  if (gthread) s_D[gts][gr] = gD;
  __syncthreads();
  if (active && p.S_out) {
    float* S = p.S_out + bh * (long)K * V;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = row0 + RG * i;
      __builtin_nontemporal_store(s[i] * s_D[ts][r], reinterpret_cast<f32x4*>(S + (long)r * V + col));
    }
  }
}

template <int K, int V, typename T, int GK>
static hipError_t launch_recurrent_kv(const RecurrentParams& p, hipStream_t stream) {
  using D = DecodeTiling<K, V>;
  const long tiles = (long)p.B * p.HV * D::NVT;
  const long blocks = (tiles + D::TPW - 1) / D::TPW;
  if ((size_t)p.B * p.HV * K * V * sizeof(float) > kCachedStateBytes)
    hipLaunchKernelGGL((recurrent_fwd_kernel<K, V, T, GK, true>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_fwd_kernel<K, V, T, GK, false>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int GK>
static hipError_t launch_recurrent_t(const RecurrentParams& p, int K, int V, hipStream_t stream) {
#define KDA_REC_CASE(KK, VV) \
  if (K == KK && V == VV) return launch_recurrent_kv<KK, VV, T, GK>(p, stream);
#define KDA_REC_ROW(KK) KDA_REC_CASE(KK, 16) KDA_REC_CASE(KK, 32) KDA_REC_CASE(KK, 64) KDA_REC_CASE(KK, 128)
  KDA_REC_ROW(16) KDA_REC_ROW(32) KDA_REC_ROW(64) KDA_REC_ROW(128)
#undef KDA_REC_ROW
#undef KDA_REC_CASE
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_recurrent_g(const RecurrentParams& p, int K, int V, hipStream_t stream) {
  switch (p.kind) {
    case KDA_GATE_SAFE: return launch_recurrent_t<T, KDA_GATE_SAFE>(p, K, V, stream);
    case KDA_GATE_STANDARD: return launch_recurrent_t<T, KDA_GATE_STANDARD>(p, K, V, stream);
    default: return launch_recurrent_t<T, KDA_GATE_NONE>(p, K, V, stream);
  }
}

hipError_t launch_recurrent(const void* q, const void* k, const void* v, int bf16,
                            const float* g_raw, const float* beta, const float* A_log,
                            const float* dt_bias, int kind, int per_head, float lower_bound,
                            const float* S0, float* o, float* S_out, int B, int T, int H, int HV,
                            int K, int V, hipStream_t stream) {
  RecurrentParams p{q, k, v, g_raw, beta, A_log, dt_bias, S0, S_out, o, B, T, H, HV, kind,
                    per_head, lower_bound};
  return bf16 ? launch_recurrent_g<uint16_t>(p, K, V, stream)
              : launch_recurrent_g<float>(p, K, V, stream);
}

template <int K, int V, typename T, int GK>
static hipError_t launch_decode_kv(const DecodeParams& p, hipStream_t stream) {
  using D = DecodeTiling<K, V>;
  const long tiles = (long)p.B * p.HV * D::NVT;
  const long blocks = (tiles + D::TPW - 1) / D::TPW;
  if ((size_t)p.B * p.HV * K * V * sizeof(float) > kCachedStateBytes)
    hipLaunchKernelGGL((decode_step_kernel<K, V, T, GK, true>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_step_kernel<K, V, T, GK, false>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int GK>
static hipError_t launch_decode_t(const DecodeParams& p, int K, int V, hipStream_t stream) {
#define KDA_DEC_CASE(KK, VV) \
  if (K == KK && V == VV) return launch_decode_kv<KK, VV, T, GK>(p, stream);
#define KDA_DEC_ROW(KK) KDA_DEC_CASE(KK, 16) KDA_DEC_CASE(KK, 32) KDA_DEC_CASE(KK, 64) KDA_DEC_CASE(KK, 128)
  KDA_DEC_ROW(16) KDA_DEC_ROW(32) KDA_DEC_ROW(64) KDA_DEC_ROW(128)
#undef KDA_DEC_ROW
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_g(const DecodeParams& p, int K, int V, hipStream_t stream) {
  switch (p.kind) {
    case KDA_GATE_SAFE: return launch_decode_t<T, KDA_GATE_SAFE>(p, K, V, stream);
    case KDA_GATE_STANDARD: return launch_decode_t<T, KDA_GATE_STANDARD>(p, K, V, stream);
    default: return launch_decode_t<T, KDA_GATE_NONE>(p, K, V, stream);
  }
}

hipError_t launch_decode(const void* q, const void* k, const void* v, int bf16,
                         const float* g_raw, const float* beta, const float* A_log,
                         const float* dt_bias, int kind, int per_head, float lower_bound,
                         float* state, float* o, int B, int H, int HV, int K, int V,
                         hipStream_t stream) {
  DecodeParams p{q, k, v, g_raw, beta, A_log, dt_bias, state, o, B, H, HV, kind, per_head,
                 lower_bound};
  return bf16 ? launch_decode_g<uint16_t>(p, K, V, stream) : launch_decode_g<float>(p, K, V, stream);
}

}  // namespace kda
