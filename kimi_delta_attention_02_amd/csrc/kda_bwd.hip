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
// the split schedule (kda_split.hip, chunk 16, without its output stage)
// writes the state entering every 16-token segment and leaves U_t = beta_t r_t
// of every token in its workspace.  One workgroup per (sequence, value head,
// 16-wide value tile) then walks the segments from the last.  Thread
// 4 kappa + c holds key row kappa, value columns 4 c .. 4 c + 3 of the tile.
// Per segment it stages the retain factors, k and q of the sixteen tokens in
// LDS, rebuilds the sixteen states from the checkpoint in registers with
// S_t = diag(alpha_t) S_{t-1} + k_t U_t^T (no reduction), then runs the
// reverse recurrence with its tile of dS in registers.  Each reverse token
// needs one sum over the keys, of dS^T k_t and of the prediction Sd_t^T k_t
// together (the residual r_t is formed again from the latter): DPP row
// rotations, row swaps and one LDS exchange across the wavefronts; sums over
// the tile's columns are in-thread plus two lane exchanges.  The per-key
// results (dq, dk, dg) and dbeta, summed over the value tiles (and the value
// heads of a GVA group), are accumulated with fp32 atomics into zeroed
// outputs, so their last bits depend on the order the tiles finish in.  A
// last kernel applies the gate's chain rule and sums dt_bias and A_log over
// the sequences.
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
  const float* u;     // U = beta r of every token, as the split schedule's state pass left it
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

// x + the value N lanes further round its 16-lane row (DPP row rotation).
// Every source lane of these permutations exists, so bound_ctrl (which only
// matters for missing ones) is set: it lets the add take the DPP operand.
template <int N>
__device__ __forceinline__ float ror_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, true));
}
// the sum of x over each group of eight lanes (quad permutations [1, 0, 3, 2]
// and [2, 3, 0, 1], then the mirror inside each half-row of 8)
__device__ __forceinline__ float oct_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1,
                                                             0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E,
                                                             0xF, 0xF, true));
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   0x141, 0xF, 0xF, true));
}
// the sum of x over each group of four lanes (quad permutations [1, 0, 3, 2]
// then [2, 3, 0, 1])
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1,
                                                             0xF, 0xF, true));
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                   0x4E, 0xF, 0xF, true));
}

template <int K>
struct BwdSmem {
  float al[kSeg][K];  // retain factors of the segment's tokens
  float k[kSeg][K];
  float q[kSeg][K];    // s q
  float u[kSeg][kBV];  // U = beta r from the forward's state pass
  float v[kSeg][kBV];
  float dout[kSeg][kBV];
  float beta[kSeg];
  float red[2][K / 16][2][kBV];  // per-wavefront key sums of a and Sd^T k (two buffers)
  float fin[K / 16][8][4];        // each wavefront's totals of the 8 groups of 4 (quantity, column)
  // the segment's results, written out together once it is done
  float dq[kSeg][K];
  float dk[kSeg][K];
  float dg[kSeg][K];
  float dv[kSeg][kBV];
  float db[kSeg];
};

// One segment's inputs in flight: this thread's share of g_raw, k and q
// (key channel tid % K, tokens tid / K + 4 i), of v, dL/do, U and beta, and
// its own row of the checkpoint.
template <typename T, int NVD>
struct SegLoads {
  float g[4];
  typename In<T>::Raw1 k[4], q[4], v[NVD];
  float dout[NVD], beta;
  float4 u, ckpt;
};

template <int K, typename T, int GK>
__global__ __launch_bounds__(4 * K) __attribute__((amdgpu_waves_per_eu(4))) void bwd_segment_kernel(
    BwdParams p) {
  constexpr int V = K, NT = 4 * K, NW = NT / 64, NVT = V / kBV;
  constexpr int NVD = (kSeg * kBV + NT - 1) / NT;  // v and dL/do elements each thread stages
  static_assert(kSeg * K / NT == 4 && NT >= 64, "thread layout");
  __shared__ BwdSmem<K> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kap = tid >> 2, cg = tid & 3, c4 = 4 * cg;
  const int vt = blockIdx.x % NVT, hd = blockIdx.x / NVT;
  const int HV = p.HV, H = p.H, T_ = p.T, NC = p.NC;
  const long b = hd / HV;
  const int hv = hd % HV, h = hv / (HV / H), v0 = vt * kBV;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const GateConsts gc = gate_consts(rate, p.lower_bound);
  const int cown = tid % K, town = tid / K;  // the key channel and first token this thread stages
  const float bias = gate_bias_pre<GK>(
      (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[hv * K + cown] : 0.0f, gc);
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);

  // Issue the loads of segment seg (rows past the end re-read the last
  // token, n >= 1; what they hold is never used).  Addresses are a base
  // uniform over the workgroup plus a 32-bit per-thread offset.
  auto issue = [&](int seg, SegLoads<T, NVD>& L) {
    const int t0 = seg * kSeg, n = min(kSeg, T_ - t0);
    const long row0 = b * T_ + t0;
    const float* gb = p.g_raw + (row0 * HV + hv) * K;
    const T* kb = kg + (row0 * H + h) * K;
    const T* qb = qg + (row0 * H + h) * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(town + 4 * i, n - 1);
      L.g[i] = gb[r * HV * K + cown];
      L.k[i] = kb[r * H * K + cown];
      L.q[i] = qb[r * H * K + cown];
    }
    const T* vb = vg + (row0 * HV + hv) * V + v0;
    const float* db = p.dout + (row0 * HV + hv) * V + v0;
#pragma unroll
    for (int i = 0; i < NVD; ++i) {  // elements past the tile re-read its first ones
      const int e = (tid + i * NT) % (kSeg * kBV);
      const int o = min(e / kBV, n - 1) * HV * V + e % kBV;
      L.v[i] = vb[o];
      L.dout[i] = db[o];
    }
    L.u = *reinterpret_cast<const float4*>(p.u + (((long)hd * NC + seg) * NVT + vt) * 256 +
                                           4 * (tid & 63));
    L.beta = p.beta[row0 * HV + hv + min(tid & 15, n - 1) * HV];
    L.ckpt = *reinterpret_cast<const float4*>(p.ckpt + ((long)hd * NC + seg) * K * V + v0 +
                                              kap * V + c4);
  };
  // Place them in LDS (gate applied, q scaled).
  auto stage = [&](const SegLoads<T, NVD>& L) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.al[town + 4 * i][cown] = gate_alpha_pre<GK>(L.g[i], bias, gc);
      sm.k[town + 4 * i][cown] = In<T>::widen(L.k[i]);
      sm.q[town + 4 * i][cown] = scale * In<T>::widen(L.q[i]);
    }
#pragma unroll
    for (int i = 0; i < NVD; ++i) {
      const int e = tid + i * NT;
      if (e < kSeg * kBV) {
        sm.v[e / kBV][e % kBV] = In<T>::widen(L.v[i]);
        sm.dout[e / kBV][e % kBV] = L.dout[i];
      }
    }
    if (tid < 64) {  // U: one 16 x 16 fragment, lane l holding rows 4 (l / 16) + r of column l % 16
      const int r0 = 4 * (tid >> 4), j = tid & 15;
      sm.u[r0][j] = L.u.x;
      sm.u[r0 + 1][j] = L.u.y;
      sm.u[r0 + 2][j] = L.u.z;
      sm.u[r0 + 3][j] = L.u.w;
    }
    if (tid < kSeg) sm.beta[tid] = L.beta;
  };
  // Add the finished segment's results to the outputs.
  auto flush = [&](int seg) {
    const int t0 = seg * kSeg, n = min(kSeg, T_ - t0);
    const long row0 = b * T_ + t0;
    float* dqb = p.dq + (row0 * H + h) * K;
    float* dkb = p.dk + (row0 * H + h) * K;
    float* dgb = p.dg + (row0 * HV + hv) * K;
    float vals[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = town + 4 * i;
      vals[i][0] = sm.dq[tt][cown];
      vals[i][1] = sm.dk[tt][cown];
      vals[i][2] = sm.dg[tt][cown];
    }
    float4 dv4 = *reinterpret_cast<const float4*>(&sm.dv[(tid >> 2) & 15][4 * (tid & 3)]);
    const float dbv = sm.db[tid & 15];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = town + 4 * i;
      if (tt < n) {
        atomicAdd(dqb + tt * H * K + cown, vals[i][0]);
        atomicAdd(dkb + tt * H * K + cown, vals[i][1]);
        atomicAdd(dgb + tt * HV * K + cown, vals[i][2]);
      }
    }
    if (tid < 64 && (tid >> 2) < n)
      *reinterpret_cast<float4*>(p.dv + (row0 * HV + hv) * V + v0 + (tid >> 2) * HV * V +
                                 4 * (tid & 3)) = dv4;
    if (tid < n) atomicAdd(p.dbeta + row0 * HV + hv + tid * HV, dbv);
  };

  // Sums over the keys of x[0..7] (columns c4 .. c4 + 3 of a, then of
  // Sd^T k).  A 16-lane row holds 4 keys x 4 column groups, so rotations by 4
  // and 8 keep the group, and the row swaps add the wavefront's four rows;
  // lanes 0..3 then hold the wavefront's partial sums of all 32 (quantity,
  // column) pairs, which go to LDS.  After the barrier lane l of every
  // wavefront reads wavefront l % 8's partials of pair group l / 8 (four
  // columns), three lane exchanges inside each group of 8 lanes add the
  // wavefronts, and the totals come back through a slot of the wavefront's
  // own (no further barrier).  The partials are double-buffered: one barrier
  // per call.
  static_assert(NW == 8 || NW == 4 || NW == 2, "wavefronts per workgroup");
  int rb = 0;
  auto key_sum8 = [&](float x[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = ror_add<4>(x[i]);
      x[i] = ror_add<8>(x[i]);
      x[i] = xor_sum<16>(x[i]);
      x[i] = xor_sum<32>(x[i]);
    }
    if (lane < 4) {
      *reinterpret_cast<float4*>(&sm.red[rb][w][0][c4]) = float4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<float4*>(&sm.red[rb][w][1][c4]) = float4{x[4], x[5], x[6], x[7]};
    }
    __syncthreads();
    const int grp = lane >> 3;  // pair group: quantity grp / 4, columns 4 (grp % 4) ..
    float4 t = *reinterpret_cast<const float4*>(
        &sm.red[rb][lane & (NW - 1)][grp >> 2][4 * (grp & 3)]);
    if (NW < 8 && (lane & 7) >= NW) t = float4{0.0f, 0.0f, 0.0f, 0.0f};
    t.x = oct_sum(t.x);
    t.y = oct_sum(t.y);
    t.z = oct_sum(t.z);
    t.w = oct_sum(t.w);
    if ((lane & 7) == 0) *reinterpret_cast<float4*>(&sm.fin[w][grp][0]) = t;
    // the slot is read back by the same wavefront: LDS accesses of one
    // wavefront complete in order
    const float4 a = *reinterpret_cast<const float4*>(&sm.fin[w][cg][0]);
    const float4 z = *reinterpret_cast<const float4*>(&sm.fin[w][4 + cg][0]);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = z.x; x[5] = z.y; x[6] = z.z; x[7] = z.w;
    rb ^= 1;
  };

  float dS[4];
  {
    const long o = ((long)hd * K + kap) * V + v0 + c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dS[i] = p.dST ? p.dST[o + i] : 0.0f;
  }
  SegLoads<T, NVD> L;
  if (NC > 0) issue(NC - 1, L);
  for (int seg = NC - 1; seg >= 0; --seg) {
    const int n = min(kSeg, T_ - seg * kSeg);
    stage(L);
    const float4 ck = L.ckpt;
    __syncthreads();
    // S_t = alpha_t S_{t-1} + k_t U_t^T, from the checkpoint
    auto advance = [&](int tt, float S[4]) {
      const float a = sm.al[tt][kap], kv = sm.k[tt][kap];
      const float4 u = *reinterpret_cast<const float4*>(&sm.u[tt][c4]);
      S[0] = a * S[0] + kv * u.x;
      S[1] = a * S[1] + kv * u.y;
      S[2] = a * S[2] + kv * u.z;
      S[3] = a * S[3] + kv * u.w;
    };
    // The reverse step of token tt, given S_{t-1} (no global memory access).
    auto reverse = [&](int tt, const float sp[4]) {
      const float a_ = sm.al[tt][kap], kv = sm.k[tt][kap], qv = sm.q[tt][kap];
      const float bt = sm.beta[tt];
      const float4 d4 = *reinterpret_cast<const float4*>(&sm.dout[tt][c4]);
      const float4 v4 = *reinterpret_cast<const float4*>(&sm.v[tt][c4]);
      const float d[4] = {d4.x, d4.y, d4.z, d4.w}, vv[4] = {v4.x, v4.y, v4.z, v4.w};
      float Sd[4], x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Sd[i] = a_ * sp[i];
        dS[i] += qv * d[i];  // the read o_t = s S_t^T q_t
        x[i] = kv * dS[i];
        x[4 + i] = kv * Sd[i];
      }
      key_sum8(x);  // a_t = dS^T k_t and the prediction Sd^T k_t, per column
      float dq = 0.0f, dk = 0.0f, dg = 0.0f, db = 0.0f;
      const float bk = bt * kv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = vv[i] - x[4 + i];
        dq += (Sd[i] + bk * r) * d[i];
        const float dr = bt * x[i];
        db += x[i] * r;
        dk += bt * dS[i] * r - Sd[i] * dr;
        const float dsd = dS[i] - kv * dr;
        dg += dsd * Sd[i];
        dS[i] = a_ * dsd;
        x[i] = dr;
      }
      dq = quad_sum(dq) * scale;
      dk = quad_sum(dk);
      dg = quad_sum(dg);
      if (cg == 0) {
        sm.dq[tt][kap] = dq;
        sm.dk[tt][kap] = dk;
        sm.dg[tt][kap] = dg;
      }
      if (kap == 0) {
        *reinterpret_cast<float4*>(&sm.dv[tt][c4]) = float4{x[0], x[1], x[2], x[3]};
        db = quad_sum(db);
        if (cg == 0) sm.db[tt] = db;
      }
    };
    // The two halves of the segment, the later first: each rebuilds its
    // eight states S_{t-1} from the checkpoint into registers, then runs
    // them in reverse.
#pragma unroll
    for (int half = 1; half >= 0; --half) {
      const int base = half * (kSeg / 2);
      float S[4] = {ck.x, ck.y, ck.z, ck.w};
      for (int tt = 0; tt < base && tt < n; ++tt) advance(tt, S);
      float st[kSeg / 2][4];
#pragma unroll
      for (int j = 0; j < kSeg / 2; ++j) {
        if (base + j < n) {
#pragma unroll
          for (int i = 0; i < 4; ++i) st[j][i] = S[i];
          advance(base + j, S);
        }
      }
#pragma unroll
      for (int j = kSeg / 2 - 1; j >= 0; --j)
        if (base + j < n) reverse(base + j, st[j]);
    }
    __syncthreads();  // the segment's results are in LDS; its inputs are no longer read
    // the next segment's loads go out before the atomics, so that waiting for
    // them does not wait for the atomics; unconditional (the last re-reads
    // segment 0) so that no earlier load stays live through the segment
    issue(max(seg - 1, 0), L);
    flush(seg);
  }
  if (p.dS0)
    *reinterpret_cast<float4*>(p.dS0 + ((long)hd * K + kap) * V + v0 + c4) =
        float4{dS[0], dS[1], dS[2], dS[3]};
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
const float* split_resolved_values(const void* workspace, long chunks, int K, int C);

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace: the segment checkpoints [B, HV, NC, K, V], then the split
// schedule's own workspace (which keeps U for the segment kernel).
size_t bwd_workspace_bytes(int B, int T, int HV, int K, int V) {
  const size_t nc = ((size_t)T + kSeg - 1) / kSeg;
  return align256((size_t)B * HV * nc * K * V * sizeof(float)) +
         (size_t)B * HV * nc * split_workspace_bytes_per_chunk(K, V, kSeg);
}

static hipError_t zero(float* p, long n, hipStream_t stream) {
  if (!p || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

template <int K, typename T, int GK>
static hipError_t launch_bwd_kt(BwdParams p, hipStream_t stream) {
  const long nblk = (long)p.B * p.HV * (K / kBV);
  if (nblk > 0) {
    hipLaunchKernelGGL((bwd_segment_kernel<K, T, GK>), dim3((unsigned)nblk), dim3(4 * K), 0, stream,
                       p);
    hipError_t e = hipGetLastError();
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
  void* split_ws = ws + align256((size_t)B * HV * NC * K * K * sizeof(float));
  hipError_t e;
  const long nq = (long)B * T * H * K, ng = (long)B * T * HV * K;
  if ((e = zero(dq, nq, stream)) != hipSuccess || (e = zero(dk, nq, stream)) != hipSuccess ||
      (e = zero(dbeta, (long)B * T * HV, stream)) != hipSuccess ||
      (e = zero(dg_raw, ng, stream)) != hipSuccess || (e = zero(dA_log, HV, stream)) != hipSuccess ||
      (e = zero(ddt_bias, (long)HV * K, stream)) != hipSuccess)
    return e;
  if (T > 0) {
    // the states and U only (no o): the split skips its output stage
    e = launch_split(q, k, v, bf16, g_raw, beta, A_log, dt_bias, kind, 0, lower_bound, S0,
                     nullptr, nullptr, ckpt, split_ws, B, T, H, HV, K, kSeg, stream);
    if (e != hipSuccess) return e;
  }
  const float* u = split_resolved_values(split_ws, (long)B * HV * NC, K, kSeg);
  BwdParams p{q, k, v, g_raw, beta, A_log, dt_bias, dout, dST, ckpt, u, dq, dk, dv, dbeta,
              dg_raw, dS0, dA_log, ddt_bias, B, T, H, HV, NC, lower_bound};
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
