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
// Schedule, three launches:
//  1. the fused chunk kernel in checkpoint mode (kda_chunk.hip) zeroes the
//     outputs the later kernels accumulate into, writes the state entering
//     every 16-token segment and U_t = beta_t r_t of every token, on its fp32
//     path whatever the input type, and once per
//     (sequence, value head, segment) E and the matrices below that do not
//     depend on the value tile;
//  2. bwd_segment_kernel: one workgroup per (sequence, value head, 16-wide
//     value tile) walks the segments from the last, carrying dL/dS of its
//     tile in LDS;
//  3. the gate kernel applies the gate's chain rule and sums dt_bias and
//     A_log over the sequences.
//
// Inside a segment the reverse recurrence of dL/dS is the adjoint of the
// forward's delta rule, dS_{t-1} = diag(alpha_t)(I - beta_t k_t k_t^T) G_t with
// G_t = dS_t + s q_t do_t^T, so everything that couples the tokens through a
// sum over the keys is a product over the segment.  With E_t the cumulative
// retain factor from the segment start (per channel), Suf_t = E_15 / E_t,
// L = strictly-lower[(k E)(k / E)^T] and M = upper[(k / E)(s q E)^T]:
//   predictions  p = (k E) S_0 + L U,             r = v - p
//   a_t = G_t^T k_t:  (I + L^T diag(beta)) A = M dL/do + (k Suf) dS_in
// (dS_in: dL/dS entering the segment's reverse pass), and dq, dk, dg and the
// dS_in of the earlier segment are products over the segment as well (see
// chunk_phase).  All of it runs on fp32 MFMA 16x16x4.  Segments whose E
// leaves [2^-100, 2^100] (where k / E would lose range) take a per-token pass
// instead: the states rebuilt from the checkpoint in registers, the sums over
// the keys by DPP and row swaps inside a wavefront and an LDS exchange across
// them.  The per-key results (dq, dk, dg) and dbeta, summed over the value
// tiles (and the value heads of a GVA group), are accumulated with fp32
// atomics into zeroed outputs, once per segment, so their last bits depend on
// the order the tiles finish in.  Arithmetic is fp32 throughout (bf16 inputs
// widened exactly).
#include <algorithm>
#include <cstdint>
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
  const float* ckpt;  // [B, HV, NC, K / 4, V, 4]: the state entering each 16-token segment, by key quads
  const float* u;     // [B, HV, NC, V / 16, 64, 4]: U = beta r of every token (MFMA accumulator order)
  float* ops;         // [B, HV, NC, 3, 64, 4]: per segment, the value-independent operands (the checkpoint forward)
  float* eseg;        // [B, HV, NC, 16, K]: per segment, the cumulative retain factors E
  int* segbad;        // [B, HV, NC]: nonzero where the forward ran the segment token by token
  float* dq;
  float* dk;
  float* dv;
  float* dbeta;
  float* dg;  // dL/dg, turned into dL/dg_raw by the gate kernel
  float* dS0;
  float* dA_log;
  float* ddt_bias;
  int B, T, H, HV, NC;
  int per_head;  // one gate value per (token, value head): g_raw, dL/dg [B, T, HV], dt_bias [HV]
  float lower_bound;
};

constexpr int kSeg = 16;  // tokens per segment (the checkpoint spacing)
constexpr int kBV = 16;   // value columns per workgroup

// The buffers the backward accumulates into, zeroed by one launch.
constexpr int kZeroBufs = 6;
struct ZeroList {
  float* p[kZeroBufs];  // NULL: skipped
  long n[kZeroBufs];
};
__global__ void bwd_zero_kernel(ZeroList z) {
  const long stride = (long)gridDim.x * blockDim.x, t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (int j = 0; j < kZeroBufs; ++j) {
    float* p = z.p[j];
    const long n = z.n[j];
    if (!p) continue;
    // 16-byte stores where the buffer is 16-byte aligned, its tail element by element
    const long n4 = (reinterpret_cast<uintptr_t>(p) & 15) == 0 ? n / 4 : 0;
    for (long i = t; i < n4; i += stride) reinterpret_cast<float4*>(p)[i] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    for (long i = 4 * n4 + t; i < n; i += stride) p[i] = 0.0f;
  }
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

// x, with the compiler unable to see its value: per-thread offsets derived
// from it inside a phase of the segment loop are formed there, rather than
// hoisted out of the loop (where they would hold registers through it)
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

constexpr int kTiles = 2;  // value tiles per workgroup

// Row stride of the tile's 16-wide arrays: 20 floats place the 16 rows of a
// column read, and the 16 columns of a row read by 16 lanes at stride one
// row, on distinct banks (a stride of 16 put every fourth row on the same
// ones), and keeps each row 16-byte aligned for the float4 accesses.
constexpr int kTS = kBV + 4;

// One value tile's arrays.  Each wavefront touches only its own tile's, from
// one base address: within the tile every offset fits a DS instruction's
// 64 KiB immediate range.
template <int K>
struct alignas(16) BwdTile {
  float u[kSeg][kTS];  // U = beta r from the forward (0 past the end)
  float v[kSeg][kTS];
  float dout[kSeg][kTS];
  float a[kSeg][kTS];    // a_t = G_t^T k_t
  float r[kSeg][kTS];    // r_t = v_t - Sd_t^T k_t
  float w1[kSeg][kTS];   // W1[t][m] = (dL/do U^T)[t][m] for m <= t, else 0
  float w2[kSeg][kTS];   // W2[t][m] = (dR U^T)[t][m] for m < t, else 0
  float s0[K][kTS];      // the tile of the checkpoint S_0
  float dsin[K][kTS];    // the tile of dL/dS entering the segment's reverse pass
  // chunked pass: partial products over the four quarters of the keys,
  // (k E) S_0 in 0..3 and (k Suf) dS_in in 4..7; written after the staging,
  // read before the next one
  float part[8][kSeg][kTS];
  // per-token pass: its key sums across the wavefronts
  float red[2][K / 16][2][kBV];
  float fin[K / 16][8][4];
};

template <int K>
struct alignas(16) BwdSmem {
  static constexpr int KP = K + 4;  // row stride: the 16 rows of an MFMA operand read spread over the banks
  float beta[kSeg];
  float4 ops[3][64];  // the segment's value-independent operands (the checkpoint forward)
  // the segment's inputs per (token, key channel).  A segment takes either the
  // chunked pass, which reads the per-key operands formed once at the staging,
  // or the per-token pass, which reads k, s q and the retain factors: each pair
  // shares its LDS, and the staging writes the one the segment's pass reads.
  float E[kSeg][KP];  // prod_{m <= t} alpha_m from the segment start
  union {
    float ke[kSeg][KP];  // chunked: k E (0 past the end)
    float k[kSeg][KP];   // per-token: k (0 past the end)
  };
  union {
    float qe[kSeg][KP];  // chunked: s q E (0 past the end)
    float q[kSeg][KP];   // per-token: s q (0 past the end)
  };
  union {
    float kh[kSeg][KP];  // chunked: k / E (0 past the end)
    float al[kSeg][KP];  // per-token: the retain factors (1 past the end)
  };
  BwdTile<K> tile[kTiles];
  union {
    // chunked pass: each wavefront of tile 1 hands its results (dq, dk, dg:
    // entry r of lane l) to the wavefront of tile 0 that owns the same keys
    float xch[K / 16][3][4][64];
    // per-token pass: its results, the tiles summed, written out together
    // once the segment is done
    struct {
      float dq[kSeg][K];
      float dk[kSeg][K];
      float dg[kSeg][K];
    } fb;
  };
};

// One segment's inputs in flight: this thread's share of E, k and q (token
// tid / (K / 4), four consecutive keys), of v, dL/do, U and beta, of the
// prep's operands, four keys of one column of the checkpoint, and the range flag.
template <typename T, int NVD, int NOPS>
struct SegLoads {
  float4 e;
  typename In<T>::Raw4 k, q;
  typename In<T>::Raw1 v[NVD];
  float dout[NVD], beta;
  float4 u, ckpt, ops[NOPS];
  int bad;
};

template <int K, typename T, int GK, bool PH>
__global__ __launch_bounds__(4 * K * kTiles) __attribute__((amdgpu_waves_per_eu(4))) void
bwd_segment_kernel(BwdParams p) {
  // NTH threads per value tile (4 per key row), NWH wavefronts; the
  // workgroup's kTiles tiles are adjacent 16-wide column blocks
  constexpr int V = K, NTH = 4 * K, NWH = NTH / 64, NT = NTH * kTiles, NVT = V / kBV;
  constexpr int NVD = (kSeg * kBV + NTH - 1) / NTH;  // v and dL/do elements each thread stages
  constexpr int NOPS = (3 * 64 + NT - 1) / NT;       // float4s of the prep's operands each thread stages
  static_assert(kSeg * K / NTH == 4 && NTH >= 64 && (NTH & (NTH - 1)) == 0, "thread layout");
  static_assert(NVT % kTiles == 0, "value tiles per workgroup");
  __shared__ BwdSmem<K> sm;
  const int gtid = threadIdx.x, tile = gtid / NTH;
  const int tid = gtid & (NTH - 1), lane = tid & 63, w = tid >> 6;  // within the tile
  const int kap = tid >> 2, cg = tid & 3, c4 = 4 * cg;
  BwdTile<K>& ts = sm.tile[tile];
  // (placing a head's value tiles on one XCD, so that their common reads
  // share its L2, measured 2% slower: their atomics then meet there)
  const int vt = blockIdx.x % (NVT / kTiles), hd = blockIdx.x / (NVT / kTiles);
  const int trow = tid / (K / 4), tcol = 4 * (tid % (K / 4));  // the staging layout of E, k, q, S_0
  const int HV = p.HV, H = p.H, T_ = p.T, NC = p.NC;
  const long b = hd / HV;
  const int hv = hd % HV, h = hv / (HV / H), v0 = (vt * kTiles + tile) * kBV;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const GateConsts gc = gate_consts(rate, p.lower_bound);
  // PH: one gate value per (token, value head) (p.per_head)
  constexpr int gK = PH ? 1 : K;  // gate stride
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);

  // Issue the loads of segment seg (rows past the end re-read the last
  // token, n >= 1).  Addresses are a base uniform over the workgroup plus a
  // 32-bit per-thread offset.
  auto issue = [&](int seg, SegLoads<T, NVD, NOPS>& L) {
    const int gtid = opaque(threadIdx.x), tid = gtid & (NTH - 1);
    const int trow = tid / (K / 4), tcol = 4 * (tid % (K / 4));
    const int v0 = (vt * kTiles + opaque(threadIdx.x) / NTH) * kBV;
    const int tile = opaque(threadIdx.x) / NTH;
    const int t0 = seg * kSeg, n = min(kSeg, T_ - t0);
    const long row0 = b * T_ + t0;
    const long sg = (long)hd * NC + seg;
    if (tile == 0) {  // E, k and q serve both tiles
      L.e = *reinterpret_cast<const float4*>(p.eseg + (sg * kSeg + trow) * K + tcol);
      const int tr = min(trow, n - 1);
      L.k = In<T>::raw4(kg, ((row0 + tr) * H + h) * K + tcol);
      L.q = In<T>::raw4(qg, ((row0 + tr) * H + h) * K + tcol);
    }
    L.bad = p.segbad[sg];
    const T* vb = vg + (row0 * HV + hv) * V + v0;
    const float* db = p.dout + (row0 * HV + hv) * V + v0;
#pragma unroll
    for (int i = 0; i < NVD; ++i) {  // elements past the tile re-read its first ones
      const int e = (tid + i * NTH) % (kSeg * kBV);
      const int o = min(e / kBV, n - 1) * HV * V + e % kBV;
      L.v[i] = vb[o];
      L.dout[i] = db[o];
    }
    L.u = *reinterpret_cast<const float4*>(p.u + (sg * NVT + v0 / kBV) * 256 + 4 * (tid & 63));
    L.beta = p.beta[row0 * HV + hv + min(tid & 15, n - 1) * HV];
    // keys 4 (tid / 16) .. + 3 of column v0 + tid % 16: 16 lanes read 256 contiguous bytes
    L.ckpt = *reinterpret_cast<const float4*>(p.ckpt + sg * K * V + ((tid >> 4) * V + v0 + (tid & 15)) * 4);
    const float4* ob = reinterpret_cast<const float4*>(p.ops + ((long)hd * NC + seg) * (3 * 64 * 4));
#pragma unroll
    for (int i = 0; i < NOPS; ++i) L.ops[i] = ob[min(gtid + i * NT, 3 * 64 - 1)];
  };
  // Place them in LDS, tokens past the end as an identity (alpha = 1, k, q,
  // v, dL/do, U and beta zero), with the cumulative retain factors E.
  // Returns whether an E of this thread leaves [2^-100, 2^100] (or is NaN).
  auto stage = [&](const SegLoads<T, NVD, NOPS>& L, int n) {
    const int gtid = opaque(threadIdx.x), tid = gtid & (NTH - 1);
    const int trow = tid / (K / 4), tcol = 4 * (tid % (K / 4));
    BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
    const int tile = opaque(threadIdx.x) / NTH;
    if (tile == 0) {
      const bool in = trow < n;
      float kv[4], qv[4];
      In<T>::unpack4(L.k, kv);
      In<T>::unpack4(L.q, qv);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kv[c] = in ? kv[c] : 0.0f;
        qv[c] = in ? scale * qv[c] : 0.0f;
      }
      *reinterpret_cast<float4*>(&sm.E[trow][tcol]) = L.e;
      if (L.bad == 0) {  // chunked pass: the per-key operands (uniform branch)
        const float e[4] = {L.e.x, L.e.y, L.e.z, L.e.w};
        float ke[4], qe[4], kh[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ke[c] = kv[c] * e[c];
          qe[c] = qv[c] * e[c];
          kh[c] = kv[c] * __builtin_amdgcn_rcpf(e[c]);
        }
        *reinterpret_cast<float4*>(&sm.ke[trow][tcol]) = float4{ke[0], ke[1], ke[2], ke[3]};
        *reinterpret_cast<float4*>(&sm.qe[trow][tcol]) = float4{qe[0], qe[1], qe[2], qe[3]};
        *reinterpret_cast<float4*>(&sm.kh[trow][tcol]) = float4{kh[0], kh[1], kh[2], kh[3]};
      } else {
        *reinterpret_cast<float4*>(&sm.k[trow][tcol]) = float4{kv[0], kv[1], kv[2], kv[3]};
        *reinterpret_cast<float4*>(&sm.q[trow][tcol]) = float4{qv[0], qv[1], qv[2], qv[3]};
      }
    }
#pragma unroll
    for (int i = 0; i < NVD; ++i) {
      const int e = tid + i * NTH;
      if (e < kSeg * kBV) {
        const bool in = e / kBV < n;
        ts.v[e / kBV][e % kBV] = in ? In<T>::widen(L.v[i]) : 0.0f;
        ts.dout[e / kBV][e % kBV] = in ? L.dout[i] : 0.0f;
      }
    }
    if (tid < 64) {  // U: one 16 x 16 fragment, lane l holding rows 4 (l / 16) + r of column l % 16
      const int r0 = 4 * (tid >> 4), j = tid & 15;
      ts.u[r0][j] = r0 < n ? L.u.x : 0.0f;
      ts.u[r0 + 1][j] = r0 + 1 < n ? L.u.y : 0.0f;
      ts.u[r0 + 2][j] = r0 + 2 < n ? L.u.z : 0.0f;
      ts.u[r0 + 3][j] = r0 + 3 < n ? L.u.w : 0.0f;
    }
    if (gtid < kSeg) sm.beta[gtid] = gtid < n ? L.beta : 0.0f;
    {  // column tid % 16 of the tile, keys 4 (tid / 16) .. + 3
      const int kr = 4 * (tid >> 4), cc = tid & 15;
      ts.s0[kr][cc] = L.ckpt.x;
      ts.s0[kr + 1][cc] = L.ckpt.y;
      ts.s0[kr + 2][cc] = L.ckpt.z;
      ts.s0[kr + 3][cc] = L.ckpt.w;
    }
#pragma unroll
    for (int i = 0; i < NOPS; ++i)
      if (gtid + i * NT < 3 * 64) (&sm.ops[0][0])[gtid + i * NT] = L.ops[i];
    return L.bad != 0;
  };
  // Add the finished segment's results to the outputs.  After the chunked
  // pass they are in the registers cq, ck, cg (lane l: tokens 4 (l / 16) + r,
  // key 16 w + l % 16) of both tiles: tile 0 adds tile 1's, handed over in
  // LDS, and issues one atomic per element.  After the per-token pass they are
  // in LDS, the tiles already summed.
  float cq[4], ckk[4], cgg[4];
  auto flush = [&](int seg, bool chunked) {
    const int gtid = opaque(threadIdx.x), tid = gtid & (NTH - 1), lane = tid & 63;
    const int t0 = seg * kSeg, n = min(kSeg, T_ - t0);
    const long row0 = b * T_ + t0;
    float* dqb = p.dq + (row0 * H + h) * K;
    float* dkb = p.dk + (row0 * H + h) * K;
    float* dgb = p.dg + (row0 * HV + hv) * K;  // per-channel gate
    if (chunked) {
      if (gtid >= NTH) return;  // tile 1 handed its results over
      const int w = tid >> 6, g4 = lane >> 4, c16 = lane & 15, key = 16 * w + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cq[r] += sm.xch[w][0][r][lane];
        ckk[r] += sm.xch[w][1][r][lane];
        cgg[r] += sm.xch[w][2][r][lane];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = 4 * g4 + r;
        if (tt < n) {
          atomicAdd(dqb + tt * H * K + key, cq[r]);
          atomicAdd(dkb + tt * H * K + key, ckk[r]);
          if (!PH) atomicAdd(dgb + tt * HV * K + key, cgg[r]);
        }
      }
      if (PH) {  // per-head gate: dg summed over this wavefront's 16 keys, one atomic per token
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = cgg[r];
          x = ror_add<8>(x);
          x = ror_add<4>(x);
          x = ror_add<2>(x);
          x = ror_add<1>(x);
          if (c16 == 0 && 4 * g4 + r < n) atomicAdd(p.dg + (row0 + 4 * g4 + r) * HV + hv, x);
        }
      }
    } else {
      for (int e = gtid; e < kSeg * K; e += NT) {
        const int tt = e / K, c = e % K;
        if (tt < n) {
          atomicAdd(dqb + tt * H * K + c, sm.fb.dq[tt][c]);
          atomicAdd(dkb + tt * H * K + c, sm.fb.dk[tt][c]);
          if (!PH) atomicAdd(dgb + tt * HV * K + c, sm.fb.dg[tt][c]);
        }
      }
      if (PH && gtid < 64) {  // per-head gate: token gtid / 4's dg summed over the key channels
        const int tt = gtid >> 2;
        float x = 0.0f;
        for (int c = gtid & 3; c < K; c += 4) x += sm.fb.dg[tt][c];
        x = quad_sum(x);
        if ((gtid & 3) == 0 && tt < n) atomicAdd(p.dg + (row0 + tt) * HV + hv, x);
      }
    }
  };

  // The segment's per-token key sums that involve the value tile, as matrix
  // products (16 x 16 outputs, fp32 MFMA 16x16x4, the key axis in steps of
  // 4): lane l supplies the operands of row l % 16 (a token, or a value
  // column of B) and key step position l / 16, and holds output rows
  // 4 (l / 16) .. + 3 of column l % 16.  Eight tasks, product task / 4 over
  // key quarter task % 4, spread over the wavefronts: (k E) S_0, then
  // (k Suf) dS_in with Suf = gamma / E.
  auto product = [&](auto PP, int task) {
    constexpr int P = decltype(PP)::value;
    BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
    const int lane = opaque(threadIdx.x) & 63, row = lane & 15, kq = lane >> 4;
    const int k0 = (task & 3) * (K / 4);
    // up to four accumulators, so that the dependent MFMA chains are short
    f32x4 acc[4] = {};
#pragma unroll
    for (int st = 0; st < K / 16; ++st) {
      const int key = k0 + 4 * st + kq;
      float x, y;
      if constexpr (P == 0) {
        x = sm.ke[row][key];
        y = ts.s0[key][row];
      } else {
        x = sm.kh[row][key] * sm.E[kSeg - 1][key];
        y = ts.dsin[key][row];
      }
      acc[st & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc[st & 3], 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      ts.part[task][4 * kq + r][row] = (acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]);
  };
  auto products = [&]() {
    const int w = (opaque(threadIdx.x) & (NTH - 1)) >> 6;
#pragma unroll 1
    for (int task = w; task < 8; task += NWH) {
      if (task < 4)
        product(std::integral_constant<int, 0>{}, task);
      else
        product(std::integral_constant<int, 1>{}, task);
    }
  };
  // From the products and the prep's operands (L_tm = g1[m][t] for m < t,
  // M_tm = g2[t][m] for m >= t, R = (I + L^T diag(beta))^{-1}):
  //   wavefront 0:        P = (k E) S_0 + L U,  r = v - P
  //   wavefront 1 % NWH:   Y = (k Suf) dS_in + M dL/do,  a = R Y (formed as
  //                       a^T = Y^T R^T), then W2 = strictly-lower[diag(beta) a U^T]
  //   wavefront 2 % NWH:   W1 = lower[dL/do U^T]
  // The products over the tokens (or the tile's columns) are 16 x 16 x 16 on
  // fp32 MFMA as above, the inner index in step r being 4 (l / 16) + r, so
  // that an accumulator serves as the next product's operand in place.
  auto solve = [&]() {
    BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
    const int tid = opaque(threadIdx.x) & (NTH - 1), lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;
    auto mfma = [](float a, float b, f32x4 c) {
      return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    };
    auto part_sum = [&](int p0, int r) {
      const int t = 4 * g4 + r;
      return (ts.part[p0][t][c16] + ts.part[p0 + 1][t][c16]) +
             (ts.part[p0 + 2][t][c16] + ts.part[p0 + 3][t][c16]);
    };
    if (w == 0) {
      const float4 l4 = sm.ops[0][lane];
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = part_sum(0, r);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = mfma(lv[r], ts.u[4 * g4 + r][c16], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) ts.r[4 * g4 + r][c16] = ts.v[4 * g4 + r][c16] - acc[r];
    }
    if (w == 1 % NWH) {
      const float4 m4 = sm.ops[1][lane], r4 = sm.ops[2][lane];
      const float mv[4] = {m4.x, m4.y, m4.z, m4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
      f32x4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = part_sum(4, r);
#pragma unroll
      for (int r = 0; r < 4; ++r) y = mfma(mv[r], ts.dout[4 * g4 + r][c16], y);
      // a^T[j][t] = sum_m Y[m][j] R[t][m]: Y's accumulator is Y^T's A operand
      f32x4 at = {};
#pragma unroll
      for (int r = 0; r < 4; ++r) at = mfma(y[r], rv[r], at);
      // lane (c16, g4) holds a[c16][4 g4 + r]
      *reinterpret_cast<float4*>(&ts.a[c16][4 * g4]) = float4{at[0], at[1], at[2], at[3]};
      // W2[t][m] = sum_j beta_t a[t][j] U[m][j]
      const float bc = sm.beta[c16];
      const float4 u4 = *reinterpret_cast<const float4*>(&ts.u[c16][4 * g4]);
      const float uv[4] = {u4.x, u4.y, u4.z, u4.w};
      f32x4 acc2 = {};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc2 = mfma(bc * at[r], uv[r], acc2);
#pragma unroll
      for (int r = 0; r < 4; ++r) ts.w2[4 * g4 + r][c16] = c16 < 4 * g4 + r ? acc2[r] : 0.0f;
    }
    if (w == 2 % NWH) {  // W1 = lower[dL/do U^T]
      f32x4 acc = {};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int j = 4 * s4 + g4;
        acc = mfma(ts.dout[c16][j], ts.u[c16][j], acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ts.w1[4 * g4 + r][c16] = c16 <= 4 * g4 + r ? acc[r] : 0.0f;
    }
  };

  // Fallback for segments whose cumulative decay leaves [2^-100, 2^100]: the
  // per-token sums over the keys of x[0..7] (columns c4 .. c4 + 3 of a, then
  // of Sd^T k).  A 16-lane row holds 4 keys x 4 column groups, so rotations
  // by 4 and 8 keep the group, and the row swaps add the wavefront's four
  // rows; lanes 0..3 then hold the wavefront's partial sums of all 32
  // (quantity, column) pairs, which go to LDS.  After the barrier lane l of
  // every wavefront reads wavefront l % 8's partials of pair group l / 8 (four
  // columns), three lane exchanges inside each group of 8 lanes add the
  // wavefronts, and the totals come back through a slot of the wavefront's
  // own (no further barrier).  The partials are double-buffered: one barrier
  // per call.
  static_assert(NWH == 8 || NWH == 4 || NWH == 2, "wavefronts per tile");
  int rb = 0;
  auto key_sum8 = [&](float x[8]) {
    const int tid = opaque(threadIdx.x) & (NTH - 1), lane = tid & 63, w = tid >> 6, cg = tid & 3,
              c4 = 4 * cg;
    BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = ror_add<4>(x[i]);
      x[i] = ror_add<8>(x[i]);
      x[i] = xor_sum<16>(x[i]);
      x[i] = xor_sum<32>(x[i]);
    }
    if (lane < 4) {
      *reinterpret_cast<float4*>(&ts.red[rb][w][0][c4]) = float4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<float4*>(&ts.red[rb][w][1][c4]) = float4{x[4], x[5], x[6], x[7]};
    }
    __syncthreads();
    const int grp = lane >> 3;  // pair group: quantity grp / 4, columns 4 (grp % 4) ..
    float4 t = *reinterpret_cast<const float4*>(
        &ts.red[rb][lane & (NWH - 1)][grp >> 2][4 * (grp & 3)]);
    if (NWH < 8 && (lane & 7) >= NWH) t = float4{0.0f, 0.0f, 0.0f, 0.0f};
    t.x = oct_sum(t.x);
    t.y = oct_sum(t.y);
    t.z = oct_sum(t.z);
    t.w = oct_sum(t.w);
    if ((lane & 7) == 0) *reinterpret_cast<float4*>(&ts.fin[w][grp][0]) = t;
    // the slot is read back by the same wavefront: LDS accesses of one
    // wavefront complete in order
    const float4 a = *reinterpret_cast<const float4*>(&ts.fin[w][cg][0]);
    const float4 z = *reinterpret_cast<const float4*>(&ts.fin[w][4 + cg][0]);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = z.x; x[5] = z.y; x[6] = z.z; x[7] = z.w;
    rb ^= 1;
  };

  // The segment's gradients as products over the segment, with no per-token
  // loop.  With W1 = lower[dL/do U^T] (m <= t), W2 = strictly-lower[dR U^T]
  // (m < t), dR = diag(beta) A, Qt = s q E, Kt = k E, Kh = k / E, Ks = k Suf
  // (the gradients with respect to each are marked d):
  //   dQt = dL/do S_0^T + W1 Kh          dKt = -dR S_0^T - W2 Kh
  //   dKh = W1^T Qt - W2^T Kt            dKs = U dS_in^T
  //   dS_0 = diag(gamma) dS_in + Qt^T dL/do - Kt^T dR   (entering the earlier segment)
  //   dq = s E dQt,  dk = E dKt + dKh / E + Suf dKs
  //   dg_t = sum_{t' >= t} (dQt Qt + dKt Kt - dKh Kh - dKs Ks)_{t'}, plus, from
  //          gamma = E_15, gamma sum_j dS_in S_0 + sum_t dKs Ks for every t.
  // Wavefront w owns keys 16 w .. 16 w + 15.  Lane l: c16 = l % 16, g4 = l / 16;
  // the MFMA accumulators hold rows 4 g4 + r of column c16.  W1 and W2 are formed
  // in both orientations so that either serves as an A operand whose inner
  // index in step r is 4 g4 + r (the lane's own accumulator entry r).
  auto chunk_phase = [&](int seg, auto FIRST) {
    constexpr bool kFirst = decltype(FIRST)::value;  // the workgroup's first value tile
    static_assert(kTiles == 2, "the products with W1 and W2 are split between two tiles");
    BwdTile<K>& ts = sm.tile[kFirst ? 0 : 1];
    const int v0 = (vt * kTiles + (kFirst ? 0 : 1)) * kBV;
    const int tid = opaque(threadIdx.x) & (NTH - 1), lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, g4 = lane >> 4, kb = 16 * w, key = kb + c16;
    auto mfma = [](float a, float b, f32x4 c) {
      return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    };
    // W1 and W2 enter the gradients linearly, so their products need them
    // only summed over the two tiles, and each runs in one tile: the first
    // takes W1's (into dQt and dKh), the second -W2's (into dKt and dKh).
    // W (masked) in both orientations: wt[r] = W[c16][4 g4 + r],
    // wd[r] = W[4 g4 + r][c16].
    const float(*wa)[kTS] = kFirst ? sm.tile[0].w1 : sm.tile[0].w2;
    const float(*wb)[kTS] = kFirst ? sm.tile[1].w1 : sm.tile[1].w2;
    const float4 wta = *reinterpret_cast<const float4*>(&wa[c16][4 * g4]);
    const float4 wtb = *reinterpret_cast<const float4*>(&wb[c16][4 * g4]);
    const float sg = kFirst ? 1.0f : -1.0f;
    const float wt[4] = {sg * (wta.x + wtb.x), sg * (wta.y + wtb.y), sg * (wta.z + wtb.z),
                         sg * (wta.w + wtb.w)};
    float wd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wd[r] = sg * (wa[4 * g4 + r][c16] + wb[4 * g4 + r][c16]);
    f32x4 dQ = {}, dKt = {}, dKs = {}, dKh = {}, dSn = {};
    const float bc = sm.beta[c16];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int c = 4 * s4 + g4;
      const float u_ = ts.u[c16][c], d_ = ts.dout[c16][c], r_ = bc * ts.a[c16][c];
      const float s0v = ts.s0[key][c], dsv = ts.dsin[key][c];
      dQ = mfma(d_, s0v, dQ);
      dKt = mfma(-r_, s0v, dKt);
      dKs = mfma(u_, dsv, dKs);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g4 + r;  // this step's inner index (a token)
      const float kh = sm.kh[m][key];
      if constexpr (kFirst) {
        dQ = mfma(wt[r], kh, dQ);
        dKh = mfma(wd[r], sm.qe[m][key], dKh);
      } else {
        dKt = mfma(wt[r], kh, dKt);
        dKh = mfma(wd[r], sm.ke[m][key], dKh);
      }
    }
    // dS_0 for this wavefront's keys: rows key 16 w + 4 g4 + r, column c16
    // (the inner index of step s4 is token 4 g4 + s4: the 16 lanes of a
    // row group read one row of dL/do and a)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int t = 4 * g4 + s4;
      dSn = mfma(sm.qe[t][key], ts.dout[t][c16], dSn);
      dSn = mfma(-sm.ke[t][key], sm.beta[t] * ts.a[t][c16], dSn);
    }
    // gamma's direct term for this lane's key: sum over the columns of
    // dS_in S_0 (columns g4 + 4 i per lane, then the four row groups)
    const float gam = sm.E[kSeg - 1][key];
    float gd = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) gd += ts.dsin[key][g4 + 4 * i] * ts.s0[key][g4 + 4 * i];
    float dGl[4], dql[4], dkl[4], ksks = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * g4 + r;
      const float e = sm.E[t][key], ie = __builtin_amdgcn_rcpf(e);
      const float qt = sm.qe[t][key], kt = sm.ke[t][key], kh = sm.kh[t][key], ks = kh * gam;
      dql[r] = scale * e * dQ[r];
      dkl[r] = e * dKt[r] + ie * dKh[r] + gam * ie * dKs[r];
      dGl[r] = dQ[r] * qt + dKt[r] * kt - dKh[r] * kh - dKs[r] * ks;
      ksks += dKs[r] * ks;
    }
    gd = xor_sum<32>(xor_sum<16>(gd));
    ksks = xor_sum<32>(xor_sum<16>(ksks));
    // the new dS entering the earlier segment (after every read of dS_in above)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kr = kb + 4 * g4 + r;
      ts.dsin[kr][c16] = dSn[r] + sm.E[kSeg - 1][kr] * ts.dsin[kr][c16];
    }
    // dg: the reverse cumulative sum over the tokens; gamma's terms belong to
    // the last token (t = 15: row group 3, entry 3)
    if (g4 == 3) dGl[3] += gam * gd + ksks;
    float suf = dGl[3];
    dGl[2] += suf;
    suf = dGl[2];
    dGl[1] += suf;
    suf = dGl[1];
    dGl[0] += suf;
    const float tot = dGl[0];  // this row group's sum
    // the sums of the later row groups (lanes 16, 32, 48 further)
    const float n1 = __shfl_down(tot, 16), n2 = __shfl_down(tot, 32), n3 = __shfl_down(tot, 48);
    const float later = (g4 < 1 ? n3 : 0.0f) + (g4 < 2 ? n2 : 0.0f) + (g4 < 3 ? n1 : 0.0f);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cq[r] = dql[r];
      ckk[r] = dkl[r];
      cgg[r] = dGl[r] + later;
    }
    if constexpr (!kFirst) {  // to the wavefront of the first tile with the same keys
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sm.xch[w][0][r][lane] = cq[r];
        sm.xch[w][1][r][lane] = ckk[r];
        sm.xch[w][2][r][lane] = cgg[r];
      }
    }
    if (w == 0) {  // dv = beta a, and the tile's part of dbeta_t = a_t . r_t
      const int t = lane >> 2, c = 4 * (lane & 3);
      const int t0 = seg * kSeg, n = min(kSeg, T_ - t0);
      const long rw = (b * T_ + t0 + t) * HV + hv;
      const float4 a4 = *reinterpret_cast<const float4*>(&ts.a[t][c]);
      const float4 r4 = *reinterpret_cast<const float4*>(&ts.r[t][c]);
      const float bt = sm.beta[t];
      const float arv = quad_sum(a4.x * r4.x + a4.y * r4.y + a4.z * r4.z + a4.w * r4.w);
      if (t < n) {
        *reinterpret_cast<float4*>(p.dv + rw * V + v0 + c) =
            float4{bt * a4.x, bt * a4.y, bt * a4.z, bt * a4.w};
        if ((lane & 3) == 0) atomicAdd(p.dbeta + rw, arv);
      }
    }
  };

  float dS[4];
  {
    const long o = ((long)hd * K + kap) * V + v0 + c4;
#pragma unroll
    for (int i = 0; i < 4; ++i) dS[i] = p.dST ? p.dST[o + i] : 0.0f;
  }
  *reinterpret_cast<float4*>(&ts.dsin[kap][c4]) = float4{dS[0], dS[1], dS[2], dS[3]};
  SegLoads<T, NVD, NOPS> L;
  if (NC > 0) issue(NC - 1, L);
  for (int seg = NC - 1; seg >= 0; --seg) {
    const int n = min(kSeg, T_ - seg * kSeg);
    const bool bad = stage(L, n);
    const bool fallback = bad;  // uniform: one flag per segment
    // the next segment's loads go out at once, so that the whole segment
    // hides their latency; unconditional (the last re-reads segment 0)
    issue(max(seg - 1, 0), L);
    __syncthreads();
    if (!fallback) {
      products();
      __syncthreads();
      solve();
      __syncthreads();
    }
    // S_t = Sd_t + k_t U_t^T with Sd_t = alpha_t S_{t-1}, from the
    // checkpoint; Sd_t is also handed back
    auto advance = [&](int tt, float S[4], float sd[4]) {
      const int tid = opaque(threadIdx.x) & (NTH - 1), kap = tid >> 2, c4 = 4 * (tid & 3);
      BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
      const float a = sm.al[tt][kap], kv = sm.k[tt][kap];
      const float4 u = *reinterpret_cast<const float4*>(&ts.u[tt][c4]);
      const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sd[i] = a * S[i];
        S[i] = sd[i] + kv * uu[i];
      }
    };
    // The reverse step of token tt, given Sd_t (no global memory access):
    // a_t and the prediction Sd_t^T k_t from one sum over the keys.  With dS
    // the gradient after the read, and beta factored out of the sums over the
    // columns j:
    //   dq = s (sum_j Sd d_j + beta k sum_j r_j d_j)
    //   dk = beta (sum_j dS r_j - sum_j Sd a_j)
    //   dg = sum_j (dS - k beta a_j) Sd,   dS <- alpha (dS - k beta a)
    auto reverse = [&](int tt, const float sd[4]) {
      const int tid = opaque(threadIdx.x) & (NTH - 1), kap = tid >> 2, cg = tid & 3, c4 = 4 * cg;
      BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
      const int v0 = (vt * kTiles + opaque(threadIdx.x) / NTH) * kBV;
      const float a_ = sm.al[tt][kap], kv = sm.k[tt][kap], qv = sm.q[tt][kap];
      const float bt = sm.beta[tt];
      const float4 d4 = *reinterpret_cast<const float4*>(&ts.dout[tt][c4]);
      const float d[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[i] += qv * d[i];  // the read o_t = s S_t^T q_t
      float a[4], r[4], x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = kv * dS[i];
        x[4 + i] = kv * sd[i];
      }
      key_sum8(x);  // a_t = dS^T k_t and the prediction Sd^T k_t, per column
      const float4 v4 = *reinterpret_cast<const float4*>(&ts.v[tt][c4]);
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
      float rd = 0.0f, ar = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = x[i];
        r[i] = vv[i] - x[4 + i];
        rd += r[i] * d[i];
        ar += a[i] * r[i];
      }
      rd = quad_sum(rd);
      ar = quad_sum(ar);
      const float kb = kv * bt;
      float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s1 += sd[i] * d[i];
        s2 += dS[i] * r[i];
        s2 -= sd[i] * a[i];
        const float dsd = dS[i] - kb * a[i];
        s3 += dsd * sd[i];
        dS[i] = a_ * dsd;
      }
      s1 = quad_sum(s1);
      s2 = quad_sum(s2);
      s3 = quad_sum(s3);
      if (cg == 0) {  // both tiles add into the zeroed results: 0 + x + y, exact in either order
        atomicAdd(&sm.fb.dq[tt][kap], scale * (s1 + kb * rd));
        atomicAdd(&sm.fb.dk[tt][kap], bt * s2);
        atomicAdd(&sm.fb.dg[tt][kap], s3);
      }
      if (kap == 0) {  // dv and the tile's part of dbeta, straight to the outputs
        const long rw = (b * T_ + seg * kSeg + tt) * HV + hv;
        *reinterpret_cast<float4*>(p.dv + rw * V + v0 + c4) =
            float4{bt * a[0], bt * a[1], bt * a[2], bt * a[3]};
        if (cg == 0) atomicAdd(p.dbeta + rw, ar);
      }
    };
    // The parts of the segment, the latest first: each rebuilds its kPart
    // states Sd_t from the checkpoint into registers, then runs them in
    // reverse.
    constexpr int kPart = 4;
    auto halves = [&]() {
      const int tid = opaque(threadIdx.x) & (NTH - 1), kap = tid >> 2, c4 = 4 * (tid & 3);
      BwdTile<K>& ts = sm.tile[opaque(threadIdx.x) / NTH];
#pragma unroll
      for (int part = kSeg / kPart - 1; part >= 0; --part) {
        const int base = part * kPart;
        const float4 ck = *reinterpret_cast<const float4*>(&ts.s0[kap][c4]);
        float S[4] = {ck.x, ck.y, ck.z, ck.w};
        float sd[kPart][4];
        for (int tt = 0; tt < base && tt < n; ++tt) advance(tt, S, sd[0]);
#pragma unroll
        for (int j = 0; j < kPart; ++j)
          if (base + j < n) advance(base + j, S, sd[j]);
#pragma unroll
        for (int j = kPart - 1; j >= 0; --j)
          if (base + j < n) reverse(base + j, sd[j]);
      }
    };
    if (fallback) {  // dL/dS in registers for the per-token pass, in the LDS tile between segments
      const int gtid = opaque(threadIdx.x), tid = gtid & (NTH - 1), kap = tid >> 2, c4 = 4 * (tid & 3);
      BwdTile<K>& ts = sm.tile[gtid / NTH];
      {  // the per-token pass takes the retain factors themselves (1 past the end)
        const int gc0 = PH ? 0 : kap;  // this thread's gate element
        const float bias = gate_bias_pre<GK>(
            (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[hv * gK + gc0] : 0.0f, gc);
        const float* gb = p.g_raw + ((b * T_ + seg * kSeg) * HV + hv) * gK;
        if (gtid < NTH) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tt = c4 + i;
            const float g = gb[min(tt, n - 1) * HV * gK + gc0];
            sm.al[tt][kap] = tt < n ? gate_alpha_pre<GK>(g, bias, gc) : 1.0f;
          }
        }
        for (int e = gtid; e < kSeg * K; e += NT) {
          (&sm.fb.dq[0][0])[e] = 0.0f;
          (&sm.fb.dk[0][0])[e] = 0.0f;
          (&sm.fb.dg[0][0])[e] = 0.0f;
        }
        __syncthreads();
      }
      const float4 d0 = *reinterpret_cast<const float4*>(&ts.dsin[kap][c4]);
      dS[0] = d0.x; dS[1] = d0.y; dS[2] = d0.z; dS[3] = d0.w;
      halves();
      *reinterpret_cast<float4*>(&ts.dsin[kap][c4]) = float4{dS[0], dS[1], dS[2], dS[3]};
    } else if (__builtin_amdgcn_readfirstlane(threadIdx.x) < NTH) {  // (uniform per wavefront)
      chunk_phase(seg, std::true_type{});
    } else {
      chunk_phase(seg, std::false_type{});
    }
    __syncthreads();  // the segment's results are in LDS; its inputs are no longer read
    flush(seg, !fallback);
  }
  __syncthreads();
  if (p.dS0) {  // (the thread's layout formed anew: nothing of it stays live through the loop)
    const int g = opaque(threadIdx.x), t = g & (NTH - 1), kr = t >> 2, cc = 4 * (t & 3);
    const int vc = (vt * kTiles + g / NTH) * kBV + cc;
    *reinterpret_cast<float4*>(p.dS0 + ((long)hd * K + kr) * V + vc) =
        *reinterpret_cast<const float4*>(&sm.tile[g / NTH].dsin[kr][cc]);
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
  constexpr int kRB = 8;  // rows whose loads are in flight together
  for (long rb = r0; rb < r1; rb += kRB) {
    float dgv[kRB], xv[kRB];
#pragma unroll
    for (int j = 0; j < kRB; ++j) {  // (rows past the block re-read its last one)
      const long i = ((rb + j < r1 ? rb + j : r1 - 1) * p.HV + hv) * K + c;
      dgv[j] = p.dg[i];
      xv[j] = p.g_raw[i];
    }
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      if (rb + j >= r1) break;
      const long i = ((rb + j) * p.HV + hv) * K + c;
      const float dg = dgv[j], x = xv[j] + bias;
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

// The per-head gate's chain rule: one thread per row (sequence, token) of
// one value head, dL/dg -> dL/dg_raw in place, the dt_bias and A_log sums
// reduced over the workgroup's rows before one atomic each.
template <int GK>
__global__ __launch_bounds__(256) void bwd_gate_head_kernel(BwdParams p, long rows) {
  const int hv = blockIdx.y, tid = threadIdx.x;
  const long r = (long)blockIdx.x * 256 + tid;
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const float bias = (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias[hv] : 0.0f;
  float dx = 0.0f, da = 0.0f;
  if (r < rows) {
    const long i = r * p.HV + hv;
    const float dg = p.dg[i], x = p.g_raw[i] + bias;
    dx = dg;
    if constexpr (GK == KDA_GATE_SAFE) {
      const float z = rate * x;
      const float sg = __builtin_amdgcn_rcpf(1.0f + exp_f(-z));
      const float d = p.lower_bound * sg * (1.0f - sg);
      dx = dg * d * rate;
      da = dg * d * z;
    } else if constexpr (GK == KDA_GATE_STANDARD) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + exp_f(-x));
      dx = -dg * rate * sg;
      da = -dg * rate * softplus_f(x);
    }
    p.dg[i] = dx;
  }
  if (GK == KDA_GATE_NONE) return;  // neither dt_bias nor A_log enters this gate
  __shared__ float red[2][256];
  red[0][tid] = dx;
  red[1][tid] = da;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) {
      red[0][tid] += red[0][tid + st];
      red[1][tid] += red[1][tid + st];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (p.ddt_bias) atomicAdd(p.ddt_bias + hv, red[0][0]);
    if (p.dA_log) atomicAdd(p.dA_log + hv, red[1][0]);
  }
}

hipError_t launch_chunk_ckpt(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                             const float* beta, const float* A_log, const float* dt_bias, int kind,
                             int per_head, float lower_bound, const float* S0, float* ckpt,
                             float* u_out, float* eseg, float* ops, int* segbad, int B, int T, int H,
                             int HV, int K, float* const zero[6], hipStream_t stream);

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace, all written by the forward in checkpoint mode: the segment
// checkpoints [B, HV, NC, K / 4, V, 4] and U [B, HV, NC, V / 16, 64, 4], then
// the per-segment operands [B, HV, NC, 3, 64, 4], E [B, HV, NC, 16, K] and
// range flags [B, HV, NC].
static size_t prep_bytes(size_t segs, int K) {
  return align256(segs * 3 * 64 * 4 * sizeof(float)) + align256(segs * kSeg * K * sizeof(float)) +
         align256(segs * sizeof(int));
}
size_t bwd_workspace_bytes(int B, int T, int HV, int K, int V) {
  const size_t segs = (size_t)B * HV * (((size_t)T + kSeg - 1) / kSeg);
  return align256(segs * K * V * sizeof(float)) + align256(segs * kSeg * V * sizeof(float)) +
         prep_bytes(segs, K);
}

static hipError_t zero(const ZeroList& z, hipStream_t stream) {
  long total = 0;
  for (int j = 0; j < kZeroBufs; ++j) total += z.p[j] ? z.n[j] : 0;
  if (total == 0) return hipSuccess;
  // enough 256-thread workgroups for a few 16-byte stores each, at most 8 per CU
  const long blocks = std::min<long>(2048, (total / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, z);
  return hipGetLastError();
}

template <int K, typename T, int GK>
static hipError_t launch_bwd_kt(BwdParams p, hipStream_t stream) {
  const long nblk = (long)p.B * p.HV * (K / kBV / kTiles);
  if (nblk > 0) {
    if (p.per_head)
      hipLaunchKernelGGL((bwd_segment_kernel<K, T, GK, true>), dim3((unsigned)nblk),
                         dim3(4 * K * kTiles), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_segment_kernel<K, T, GK, false>), dim3((unsigned)nblk),
                         dim3(4 * K * kTiles), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long rows = (long)p.B * p.T;
  if (rows == 0) return hipSuccess;
  if (p.per_head)
    hipLaunchKernelGGL((bwd_gate_head_kernel<GK>),
                       dim3((unsigned)((rows + 255) / 256), (unsigned)p.HV), dim3(256), 0, stream,
                       p, rows);
  else
    hipLaunchKernelGGL((bwd_gate_kernel<GK>), dim3((unsigned)((rows + 63) / 64), (unsigned)p.HV),
                       dim3(K), 0, stream, p, K, rows);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                      const float* beta, const float* A_log, const float* dt_bias, int kind,
                      int per_head, float lower_bound, const float* S0, const float* dout, const float* dST,
                      float* dq, float* dk, float* dv, float* dbeta, float* dg_raw, float* dA_log,
                      float* ddt_bias, float* dS0, void* workspace, int B, int T, int H, int HV,
                      int K, hipStream_t stream) {
  const int NC = (T + kSeg - 1) / kSeg;
  char* ws = static_cast<char*>(workspace);
  const size_t segs = (size_t)B * HV * NC;
  float* ckpt = reinterpret_cast<float*>(ws);
  float* u = reinterpret_cast<float*>(ws + align256(segs * K * K * sizeof(float)));
  float* ops = reinterpret_cast<float*>(reinterpret_cast<char*>(u) + align256(segs * kSeg * K * sizeof(float)));
  float* eseg = reinterpret_cast<float*>(reinterpret_cast<char*>(ops) + align256(segs * 3 * 64 * 4 * sizeof(float)));
  int* segbad = reinterpret_cast<int*>(reinterpret_cast<char*>(eseg) + align256(segs * kSeg * K * sizeof(float)));
  hipError_t e;
  const int gK = per_head ? 1 : K;  // gate values per (token, value head)
  const long nq = (long)B * T * H * K, ng = (long)B * T * HV * gK;
  if (T > 0) {
    // the forward in checkpoint mode: every segment's entry state and U, no
    // o; it also zeroes the outputs the later kernels accumulate into
    float* const zero[6] = {dq, dk, dbeta, dg_raw, dA_log, ddt_bias};
    e = launch_chunk_ckpt(q, k, v, bf16, g_raw, beta, A_log, dt_bias, kind, per_head, lower_bound, S0,
                          ckpt, u, eseg, ops, segbad, B, T, H, HV, K, zero, stream);
    if (e != hipSuccess) return e;
  } else {  // no tokens: only the per-head sums exist, and they are zero
    const ZeroList zl{{dq, dk, dbeta, dg_raw, dA_log, ddt_bias},
                      {nq, nq, (long)B * T * HV, ng, (long)HV, (long)HV * gK}};
    if ((e = zero(zl, stream)) != hipSuccess) return e;
  }
  BwdParams p{q, k, v, g_raw, beta, A_log, dt_bias, dout, dST, ckpt, u, ops, eseg, segbad, dq, dk, dv, dbeta,
              dg_raw, dS0, dA_log, ddt_bias, B, T, H, HV, NC, per_head, lower_bound};
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
