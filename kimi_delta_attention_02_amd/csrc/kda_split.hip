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
// The state pass is a chain of dependent products, so its per-chunk latency
// sets the pace: each chunk's W, Kt^T and gamma form one contiguous block of
// the workspace that all wavefronts copy into a double-buffered LDS slot one
// chunk ahead, and u is loaded into registers one chunk ahead.  With bf16
// inputs (K, C >= 32) W and Kt^T are stored as hi + lo bf16 pairs, and the
// chain runs on the bf16 MFMA (16x16x32, hi*hi + hi*lo + lo*hi), with the key
// (for W) and token (for Kt^T) axes permuted inside each 32-wide slice so that
// the state and U serve as B operands straight from the accumulator layout.
// Everything else, and the fp32-input chain, uses the fp32 MFMA (16x16x4);
// bf16 inputs are widened on load.
#include <mutex>
#include <type_traits>

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
  float* h;    // entry state of every chunk: the caller's [B, HV, NC, K, V] (h_plain)
               // or, in the workspace, 16 x 16 fragments (see frag_index)
  char* ops;   // workspace: per (b, hv, chunk) the LDS image of W, Kt^T, gamma
  float* u;    //            u, then U: C x V per (b, hv, chunk), as fragments
  int B, T, H, HV, NC, kind, per_head, h_plain;
  float lower_bound;
};

constexpr int kSplitThreads = 512;

// u, U and the workspace copy of h are kept as 16 x 16 MFMA accumulator
// fragments: fragment (column block cb, row block rb) of a chunk's R x N
// matrix is 64 lanes x 4 floats, lane l holding rows 16 rb + 4 (l / 16) + r
// of column 16 cb + l % 16, so every lane moves 16 contiguous bytes.
__device__ __forceinline__ long frag_index(long mat, int ncb, int nrb, int cb, int rb, int lane) {
  return (((mat * ncb + cb) * nrb + rb) * 64 + lane) * 4;
}


__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Shared memory of a chunk: the log2 cumulative decay inside each 16-token
// sub-block, and the k rows (plus q or v rows) in fp32, row stride K + 4
// (16-byte rows, spread over the banks).  The exponent of every decay factor
// is formed from these local sums and whole sub-block totals, never as the
// difference of two long prefix sums, so its rounding error scales with the
// factor's own exponent (terms of one sign add without cancellation).
template <int K, int C>
struct alignas(16) ChunkRows {
  static constexpr int LD = K + 4;
  alignas(16) float G2[C * LD];  // G2[i] = sum of log2 alpha over the sub-block of i, up to i
  alignas(16) float k[C * LD];
  alignas(16) float x[C * LD];   // q rows (output pass) or v rows (intra pass)
  alignas(16) float beta[C];
  alignas(16) float graw[C];     // per-head gate inputs
  // whole sub-block sums of G2 per channel, each added in increasing
  // sub-block order: pre[J][c] over sub-blocks 0 .. J-1 (J = 0 .. C/16),
  // suf[J][c] over sub-blocks J+1 .. C/16-1
  alignas(16) float pre[(C / 16 + 1) * K];
  alignas(16) float suf[(C / 16) * K];
  int steep[C / 16];             // sub-block whose decay leaves [2^-100, 2^100] in some channel
};

// log2 decay of whole sub-blocks J0 .. J1 - 1 in channel c
template <int K, int C>
__device__ __forceinline__ float blocks_log2(const ChunkRows<K, C>& L, int J0, int J1, int c) {
  float s = 0.0f;
  for (int J = J0; J < J1; ++J) s += L.G2[(J * 16 + 15) * ChunkRows<K, C>::LD + c];
  return s;
}

// The global inputs of one chunk as this thread loads them: raw gate inputs,
// k and q / v rows (four elements per load), beta, the per-head gate input,
// and the gate constants of its (channel, sub-block) pairs.  Issued a whole
// chunk ahead by the persistent intra and output kernels.
template <int K, int C, typename T>
struct ChunkRegs {
  static constexpr int Q4 = K / 4;
  static constexpr int NL = (C * Q4 + kSplitThreads - 1) / kSplitThreads;
  static constexpr int NPR = (K * (C / 16) + kSplitThreads - 1) / kSplitThreads;
  float4 g[NL];
  typename In<T>::Raw4 a[NL], x[NL];
  float beta, graw, alog;
  float bias[NPR];
};

template <int K, int C, typename T>
__device__ __forceinline__ void chunk_issue(const SplitParams& p, long ch, bool xq,
                                            ChunkRegs<K, C, T>& R) {
  using CR = ChunkRegs<K, C, T>;
  constexpr int Q4 = CR::Q4;
  const int tid = threadIdx.x;
  const int HV = p.HV, T_ = p.T;
  const long bh = ch / p.NC;
  const int t0 = (int)(ch % p.NC) * C;
  const int hv = (int)(bh % HV);
  const long b = bh / HV;
  const int hq = hv / (HV / p.H);
  const T* kp = static_cast<const T*>(p.k);
  const T* xp = static_cast<const T*>(xq ? p.q : p.v);
  const int xheads = xq ? p.H : HV, xh = xq ? hq : hv;
  R.alog = p.kind != KDA_GATE_NONE ? p.A_log[hv] : 0.0f;
  const int gK = p.per_head ? 1 : K;
#pragma unroll
  for (int j = 0; j < CR::NPR; ++j) {
    const int pr = tid + j * kSplitThreads, kap = pr % K;
    R.bias[j] = (p.dt_bias && p.kind != KDA_GATE_NONE && pr < K * (C / 16))
                    ? p.dt_bias[(long)hv * gK + (p.per_head ? 0 : kap)] : 0.0f;
  }
#pragma unroll
  for (int it = 0; it < CR::NL; ++it) {
    const int e = tid + it * kSplitThreads;
    const int i = e / Q4, c4 = (e % Q4) * 4;
    const int t = t0 + i;
    R.g[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e < C * Q4 && t < T_) {
      if (!p.per_head)
        R.g[it] = *reinterpret_cast<const float4*>(p.g_raw + ((b * T_ + t) * HV + hv) * (long)K + c4);
      R.a[it] = In<T>::raw4(kp, ((b * T_ + t) * p.H + hq) * (long)K + c4);
      R.x[it] = In<T>::raw4(xp, ((b * T_ + t) * xheads + xh) * (long)K + c4);
    }
  }
  R.beta = R.graw = 0.0f;
  if (tid < C && t0 + tid < T_) {
    R.beta = p.beta[(b * T_ + t0 + tid) * HV + hv];
    if (p.per_head) R.graw = p.g_raw[(b * T_ + t0 + tid) * HV + hv];
  }
}

// Chunk ch into L from the registers: G2 (see ChunkRows) and its sub-block
// sum tables, k, and q or v widened to fp32, beta.  Tokens at or past T read as g = 0, k = q = v = 0,
// beta = 0, which leave the state unchanged.  Ends with a barrier.
template <int K, int C, typename T>
__device__ void chunk_store(const SplitParams& p, long ch, const ChunkRegs<K, C, T>& R,
                            ChunkRows<K, C>& L) {
  using CR = ChunkRegs<K, C, T>;
  constexpr int LD = ChunkRows<K, C>::LD, NB = C / 16, Q4 = CR::Q4;
  const int tid = threadIdx.x;
  const int T_ = p.T;
  const int t0 = (int)(ch % p.NC) * C;
#pragma unroll
  for (int it = 0; it < CR::NL; ++it) {
    const int e = tid + it * kSplitThreads;
    const int i = e / Q4, c4 = (e % Q4) * 4;
    if (e < C * Q4) {
      float a[4] = {0.f, 0.f, 0.f, 0.f}, x[4] = {0.f, 0.f, 0.f, 0.f};
      if (t0 + i < T_) {
        In<T>::unpack4(R.a[it], a);
        In<T>::unpack4(R.x[it], x);
      }
      *reinterpret_cast<float4*>(L.G2 + i * LD + c4) = R.g[it];
      *reinterpret_cast<float4*>(L.k + i * LD + c4) = make_float4(a[0], a[1], a[2], a[3]);
      *reinterpret_cast<float4*>(L.x + i * LD + c4) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
  if (tid < NB) L.steep[tid] = 0;
  if (tid < C) {
    L.beta[tid] = R.beta;
    L.graw[tid] = R.graw;
  }
  __syncthreads();

  // gate and the cumulative sum inside each sub-block, in place: one
  // (channel, sub-block) pair per thread and pass
  const float rate = p.kind != KDA_GATE_NONE ? exp_f(R.alog) : 1.0f;
#pragma unroll
  for (int jp = 0; jp < CR::NPR; ++jp) {
    const int pr = tid + jp * kSplitThreads;
    if (pr >= K * NB) break;
    const int kap = pr % K, J = pr / K;
    float run = 0.0f;
    bool steep = false;
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const int i = J * 16 + j;
      float g = 0.0f;
      if (t0 + i < T_) {
        const float graw = p.per_head ? L.graw[i] : L.G2[i * LD + kap];
        g = gate_log_decay(graw, R.bias[jp], rate, p.kind, p.lower_bound);
      }
      run += g * kLog2e;
      steep |= !(run >= -100.0f && run <= 100.0f);
      L.G2[i * LD + kap] = run;
    }
    if (steep) L.steep[J] = 1;  // every writer stores 1
  }
  __syncthreads();
  for (int kap = tid; kap < K; kap += kSplitThreads) {
    L.pre[kap] = 0.0f;
    for (int J = 0; J < NB; ++J) {
      L.pre[(J + 1) * K + kap] = blocks_log2(L, 0, J + 1, kap);
      L.suf[J * K + kap] = blocks_log2(L, J + 1, NB, kap);
    }
  }
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

// The 16 x 16 block (I, J), I >= J, of  sum_k a_ik k_jk 2^(G_ik - G_jk) (G
// the log2 cumulative decay over the chunk), on MFMA; result in the
// accumulator layout.  I > J: the factor splits at the last token of J,
// 2^(G_i - G_Jend) 2^(G_Jend - G_j), both at most 1 for a non-positive decay.
// I == J: it splits at the start of the sub-block, 2^(Lc_i) 2^(-Lc_j), whose
// second factor is bounded by 2^100 unless the sub-block is steep (then the
// caller takes the direct form).  Entries above the diagonal are not
// meaningful.  Key channel of instruction r of step kb in lane group g:
// 16 kb + 4 g + r, so each lane reads four consecutive channels at once.
template <int K, int C>
__device__ __forceinline__ f32x4 decayed_block(const ChunkRows<K, C>& L, const float* arows, int I,
                                               int J, int lane) {
  constexpr int LD = ChunkRows<K, C>::LD;
  const int ai = I * 16 + (lane & 15), bj = J * 16 + (lane & 15), je = J * 16 + 15;
  const int c0 = 4 * (lane >> 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int kb = 0; kb < K / 16; ++kb) {
    const int c = kb * 16 + c0;
    const float4 a4 = *reinterpret_cast<const float4*>(arows + ai * LD + c);
    const float4 b4 = *reinterpret_cast<const float4*>(L.k + bj * LD + c);
    const float4 gi = *reinterpret_cast<const float4*>(L.G2 + ai * LD + c);
    const float4 gj = *reinterpret_cast<const float4*>(L.G2 + bj * LD + c);
    float4 ea = gi, eb = make_float4(-gj.x, -gj.y, -gj.z, -gj.w);
    if (I > J) {
      const float4 ge = *reinterpret_cast<const float4*>(L.G2 + je * LD + c);
      eb = make_float4(ge.x - gj.x, ge.y - gj.y, ge.z - gj.z, ge.w - gj.w);
      for (int M = J + 1; M < I; ++M) {  // whole sub-blocks between J and I
        const float4 gm = *reinterpret_cast<const float4*>(L.G2 + (M * 16 + 15) * LD + c);
        ea = make_float4(ea.x + gm.x, ea.y + gm.y, ea.z + gm.z, ea.w + gm.w);
      }
    }
    acc = mfma4(a4.x * __builtin_amdgcn_exp2f(ea.x), b4.x * __builtin_amdgcn_exp2f(eb.x), acc);
    acc = mfma4(a4.y * __builtin_amdgcn_exp2f(ea.y), b4.y * __builtin_amdgcn_exp2f(eb.y), acc);
    acc = mfma4(a4.z * __builtin_amdgcn_exp2f(ea.z), b4.z * __builtin_amdgcn_exp2f(eb.z), acc);
    acc = mfma4(a4.w * __builtin_amdgcn_exp2f(ea.w), b4.w * __builtin_amdgcn_exp2f(eb.w), acc);
  }
  return acc;
}

// The same block on hi/lo bf16 MFMA (16x16x32, three products per slice of
// 32 keys, the lo*lo term dropped): lane group g takes keys 32 s + 8 g .. +7 of
// both rows.  The decay factors are split exactly as above; bf16 keeps fp32's
// exponent range, so the 2^100 bound of the diagonal split still holds.
template <int K, int C>
__device__ __forceinline__ f32x4 decayed_block_bf16(const ChunkRows<K, C>& L, const float* arows,
                                                    int I, int J, int lane) {
  constexpr int LD = ChunkRows<K, C>::LD;
  const int ai = I * 16 + (lane & 15), bj = J * 16 + (lane & 15), je = J * 16 + 15;
  const int c0 = 8 * (lane >> 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int s = 0; s < K / 32; ++s) {
    float av[8], bv[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 32 * s + c0 + 4 * h;
      const float4 a4 = *reinterpret_cast<const float4*>(arows + ai * LD + c);
      const float4 b4 = *reinterpret_cast<const float4*>(L.k + bj * LD + c);
      const float4 gi = *reinterpret_cast<const float4*>(L.G2 + ai * LD + c);
      const float4 gj = *reinterpret_cast<const float4*>(L.G2 + bj * LD + c);
      float4 ea = gi, eb = make_float4(-gj.x, -gj.y, -gj.z, -gj.w);
      if (I > J) {
        const float4 ge = *reinterpret_cast<const float4*>(L.G2 + je * LD + c);
        eb = make_float4(ge.x - gj.x, ge.y - gj.y, ge.z - gj.z, ge.w - gj.w);
        for (int M = J + 1; M < I; ++M) {  // whole sub-blocks between J and I
          const float4 gm = *reinterpret_cast<const float4*>(L.G2 + (M * 16 + 15) * LD + c);
          ea = make_float4(ea.x + gm.x, ea.y + gm.y, ea.z + gm.z, ea.w + gm.w);
        }
      }
      av[4 * h + 0] = a4.x * __builtin_amdgcn_exp2f(ea.x);
      av[4 * h + 1] = a4.y * __builtin_amdgcn_exp2f(ea.y);
      av[4 * h + 2] = a4.z * __builtin_amdgcn_exp2f(ea.z);
      av[4 * h + 3] = a4.w * __builtin_amdgcn_exp2f(ea.w);
      bv[4 * h + 0] = b4.x * __builtin_amdgcn_exp2f(eb.x);
      bv[4 * h + 1] = b4.y * __builtin_amdgcn_exp2f(eb.y);
      bv[4 * h + 2] = b4.z * __builtin_amdgcn_exp2f(eb.z);
      bv[4 * h + 3] = b4.w * __builtin_amdgcn_exp2f(eb.w);
    }
    uint4 ah, al, bh, bl;
    split2_bf16(av[0], av[1], ah.x, al.x);
    split2_bf16(av[2], av[3], ah.y, al.y);
    split2_bf16(av[4], av[5], ah.z, al.z);
    split2_bf16(av[6], av[7], ah.w, al.w);
    split2_bf16(bv[0], bv[1], bh.x, bl.x);
    split2_bf16(bv[2], bv[3], bh.y, bl.y);
    split2_bf16(bv[4], bv[5], bh.z, bl.z);
    split2_bf16(bv[6], bv[7], bh.w, bl.w);
    const bf16x8 a_h = __builtin_bit_cast(bf16x8, ah), a_l = __builtin_bit_cast(bf16x8, al);
    const bf16x8 b_h = __builtin_bit_cast(bf16x8, bh), b_l = __builtin_bit_cast(bf16x8, bl);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_h, b_h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_h, b_l, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_l, b_h, acc, 0, 0, 0);
  }
  return acc;
}

// Every block (I, J), J <= I, of the chunk's decayed product: MFMA blocks,
// with the diagonal blocks of steep sub-blocks summed directly.  out(i, j, v)
// receives each value with j <= i (strict: j < i); the rest of the diagonal
// blocks gets 0.
template <int K, int C, bool STRICT, bool BF, class Out>
__device__ __forceinline__ void decayed_lower(const ChunkRows<K, C>& L, const float* arows, int tid,
                                              Out out) {
  constexpr int NB = C / 16, NP = NB * (NB + 1) / 2, NW = kSplitThreads / 64;
  const int lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  for (int pi = w; pi < NP; pi += NW) {
    int I, J;
    tri_pair(pi, false, I, J);
    if (I == J && L.steep[J]) continue;
    f32x4 acc;
    if constexpr (BF) acc = decayed_block_bf16<K, C>(L, arows, I, J, lane);
    else acc = decayed_block<K, C>(L, arows, I, J, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = I * 16 + 4 * g4 + r, j = J * 16 + (lane & 15);
      const bool keep = I > J || (STRICT ? j < i : j <= i);
      out(i, j, keep ? acc[r] : 0.0f);
    }
  }
  for (int J = 0; J < NB; ++J) {
    if (!L.steep[J]) continue;
    for (int e = tid; e < 256; e += kSplitThreads) {
      const int i = J * 16 + (e >> 4), j = J * 16 + (e & 15);
      const bool keep = STRICT ? j < i : j <= i;
      out(i, j, keep ? decayed_dot<K, C>(L, arows, i, j) : 0.0f);
    }
  }
}

// ----------------------------------------------------------------- chain operand layout
// Position of element e (0..31) of a 32-wide slice in the bf16 operand rows:
// lanes of group g read positions 8g .. 8g+7, which must be the elements
// 4g .. 4g+3 and 16+4g .. 16+4g+3 that the accumulator layout gives them
// (rows 4g + r of two consecutive 16-row blocks).
__device__ __forceinline__ int slice_pos(int e) { return 8 * ((e & 15) >> 2) + (e & 3) + 4 * (e >> 4); }

// The chain pass reads bf16 operands when the inputs are bf16 and both
// contractions are at least 32 long.
template <int K, int C, typename T>
struct ChainBF {
  static constexpr bool value = std::is_same<T, uint16_t>::value && K >= 32 && C >= 32;
};

// ----------------------------------------------------------------- chain operands
// The chain operands of one chunk in LDS.  fp32: W [C][K+4], Kt^T [K][C+4];
// bf16: hi and lo words of W [C][K] and Kt^T [K][C], unpadded, with the
// 16-byte chunk j of row r at chunk position j ^ (r mod chunks per row)
// (see img_pos), so that the operand reads of 16 rows spread over the banks;
// then gamma [K].
template <int K, int C, bool BF>
struct ChainOps;
template <int K, int C>
struct alignas(16) ChainOps<K, C, false> {
  static constexpr int LW = K + 4, LK = C + 4;
  alignas(16) float w[C * LW];
  alignas(16) float kt[K * LK];
  alignas(16) float gam[K];
};
template <int K, int C>
struct alignas(16) ChainOps<K, C, true> {
  static constexpr int LW = K, LK = C;
  alignas(16) uint16_t wh[C * LW];
  alignas(16) uint16_t wl[C * LW];
  alignas(16) uint16_t kh[K * LK];
  alignas(16) uint16_t kl[K * LK];
  alignas(16) float gam[K];
};

// Element offset of 16-byte chunk j of row r in a bf16 image array of rows of
// N elements (N / 8 chunks, a power of two).
template <int N>
__device__ __forceinline__ int img_pos(int r, int j) {
  return r * N + 8 * (j ^ (r & (N / 8 - 1)));
}

// Bytes of one chunk's image in the workspace: the larger layout, rounded
// up to whole 1 KiB copies (one wavefront-wide 16-byte load per lane).
template <int K, int C>
constexpr int split_image_bytes() {
  constexpr int a = (int)sizeof(ChainOps<K, C, false>), b = (int)sizeof(ChainOps<K, C, true>);
  return ((a > b ? a : b) + 1023) / 1024 * 1024;
}

// ----------------------------------------------------------------- intra
template <int K, int C, typename T>
__global__ __launch_bounds__(kSplitThreads) void split_intra_kernel(SplitParams p) {
  constexpr int NB = C / 16, LD = ChunkRows<K, C>::LD, LR = C + 4, LX = 20;
  constexpr bool BF = ChainBF<K, C, T>::value;
  __shared__ ChunkRows<K, C> L;
  __shared__ alignas(16) float R[C * LR];
  __shared__ alignas(16) float Xd[NB * 16 * LX];
  __shared__ alignas(16) float Ws[C * LD];  // W in fp32, rows of keys, before the image layout
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  const long nch = (long)p.B * p.HV * p.NC;
  ChunkRegs<K, C, T> cr;
  if ((long)blockIdx.x < nch) chunk_issue<K, C, T>(p, blockIdx.x, false, cr);
  for (long ch = blockIdx.x; ch < nch; ch += gridDim.x) {
  chunk_store<K, C, T>(p, ch, cr, L);
  if (ch + gridDim.x < nch) chunk_issue<K, C, T>(p, ch + gridDim.x, false, cr);  // lands during this chunk

  // R = diag(beta) times the strictly lower decayed k k^T
  decayed_lower<K, C, true, std::is_same<T, uint16_t>::value && K >= 32>(
      L, L.k, tid, [&](int i, int j, float v) { R[i * LR + j] = L.beta[i] * v; });
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
  // Y_I = X_II (B_I - sum_{J<I} R_IJ Y_J); each wavefront takes two 16-wide
  // column blocks at a time (two independent product chains)
  constexpr int NCB = 2 * (K / 16);
  for (int cb0 = 2 * w; cb0 < NCB; cb0 += 2 * (kSplitThreads / 64)) {
    f32x4 y[2][NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4 t[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cb = cb0 + h;
        const bool isw = cb < K / 16;
        const int col = (isw ? cb : cb - K / 16) * 16 + (lane & 15);
        float pre = 0.0f;
        if (isw) pre = L.pre[I * K + col];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = I * 16 + 4 * g4 + r;
          const float x = isw ? L.k[i * LD + col] * __builtin_amdgcn_exp2f(L.G2[i * LD + col] + pre)
                              : L.x[i * LD + col];
          t[h][r] = L.beta[i] * x;
        }
      }
#pragma unroll
      for (int J = 0; J < I; ++J) {
        const float4 a = *reinterpret_cast<const float4*>(R + (I * 16 + (lane & 15)) * LR + J * 16 + 4 * g4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          t[h] = mfma4(-a.x, y[h][J][0], t[h]);
          t[h] = mfma4(-a.y, y[h][J][1], t[h]);
          t[h] = mfma4(-a.z, y[h][J][2], t[h]);
          t[h] = mfma4(-a.w, y[h][J][3], t[h]);
        }
      }
      const float4 a = *reinterpret_cast<const float4*>(Xd + (I * 16 + (lane & 15)) * LX + 4 * g4);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mfma4(a.x, t[h][0], z);
        z = mfma4(a.y, t[h][1], z);
        z = mfma4(a.z, t[h][2], z);
        z = mfma4(a.w, t[h][3], z);
        y[h][I] = z;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cb = cb0 + h;
      if (cb >= K / 16) {  // u: fragments straight to the workspace
#pragma unroll
        for (int I = 0; I < NB; ++I)
          *reinterpret_cast<f32x4*>(p.u + frag_index(ch, K / 16, NB, cb - K / 16, I, lane)) = y[h][I];
      } else {  // W: through LDS, to be written out in the image layout
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
          for (int r = 0; r < 4; ++r) Ws[(I * 16 + 4 * g4 + r) * LD + cb * 16 + (lane & 15)] = y[h][I][r];
      }
    }
  }
  __syncthreads();

  // the chunk's operand image: W, Kt^T and gamma, 16 bytes per store
  using Ops = ChainOps<K, C, BF>;
  Ops& img = *reinterpret_cast<Ops*>(p.ops + ch * (long)split_image_bytes<K, C>());
  if constexpr (BF) {
    // W rows: positions 8 g .. 8 g + 7 of key slice q are keys 32 q + 4 g + (0..3)
    // and 32 q + 16 + 4 g + (0..3)
    for (int e = tid; e < C * (K / 8); e += kSplitThreads) {
      const int i = e / (K / 8), q = (e % (K / 8)) >> 2, g = e & 3;
      const float4 lo4 = *reinterpret_cast<const float4*>(Ws + i * LD + 32 * q + 4 * g);
      const float4 hi4 = *reinterpret_cast<const float4*>(Ws + i * LD + 32 * q + 16 + 4 * g);
      uint4 h, l;
      split2_bf16(lo4.x, lo4.y, h.x, l.x);
      split2_bf16(lo4.z, lo4.w, h.y, l.y);
      split2_bf16(hi4.x, hi4.y, h.z, l.z);
      split2_bf16(hi4.z, hi4.w, h.w, l.w);
      *reinterpret_cast<uint4*>(img.wh + img_pos<Ops::LW>(i, 4 * q + g)) = h;
      *reinterpret_cast<uint4*>(img.wl + img_pos<Ops::LW>(i, 4 * q + g)) = l;
    }
    // Kt^T rows (key channels): token slices permuted the same way
    for (int e = tid; e < K * (C / 8); e += kSplitThreads) {
      const int kap = e / (C / 8), q = (e % (C / 8)) >> 2, g = e & 3;
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int i = 32 * q + 4 * g + (m & 3) + 16 * (m >> 2);
        const int I = i >> 4;
        const float rest = (L.G2[(I * 16 + 15) * LD + kap] - L.G2[i * LD + kap]) + L.suf[I * K + kap];
        v[m] = L.k[i * LD + kap] * __builtin_amdgcn_exp2f(rest);
      }
      uint4 h, l;
      split2_bf16(v[0], v[1], h.x, l.x);
      split2_bf16(v[2], v[3], h.y, l.y);
      split2_bf16(v[4], v[5], h.z, l.z);
      split2_bf16(v[6], v[7], h.w, l.w);
      *reinterpret_cast<uint4*>(img.kh + img_pos<Ops::LK>(kap, 4 * q + g)) = h;
      *reinterpret_cast<uint4*>(img.kl + img_pos<Ops::LK>(kap, 4 * q + g)) = l;
    }
  } else {
    for (int e = tid; e < C * (K / 4); e += kSplitThreads) {
      const int i = e / (K / 4), c4 = (e % (K / 4)) * 4;
      *reinterpret_cast<float4*>(img.w + i * Ops::LW + c4) = *reinterpret_cast<const float4*>(Ws + i * LD + c4);
    }
    for (int e = tid; e < K * (C / 4); e += kSplitThreads) {
      const int kap = e / (C / 4), i0 = (e % (C / 4)) * 4;
      float v[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = i0 + m, I = i >> 4;
        const float rest = (L.G2[(I * 16 + 15) * LD + kap] - L.G2[i * LD + kap]) + L.suf[I * K + kap];
        v[m] = L.k[i * LD + kap] * __builtin_amdgcn_exp2f(rest);
      }
      *reinterpret_cast<float4*>(img.kt + kap * Ops::LK + i0) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
  for (int kap = tid; kap < K; kap += kSplitThreads)
    img.gam[kap] = __builtin_amdgcn_exp2f(L.pre[NB * K + kap]);
  __syncthreads();  // LDS is refilled by the next chunk
  }
}

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// hi and lo words of eight values (two accumulator fragments) as bf16x8 operands
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  uint4 h, l;
  split2_bf16(a[0], a[1], h.x, l.x);
  split2_bf16(a[2], a[3], h.y, l.y);
  split2_bf16(b[0], b[1], h.z, l.z);
  split2_bf16(b[2], b[3], h.w, l.w);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// u of chunk index ch, column block cb: the lane's fragments
template <int K, int C>
__device__ __forceinline__ void fetch_u(const SplitParams& p, long ch, f32x4 (&un)[C / 16], int cb,
                                        int lane) {
#pragma unroll
  for (int I = 0; I < C / 16; ++I)
    un[I] = *reinterpret_cast<const f32x4*>(p.u + frag_index(ch, K / 16, C / 16, cb, I, lane));
}

// Copies n bytes (a multiple of 16) from the workspace into LDS with direct
// global-to-LDS loads: 16 bytes per lane, 1 KiB per wavefront instruction, no
// registers involved; copier wavefront cw of NCP takes every NCP-th KiB.
template <int NCP, int N>
__device__ __forceinline__ void copy_to_lds(const char* src, char* dst, int cw, int lane) {
  constexpr int ROUNDS = (N + NCP * 1024 - 1) / (NCP * 1024);
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int j = (r * NCP + cw) * 1024;
    if (j + lane * 16 < N)
      __builtin_amdgcn_global_load_lds(src + j + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + j), 16, 0, 0);
  }
}

// The direct copies count as vector memory loads of the issuing wavefront,
// and its LDS waits cover them too; the barrier's own waits do not, so the
// copying wavefront waits for them (vmcnt(0)) before the barrier that
// publishes them.
__device__ __forceinline__ void image_landed() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Byte ranges of a chunk's image: W (or its hi/lo pair) first, then Kt^T and
// gamma.
template <int K, int C, bool BF>
struct ImageHalves {
  using Ops = ChainOps<K, C, BF>;
  static constexpr int WB = (int)(sizeof(Ops::w) + 0);                         // W bytes
  static constexpr int KB = (int)sizeof(Ops) - WB;                             // Kt^T + gamma bytes
  static constexpr int GOFF = (int)(sizeof(Ops::kt) + 0);                      // gamma within them
};
template <int K, int C>
struct ImageHalves<K, C, true> {
  using Ops = ChainOps<K, C, true>;
  static constexpr int WB = (int)(sizeof(Ops::wh) + sizeof(Ops::wl));
  static constexpr int KB = (int)sizeof(Ops) - WB;
  static constexpr int GOFF = (int)(sizeof(Ops::kh) + sizeof(Ops::kl));
};

// One workgroup per (b, hv, 16-wide column block of the state): one
// wavefront holds that block of the fp32 state in registers for the whole
// sequence, lane l rows 16 kb + 4 (l / 16) + r of column l % 16 (the MFMA
// accumulator layout, which is also the B operand layout of the fp32
// products; the bf16 products take two such fragments per 32-wide slice).
// Further wavefronts only stream operands into LDS, so the copy's latency
// never enters the computing wavefront's LDS waits; several of them keep
// enough copies in flight (one wavefront can have 63 outstanding).
//
// The chain is software-pipelined across chunks: iteration c forms h_{c+1} =
// diag(gamma_c) h_c + Kt_c^T U_c one 32-row slice at a time and, as each slice
// is final, adds its part of W_{c+1} h_{c+1}, so the products of the two
// halves of the recurrence keep the matrix core busy together; U_{c+1} =
// u_{c+1} - W_{c+1} h_{c+1} closes the iteration.  W and Kt^T are therefore
// double-buffered separately: iteration c reads Kt_c and W_{c+1} while the
// copier brings Kt_{c+1} and W_{c+2}.  The column blocks of a head are
// independent workgroups with equal blockIdx % 8, so one XCD's L2 serves
// their common operand images.
#ifndef KDA_STATE_COPIERS
#define KDA_STATE_COPIERS 4
#endif
constexpr int kCopiers = KDA_STATE_COPIERS;  // copying wavefronts per state-pass workgroup

template <int K, int C, bool BF>
__global__ __launch_bounds__(64 * (1 + kCopiers)) void split_state_kernel(SplitParams p) {
  constexpr int NB = C / 16, NKB = K / 16, IMG = split_image_bytes<K, C>();
  using Ops = ChainOps<K, C, BF>;
  using IH = ImageHalves<K, C, BF>;
  constexpr int WB = IH::WB, KB = IH::KB;
  constexpr int WBR = (WB + 15) / 16 * 16, KBR = (KB + 15) / 16 * 16;
  __shared__ alignas(16) char wbuf[2][WBR];
  __shared__ alignas(16) char kbuf[2][KBR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  const long nh = (long)p.B * p.HV;
  const long bh = blockIdx.x % nh;
  const int cb = (int)(blockIdx.x / nh);
  const int NC = p.NC;
  const int col = cb * 16 + (lane & 15);
  const char* src = p.ops + bh * NC * (long)IMG;  // image of chunk c at src + c IMG

  if (w >= 1) {  // the copying wavefronts: the same barriers as the computing one
    const int cw = w - 1;
    if (NC > 0) {
      copy_to_lds<kCopiers, WB>(src, wbuf[0], cw, lane);
      copy_to_lds<kCopiers, KB>(src + WB, kbuf[0], cw, lane);
      if (NC > 1) copy_to_lds<kCopiers, WB>(src + IMG, wbuf[1], cw, lane);
    }
    image_landed();
    __syncthreads();
    __syncthreads();  // W_0 consumed
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) copy_to_lds<kCopiers, KB>(src + (c + 1) * (long)IMG + WB, kbuf[(c + 1) & 1], cw, lane);
      if (c + 2 < NC) copy_to_lds<kCopiers, WB>(src + (c + 2) * (long)IMG, wbuf[c & 1], cw, lane);
      image_landed();
      __syncthreads();
    }
    return;
  }

  // operand views of the buffers
  auto Wv = [&](int slot) { return reinterpret_cast<const char*>(wbuf[slot]); };
  auto Kv = [&](int slot) { return reinterpret_cast<const char*>(kbuf[slot]); };

  f32x4 s[NKB];
  const float* S0 = p.S0 ? p.S0 + bh * (long)K * K : nullptr;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[kb][r] = S0 ? S0[(kb * 16 + 4 * g4 + r) * K + col] : 0.0f;
  f32x4 x[NB], un[NB];
  if (NC > 0) fetch_u<K, C>(p, bh * NC, x, cb, lane);
  if (NC > 1) fetch_u<K, C>(p, bh * NC + 1, un, cb, lane);
  __syncthreads();

  // X_c: add the part of W h over key slice q (bf16) or key block kb (fp32)
  auto x_part = [&](const char* wsrc, int q) {
    if constexpr (BF) {
      const uint16_t* wh = reinterpret_cast<const uint16_t*>(wsrc);
      const uint16_t* wl = wh + C * Ops::LW;
      bf16x8 bh_, bl_, ah[NB], al[NB];
      split8(s[2 * q], s[2 * q + 1], bh_, bl_);
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const int pos = img_pos<Ops::LW>(I * 16 + (lane & 15), 4 * q + g4);
        ah[I] = *reinterpret_cast<const bf16x8*>(wh + pos);
        al[I] = *reinterpret_cast<const bf16x8*>(wl + pos);
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) x[I] = mfma32(ah[I], bh_, x[I]);
#pragma unroll
      for (int I = 0; I < NB; ++I) x[I] = mfma32(ah[I], bl_, x[I]);
#pragma unroll
      for (int I = 0; I < NB; ++I) x[I] = mfma32(al[I], bh_, x[I]);
    } else {
      const float* wf = reinterpret_cast<const float*>(wsrc);
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const float4 a = *reinterpret_cast<const float4*>(wf + (I * 16 + (lane & 15)) * Ops::LW + q * 16 + 4 * g4);
        x[I] = mfma4(a.x, s[q][0], x[I]);
        x[I] = mfma4(a.y, s[q][1], x[I]);
        x[I] = mfma4(a.z, s[q][2], x[I]);
        x[I] = mfma4(a.w, s[q][3], x[I]);
      }
    }
  };
  constexpr int NQ = BF ? K / 32 : NKB;  // key slices (bf16) or blocks (fp32) of x_part
  constexpr int RPQ = BF ? 2 : 1;        // state row blocks per slice

  // X_0 = W_0 h_0, then U_0 = u_0 - X_0
  if (NC > 0) {
    f32x4 xw[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      xw[I] = x[I];
      x[I] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) x_part(Wv(0), q);
#pragma unroll
    for (int I = 0; I < NB; ++I) x[I] = xw[I] - x[I];
  }
  __syncthreads();  // W_0 consumed

  for (int c = 0; c < NC; ++c) {
    const long ch = bh * NC + c;
    const bool more = c + 1 < NC;
    // this iteration's U and h_c go out; u_{c+2} comes in
    f32x4 ucur[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      ucur[I] = x[I];
      *reinterpret_cast<f32x4*>(p.u + frag_index(ch, NKB, NB, cb, I, lane)) = x[I];
      x[I] = un[I];  // u_{c+1}: X_{c+1} accumulates into its negative below
    }
    if (c + 2 < NC) fetch_u<K, C>(p, ch + 2, un, cb, lane);
    if (p.h_plain) {
      float* hc = p.h + ch * (long)K * K;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) hc[(kb * 16 + 4 * g4 + r) * K + col] = s[kb][r];
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        *reinterpret_cast<f32x4*>(p.h + frag_index(ch, NKB, NKB, cb, kb, lane)) = s[kb];
    }
    // X_{c+1} is accumulated negated onto u_{c+1}, so U_{c+1} = x at the end
#pragma unroll
    for (int I = 0; I < NB; ++I) x[I] = -x[I];

    const char* kt = Kv(c & 1);
    const float* gm = reinterpret_cast<const float*>(kt + IH::GOFF);
    bf16x8 uh[NB / 2 > 0 ? NB / 2 : 1], ul[NB / 2 > 0 ? NB / 2 : 1];
    if constexpr (BF) {
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) split8(ucur[2 * q], ucur[2 * q + 1], uh[q], ul[q]);
    }
    // rows of h_{c+1} in slices; each finished slice feeds X_{c+1}
    auto s_part = [&](int q) {
#pragma unroll
      for (int rr = 0; rr < RPQ; ++rr) {
        const int kb = q * RPQ + rr;
        const float4 gg = *reinterpret_cast<const float4*>(gm + kb * 16 + 4 * g4);
        s[kb] = f32x4{gg.x * s[kb][0], gg.y * s[kb][1], gg.z * s[kb][2], gg.w * s[kb][3]};
      }
      if constexpr (BF) {
        const uint16_t* kh = reinterpret_cast<const uint16_t*>(kt);
        const uint16_t* kl = kh + K * Ops::LK;
#pragma unroll
        for (int t = 0; t < NB / 2; ++t) {
          bf16x8 ah[RPQ], al[RPQ];
#pragma unroll
          for (int rr = 0; rr < RPQ; ++rr) {
            const int pos = img_pos<Ops::LK>((q * RPQ + rr) * 16 + (lane & 15), 4 * t + g4);
            ah[rr] = *reinterpret_cast<const bf16x8*>(kh + pos);
            al[rr] = *reinterpret_cast<const bf16x8*>(kl + pos);
          }
#pragma unroll
          for (int rr = 0; rr < RPQ; ++rr) s[q * RPQ + rr] = mfma32(ah[rr], uh[t], s[q * RPQ + rr]);
#pragma unroll
          for (int rr = 0; rr < RPQ; ++rr) s[q * RPQ + rr] = mfma32(ah[rr], ul[t], s[q * RPQ + rr]);
#pragma unroll
          for (int rr = 0; rr < RPQ; ++rr) s[q * RPQ + rr] = mfma32(al[rr], uh[t], s[q * RPQ + rr]);
        }
      } else {
        const float* kf = reinterpret_cast<const float*>(kt);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          const float4 a = *reinterpret_cast<const float4*>(kf + (q * 16 + (lane & 15)) * Ops::LK + I * 16 + 4 * g4);
          s[q] = mfma4(a.x, ucur[I][0], s[q]);
          s[q] = mfma4(a.y, ucur[I][1], s[q]);
          s[q] = mfma4(a.z, ucur[I][2], s[q]);
          s[q] = mfma4(a.w, ucur[I][3], s[q]);
        }
      }
    };
    s_part(0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q + 1 < NQ) s_part(q + 1);
      if (more) x_part(Wv((c + 1) & 1), q);
    }
#pragma unroll
    for (int I = 0; I < NB; ++I) x[I] = -x[I];  // U_{c+1} = u_{c+1} - X_{c+1}
    __syncthreads();  // next operands in place; these may be overwritten
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
  __shared__ alignas(16) float A[C * LR];
  float* Q = L.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const long nch = (long)p.B * p.HV * p.NC;
  ChunkRegs<K, C, T> cr;
  if ((long)blockIdx.x < nch) chunk_issue<K, C, T>(p, blockIdx.x, true, cr);
  for (long ch = blockIdx.x; ch < nch; ch += gridDim.x) {
  const long bh = ch / p.NC;
  const int c = (int)(ch % p.NC);
  chunk_store<K, C, T>(p, ch, cr, L);
  if (ch + gridDim.x < nch) chunk_issue<K, C, T>(p, ch + gridDim.x, true, cr);  // lands during this chunk

  // A = s times the lower (diagonal included) decayed q k^T
  decayed_lower<K, C, false, std::is_same<T, uint16_t>::value && K >= 32>(
      L, Q, tid, [&](int i, int j, float v) { A[i * LR + j] = scale * v; });
  __syncthreads();
  // Q <- s q exp(G)
  for (int e = tid; e < C * K; e += kSplitThreads) {
    const int i = e / K, kap = e % K;
    Q[i * LD + kap] *= scale * __builtin_amdgcn_exp2f(L.G2[i * LD + kap] + L.pre[(i >> 4) * K + kap]);
  }
  __syncthreads();

  const int hv = (int)(bh % p.HV);
  const long b = bh / p.HV;
  const int t0 = c * C;
  constexpr int NKB = K / 16;
  for (int cb = w; cb < NKB; cb += kSplitThreads / 64) {
    const int col = cb * 16 + (lane & 15);
    // h_c as B operand fragments: lane holds keys 16 kb + 4 (l / 16) + r
    f32x4 hf[NKB];
    if (p.h_plain) {
      const float* hc = p.h + ch * (long)K * K;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) hf[kb][r] = hc[(kb * 16 + 4 * g4 + r) * K + col];
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        hf[kb] = *reinterpret_cast<const f32x4*>(p.h + frag_index(ch, NKB, NKB, cb, kb, lane));
    }
    f32x4 uf[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J)
      uf[J] = *reinterpret_cast<const f32x4*>(p.u + frag_index(ch, NKB, NB, cb, J, lane));
#pragma unroll 1
    for (int I = 0; I < NB; ++I) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* qrow = Q + (I * 16 + (lane & 15)) * LD + 4 * g4;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const float4 a = *reinterpret_cast<const float4*>(qrow + kb * 16);
        acc = mfma4(a.x, hf[kb][0], acc);
        acc = mfma4(a.y, hf[kb][1], acc);
        acc = mfma4(a.z, hf[kb][2], acc);
        acc = mfma4(a.w, hf[kb][3], acc);
      }
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J > I) break;
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
  __syncthreads();  // LDS is refilled by the next chunk
  }
}

// ----------------------------------------------------------------- launch
template <int K, int C, typename T>
static hipError_t launch_split_kc(const SplitParams& p, hipStream_t stream) {
  const long heads = (long)p.B * p.HV;
  const long chunks = heads * p.NC;
  // the intra and output kernels are persistent: one workgroup per compute
  // unit (their LDS allows no more), each walking chunks with a stride of
  // the grid and loading the next chunk's inputs while it computes this one
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const unsigned grid = (unsigned)(chunks < cus ? chunks : cus);
  if (chunks > 0) {
    hipLaunchKernelGGL((split_intra_kernel<K, C, T>), dim3(grid), dim3(kSplitThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((split_state_kernel<K, C, ChainBF<K, C, T>::value>),
                     dim3((unsigned)(heads * (K / 16))), dim3(64 * (1 + kCopiers)), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunks == 0 || !p.o) return e;  // no o wanted: the states and U only
  hipLaunchKernelGGL((split_output_kernel<K, C, T>), dim3(grid), dim3(kSplitThreads), 0, stream, p);
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

// Workspace bytes per (b, hv, chunk): the chain operand image, u / U and the
// entry state.
static size_t image_bytes(int K, int C) {
#define KDA_IMG_CASE(KK, CC) \
  if (K == KK && C == CC) return (size_t)split_image_bytes<KK, CC>();
#define KDA_IMG_ROW(KK) KDA_IMG_CASE(KK, 16) KDA_IMG_CASE(KK, 32) KDA_IMG_CASE(KK, 64)
  KDA_IMG_ROW(16) KDA_IMG_ROW(32) KDA_IMG_ROW(64) KDA_IMG_ROW(128)
#undef KDA_IMG_ROW
#undef KDA_IMG_CASE
  return 0;
}

size_t split_workspace_bytes_per_chunk(int K, int V, int C) {
  return image_bytes(K, C) + ((size_t)C * V + (size_t)K * V) * sizeof(float);
}

// Scratch of the allocation-free entry point (kda_chunk_fwd_split_noalloc): the
// split schedule's workspace in a fixed device array.  Each device holds its
// own copy for the life of the process; host code must never pass the array's
// name to a kernel (on the host it only stands for the symbol), only the
// device address hipGetSymbolAddress gives for the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// This device's address of `scratch`, looked up once per device (the first
// call on it) and kept; the lookup allocates nothing.
hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
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
  p.ops = static_cast<char*>(workspace);
  p.u = ws ? reinterpret_cast<float*>(p.ops + n * image_bytes(K, C)) : nullptr;
  p.h = h ? h : (ws ? p.u + n * (size_t)C * K : nullptr);
  p.h_plain = h ? 1 : 0;
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
