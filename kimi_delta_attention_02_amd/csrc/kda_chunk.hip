// Chunkwise KDA forward: gate, intra-chunk triangular solve and inter-chunk
// state propagation fused in one kernel.
//
// Algebra (the "DeltaNet family" page, section "Chunkwise KDA", written in the
// K x V state layout of the "K3 notes").  For a block of n = 16 tokens entering
// with state S, with E_i = prod_{m<=i} alpha_m (alpha = exp(g), per key
// channel), gamma = E_{n-1} and Suf_j = prod_{m>j} alpha_m = gamma / E_j:
//
//   temporary errors   Ebar_i = beta_i (v_i - (k_i * E_i) . S)
//   coupling           R_ij   = beta_i sum_c k_ic k_jc E_ic / E_jc        (j < i)
//   resolved errors    U      = (I + R)^{-1} Ebar        (causal triangular solve)
//   outputs            O_i    = s (q_i * E_i) . S + sum_{j<=i} A_ij U_j,
//                      A_ij   = s sum_c q_ic k_jc E_ic / E_jc             (j <= i)
//   block-end state    S'     = diag(gamma) S + (k * Suf)^T U
//
// with s = 1/sqrt(K).  The ratio E_i / E_j is factored as (x_i E_i / gamma) .
// (y_j Suf_j): both factors stay finite as long as gamma >= 2^-100 in every
// channel (at most 69 nats of decay inside 16 tokens; the safe gate with
// lower bound -5 never exceeds 80 nats, and real data far less).  A block
// that breaks the bound is run token by token instead (same recurrence, no
// factorisation), so every input is handled exactly.
//
// Schedule.  One workgroup (4 wavefronts) owns one (sequence b, value head hv,
// 32-wide value tile) and walks the sequence in 16-token blocks, keeping its
// K x 32 slice of the fp32 state in registers (MFMA accumulator layout) for
// the whole sequence.  The four value tiles of one head are placed on the same
// XCD so that their shared q, k, g_raw reads hit that XCD's L2.  Per block:
//   prep   all threads: gate, cumulative products, scaled operands -> LDS
//   B      wave 0: A (MFMA); wave 1: R (MFMA); waves 2..: K_hat S, Q_hat S, Ebar
//   B2     wave 1: (I + R)^{-1} by forward substitution (fp32)
//   C      waves 2..: U = (I + R)^{-1} Ebar
//   D      waves 2..: O;  all waves: state update of their own state blocks
// bf16 inputs use bf16 MFMA with fp32 accumulation.  Every operand of these
// products is derived (scaled by decay factors, the state, or a solve result),
// and a single bf16 rounding of them costs far more than the 1e-2 error budget
// (the outputs are ~100x smaller than the values they are built from), so each
// operand is carried as a pair of bf16 words hi + lo (~16 significant bits) and
// a product takes 3 MFMAs (hi*hi + hi*lo + lo*hi) over the key axis, or 2 over
// the 16-token axis, where one k = 32 instruction covers the hi and lo halves.
// fp32 inputs use fp32 MFMA throughout.
#include <type_traits>

#include "kda_device.h"

namespace kda {

struct ChunkParams {
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
  int B, T, H, HV, kind;
  float lower_bound;
};

constexpr int kTok = 16;     // tokens per block
constexpr int kCat = 40;     // row stride of [hi t0..15 | lo t0..15] operands (+8 pad)
constexpr float kGammaMin = 7.888609052210118e-31f;  // 2^-100
constexpr float kGammaMax = 1.2676506002282294e30f;  // 2^100 (only a positive log-decay can get here)

// ------------------------------------------------------------------ LDS

template <int K, int BV>
struct SmemBF16 {
  static constexpr int LD = K + 8;  // row stride of [16][K] and [BV][K] operands
  uint16_t qr_hi[kTok * LD], qr_lo[kTok * LD];  // q E / gamma      rows of A
  uint16_t qh_hi[kTok * LD], qh_lo[kTok * LD];  // q E              Q_hat S
  uint16_t kr_hi[kTok * LD], kr_lo[kTok * LD];  // k E / gamma      rows of R
  uint16_t kh_hi[kTok * LD], kh_lo[kTok * LD];  // k E              K_hat S
  uint16_t ke_hi[kTok * LD], ke_lo[kTok * LD];  // k Suf            columns of A and R
  uint16_t keT[K * kCat];                       // (k Suf)^T  [c][hi t | lo t]
  uint16_t st_hi[BV * LD], st_lo[BV * LD];      // S^T        [v][c]
  uint16_t aqk[kTok * kCat];                    // A          [i][hi j | lo j]
  uint16_t akk[kTok * kCat];                    // (I+R)^-1   [i][hi j | lo j]
  uint16_t ebT[BV * kCat];                      // Ebar^T     [v][hi t | lo t]
  uint16_t uT[BV * kCat];                       // U^T        [v][hi t | lo t]
  float r[kTok * 17 > (K / 16) * BV ? kTok * 17 : (K / 16) * BV];
  float gam[K];
  float beta[kTok];
};

template <int K, int BV>
struct SmemF32 {
  static constexpr int LD = K + 1;
  float qr[kTok * LD], qh[kTok * LD], kr[kTok * LD], kh[kTok * LD], ke[kTok * LD];
  float keT[K * 17];  // [c][t]
  float st[BV * LD];  // [v][c]
  float aqk[kTok * 17], akk[kTok * 17];
  float ebT[BV * 17], uT[BV * 17];
  float r[kTok * 17 > (K / 16) * BV ? kTok * 17 : (K / 16) * BV];
  float gam[K];
  float beta[kTok];
};

// ------------------------------------------------------------ MFMA tiles
// Output fragments use the 16x16 accumulator layout: lane l holds rows
// 4 * (l / 16) + r (r = 0..3) of column l % 16.

// acc += A (16 x K, row-major) * Bt^T, where Bt (16 x K, row-major) holds the
// columns of B.  HL = 1: hi*hi.  HL = 3: hi*hi + hi*lo + lo*hi.
template <int K, int HL>
__device__ __forceinline__ void mma_kappa_bf16(f32x4& acc, const uint16_t* Ah, const uint16_t* Al,
                                               const uint16_t* Bh, const uint16_t* Bl, int ld,
                                               int lane) {
  const int row = lane & 15;
  if constexpr (K % 32 == 0) {
    const int kq = (lane >> 4) * 8;
#pragma unroll
    for (int s = 0; s < K; s += 32) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ah + row * ld + s + kq);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bh + row * ld + s + kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      if constexpr (HL == 3) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + row * ld + s + kq);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Bl + row * ld + s + kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
      }
    }
  } else {  // K == 16
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const int kq = (lane >> 4) * 4;
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(Ah + row * ld + kq);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(Bh + row * ld + kq);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    if constexpr (HL == 3) {
      const bf16x4 al = *reinterpret_cast<const bf16x4*>(Al + row * ld + kq);
      const bf16x4 bl = *reinterpret_cast<const bf16x4*>(Bl + row * ld + kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, b, acc, 0, 0, 0);
    }
  }
}

// acc += A (16 x 16 tokens) * B (16 tokens x 16) over the token axis, with
// operands stored as rows [hi t0..15 | lo t0..15] (A by row, B by column):
// (A_hi + A_lo)(B_hi + B_lo) in two MFMAs, since one k = 32 instruction takes
// the hi and the lo half of A against the same half of B.
__device__ __forceinline__ void mma_tok_bf16(f32x4& acc, const uint16_t* Acat, const uint16_t* Bcat,
                                             int lane) {
  const int row = lane & 15, g = lane >> 4;
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(Acat + row * kCat + 8 * g);
  const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(Bcat + row * kCat + 8 * (g & 1));
  const bf16x8 b2 = *reinterpret_cast<const bf16x8*>(Bcat + row * kCat + 16 + 8 * (g & 1));
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, acc, 0, 0, 0);
}

// fp32: acc += A (16 x n, row stride lda) * Bt^T (Bt: 16 x n, stride ldb).
template <int N>
__device__ __forceinline__ void mma_f32(f32x4& acc, const float* A, int lda, const float* Bt,
                                        int ldb, int lane) {
  const int row = lane & 15, kk = lane >> 4;
#pragma unroll
  for (int s = 0; s < N; s += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[row * lda + s + kk], Bt[row * ldb + s + kk], acc,
                                               0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo_half, uint16_t hi_half) {
  return (uint32_t)lo_half | ((uint32_t)hi_half << 16);
}

// ----------------------------------------------------------------- kernel

template <int K, typename T>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkParams p) {
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr int V = K;
  constexpr int BV = V < 32 ? V : 32;
  constexpr int NCB = BV / 16, NKB = K / 16, NVT = V / BV;
  constexpr int NBLK = NKB * NCB;
  constexpr int BPW = (NBLK + 3) / 4;
  using Smem = typename std::conditional<F32, SmemF32<K, BV>, SmemBF16<K, BV>>::type;
  constexpr int LD = Smem::LD;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T_ = p.T, HV = p.HV, H = p.H;

  // workgroup -> (head, value tile): the NVT tiles of a head share blockIdx % 8
  const int nheads = p.B * HV;
  const int x8 = blockIdx.x & 7, y8 = blockIdx.x >> 3;
  const int hd = (y8 / NVT) * 8 + x8, vt = y8 % NVT;
  if (hd >= nheads) return;
  const long b = hd / HV;
  const int hv = hd % HV;
  const int h = hv / (HV / H);
  const int v0 = vt * BV;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const float rate = p.kind != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const float* bias = (p.dt_bias && p.kind != KDA_GATE_NONE) ? p.dt_bias + (long)hv * K : nullptr;
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);

  // ---- state slice: blocks blk = w + 4 i, (kb, cb) = (blk / NCB, blk % NCB)
  f32x4 sacc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int blk = w + 4 * i;
    if (blk < NBLK && p.S0) {
      const int kb = blk / NCB, cb = blk % NCB;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * kb + 4 * (lane >> 4) + r;
        sacc[i][r] = p.S0[((long)hd * K + c) * V + v0 + 16 * cb + (lane & 15)];
      }
    }
  }

  // S^T operand for the next block's products with the state
  auto write_state_operand = [&]() {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = w + 4 * i;
      if (blk >= NBLK) continue;
      const int kb = blk / NCB, cb = blk % NCB;
      const int vcol = 16 * cb + (lane & 15), c0 = 16 * kb + 4 * (lane >> 4);
      if constexpr (F32) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.st[vcol * LD + c0 + r] = sacc[i][r];
      } else {
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) split_bf16(sacc[i][r], hi[r], lo[r]);
        *reinterpret_cast<uint2*>(sm.st_hi + vcol * LD + c0) = uint2{pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
        *reinterpret_cast<uint2*>(sm.st_lo + vcol * LD + c0) = uint2{pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
      }
    }
  };
  write_state_operand();

  for (int t0 = 0; t0 < T_; t0 += kTok) {
    // ------------------------------------------------------------ prep
    // thread (tp, cq): tokens 2tp, 2tp+1 of the block, channels 4cq .. 4cq+3
    bool overflow = false;
    if (tid < 2 * K) {
      const int tp = tid & 7, c0 = (tid >> 3) * 4;
      float al[2][4], qv[2][4], kv[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = t0 + 2 * tp + j;
        if (t < T_) {
          const long row = (b * T_ + t);
          const float4 g4 = *reinterpret_cast<const float4*>(p.g_raw + (row * HV + hv) * K + c0);
          const float gr[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            al[j][c] = exp_f(gate_log_decay(gr[c], bias ? bias[c0 + c] : 0.0f, rate, p.kind,
                                            p.lower_bound));
          In<T>::load4(qg, (row * H + h) * K + c0, qv[j]);
          In<T>::load4(kg, (row * H + h) * K + c0, kv[j]);
        } else {  // padding past the end: no decay, no write, no read
#pragma unroll
          for (int c = 0; c < 4; ++c) al[j][c] = 1.0f, qv[j][c] = 0.0f, kv[j][c] = 0.0f;
        }
      }
      float E0[4], E1[4], S0f[4], S1f[4], gam[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // inclusive product over the pairs of lanes 0..tp (8-lane segment)
        const float pair = al[0][c] * al[1][c];
        float x = pair;
#pragma unroll
        for (int d = 1; d < 8; d <<= 1) {
          const float y = __shfl_up(x, d, 8);
          if (tp >= d) x *= y;
        }
        float ex = __shfl_up(x, 1, 8);
        if (tp == 0) ex = 1.0f;
        E0[c] = ex * al[0][c];
        E1[c] = x;
        gam[c] = __shfl(x, 7, 8);
        // product over the pairs of lanes tp..7, then exclusive of lane tp
        float z = pair;
#pragma unroll
        for (int d = 1; d < 8; d <<= 1) {
          const float y = __shfl_down(z, d, 8);
          if (tp + d < 8) z *= y;
        }
        float sx = __shfl_down(z, 1, 8);
        if (tp == 7) sx = 1.0f;
        S1f[c] = sx;
        S0f[c] = al[1][c] * sx;
        overflow |= !(gam[c] >= kGammaMin && gam[c] <= kGammaMax);
      }
      float ig[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ig[c] = __builtin_amdgcn_rcpf(gam[c]);
      if (tp == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) sm.gam[c0 + c] = gam[c];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = 2 * tp + j;
        const float* E = j ? E1 : E0;
        const float* Sf = j ? S1f : S0f;
        float qr[4], qh[4], kr[4], kh[4], ke[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          qh[c] = qv[j][c] * E[c];
          kh[c] = kv[j][c] * E[c];
          qr[c] = qh[c] * ig[c];
          kr[c] = kh[c] * ig[c];
          ke[c] = kv[j][c] * Sf[c];
        }
        if constexpr (F32) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            sm.qr[t * LD + c0 + c] = qr[c];
            sm.qh[t * LD + c0 + c] = qh[c];
            sm.kr[t * LD + c0 + c] = kr[c];
            sm.kh[t * LD + c0 + c] = kh[c];
            sm.ke[t * LD + c0 + c] = ke[c];
            sm.keT[(c0 + c) * 17 + t] = ke[c];
          }
        } else {
          uint16_t h4[4], l4[4];
          auto put = [&](uint16_t* dh, uint16_t* dl, const float* x) {
#pragma unroll
            for (int c = 0; c < 4; ++c) split_bf16(x[c], h4[c], l4[c]);
            *reinterpret_cast<uint2*>(dh + t * LD + c0) = uint2{pack2(h4[0], h4[1]), pack2(h4[2], h4[3])};
            if (dl)
              *reinterpret_cast<uint2*>(dl + t * LD + c0) = uint2{pack2(l4[0], l4[1]), pack2(l4[2], l4[3])};
          };
          put(sm.qr_hi, sm.qr_lo, qr);
          put(sm.qh_hi, sm.qh_lo, qh);
          put(sm.kr_hi, sm.kr_lo, kr);
          put(sm.kh_hi, sm.kh_lo, kh);
          put(sm.ke_hi, sm.ke_lo, ke);
#pragma unroll
          for (int c = 0; c < 4; ++c) {  // h4 / l4 hold the split of ke
            sm.keT[(c0 + c) * kCat + t] = h4[c];
            sm.keT[(c0 + c) * kCat + 16 + t] = l4[c];
          }
        }
      }
    }
    if (tid < kTok) sm.beta[tid] = (t0 + tid < T_) ? p.beta[(b * T_ + t0 + tid) * HV + hv] : 0.0f;
    const int fallback = __syncthreads_or(overflow ? 1 : 0);

    if (fallback) {
      // ---------------- token-by-token recurrence for this block (exact, slow)
      for (int tt = 0; tt < kTok && t0 + tt < T_; ++tt) {
        const long row = b * T_ + t0 + tt;
        const float bt = sm.beta[tt];
        float kk[BPW][4], qq[BPW][4];
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          const int blk = w + 4 * i;
          if (blk >= NBLK) continue;
          const int kb = blk / NCB, cb = blk % NCB;
          float part = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * kb + 4 * (lane >> 4) + r;
            const float a = exp_f(gate_log_decay(p.g_raw[(row * HV + hv) * K + c],
                                                 bias ? bias[c] : 0.0f, rate, p.kind, p.lower_bound));
            kk[i][r] = In<T>::at(kg, (row * H + h) * K + c);
            qq[i][r] = In<T>::at(qg, (row * H + h) * K + c);
            sacc[i][r] *= a;
            part += kk[i][r] * sacc[i][r];
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          if (lane < 16) sm.r[kb * BV + 16 * cb + lane] = part;
        }
        __syncthreads();
        float opart[BPW];
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          const int blk = w + 4 * i;
          opart[i] = 0.0f;
          if (blk >= NBLK) continue;
          const int cb = blk % NCB, col = 16 * cb + (lane & 15);
          float pr = 0.0f;
          for (int kb2 = 0; kb2 < NKB; ++kb2) pr += sm.r[kb2 * BV + col];
          const float rr = bt * (In<T>::at(vg, (row * HV + hv) * V + v0 + col) - pr);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sacc[i][r] += kk[i][r] * rr;
            opart[i] += qq[i][r] * sacc[i][r];
          }
          opart[i] += __shfl_xor(opart[i], 16);
          opart[i] += __shfl_xor(opart[i], 32);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
          const int blk = w + 4 * i;
          if (blk >= NBLK) continue;
          const int kb = blk / NCB, cb = blk % NCB;
          if (lane < 16) sm.r[kb * BV + 16 * cb + lane] = opart[i];
        }
        __syncthreads();
        if (tid < BV) {
          float ov = 0.0f;
          for (int kb2 = 0; kb2 < NKB; ++kb2) ov += sm.r[kb2 * BV + tid];
          p.o[(row * HV + hv) * V + v0 + tid] = scale * ov;
        }
        __syncthreads();
      }
      write_state_operand();
      __syncthreads();
      continue;
    }

    // ------------------------------------------------- B: A, R, K_hat S, Q_hat S
    f32x4 qs = {0.f, 0.f, 0.f, 0.f};
    const int cbw = w - 2;  // value column block of waves 2, 3
    if (w == 0) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) mma_f32<K>(acc, sm.qr, LD, sm.ke, LD, lane);
      else mma_kappa_bf16<K, 3>(acc, sm.qr_hi, sm.qr_lo, sm.ke_hi, sm.ke_lo, LD, lane);
      const int j = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (lane >> 4) + r;
        const float a = j <= i ? scale * acc[r] : 0.0f;
        if constexpr (F32) {
          sm.aqk[i * 17 + j] = a;
        } else {
          uint16_t hi, lo;
          split_bf16(a, hi, lo);
          sm.aqk[i * kCat + j] = hi;
          sm.aqk[i * kCat + 16 + j] = lo;
        }
      }
    } else if (w == 1) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) mma_f32<K>(acc, sm.kr, LD, sm.ke, LD, lane);
      else mma_kappa_bf16<K, 3>(acc, sm.kr_hi, sm.kr_lo, sm.ke_hi, sm.ke_lo, LD, lane);
      const int j = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * (lane >> 4) + r;
        sm.r[i * 17 + j] = j < i ? sm.beta[i] * acc[r] : 0.0f;
      }
    } else if (cbw < NCB) {
      f32x4 pk = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) {
        mma_f32<K>(pk, sm.kh, LD, sm.st + cbw * 16 * LD, LD, lane);
        mma_f32<K>(qs, sm.qh, LD, sm.st + cbw * 16 * LD, LD, lane);
      } else {
        mma_kappa_bf16<K, 3>(pk, sm.kh_hi, sm.kh_lo, sm.st_hi + cbw * 16 * LD,
                             sm.st_lo + cbw * 16 * LD, LD, lane);
        mma_kappa_bf16<K, 3>(qs, sm.qh_hi, sm.qh_lo, sm.st_hi + cbw * 16 * LD,
                             sm.st_lo + cbw * 16 * LD, LD, lane);
      }
      const int vcol = 16 * cbw + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (lane >> 4) + r;
        const float vv = (t0 + t < T_) ? In<T>::at(vg, ((b * T_ + t0 + t) * HV + hv) * V + v0 + vcol) : 0.0f;
        const float e = sm.beta[t] * (vv - pk[r]);
        if constexpr (F32) {
          sm.ebT[vcol * 17 + t] = e;
        } else {
          uint16_t hi, lo;
          split_bf16(e, hi, lo);
          sm.ebT[vcol * kCat + t] = hi;
          sm.ebT[vcol * kCat + 16 + t] = lo;
        }
      }
    }
    __syncthreads();

    // ------------------------------------------- B2: (I + R)^{-1}, fp32 substitution
    if (w == 1 && lane < 16) {
      const int c = lane;
      float X[kTok];
#pragma unroll
      for (int i = 0; i < kTok; ++i) {
        float s = (i == c) ? 1.0f : 0.0f;
#pragma unroll
        for (int m = 0; m < i; ++m) s -= sm.r[i * 17 + m] * X[m];
        X[i] = s;
      }
#pragma unroll
      for (int i = 0; i < kTok; ++i) {
        if constexpr (F32) {
          sm.akk[i * 17 + c] = X[i];
        } else {
          uint16_t hi, lo;
          split_bf16(X[i], hi, lo);
          sm.akk[i * kCat + c] = hi;
          sm.akk[i * kCat + 16 + c] = lo;
        }
      }
    }
    __syncthreads();

    // ------------------------------------------------------- C: U = (I+R)^-1 Ebar
    if (w >= 2 && cbw < NCB) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) mma_f32<kTok>(u, sm.akk, 17, sm.ebT + cbw * 16 * 17, 17, lane);
      else mma_tok_bf16(u, sm.akk, sm.ebT + cbw * 16 * kCat, lane);
      const int vcol = 16 * cbw + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (lane >> 4) + r;
        if constexpr (F32) {
          sm.uT[vcol * 17 + t] = u[r];
        } else {
          uint16_t hi, lo;
          split_bf16(u[r], hi, lo);
          sm.uT[vcol * kCat + t] = hi;
          sm.uT[vcol * kCat + 16 + t] = lo;
        }
      }
    }
    __syncthreads();

    // ------------------------------------------- D: outputs and the state update
    if (w >= 2 && cbw < NCB) {
      f32x4 ov = qs * scale;
      if constexpr (F32) mma_f32<kTok>(ov, sm.aqk, 17, sm.uT + cbw * 16 * 17, 17, lane);
      else mma_tok_bf16(ov, sm.aqk, sm.uT + cbw * 16 * kCat, lane);
      const int vcol = 16 * cbw + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (lane >> 4) + r;
        if (t0 + t < T_) p.o[((b * T_ + t0 + t) * HV + hv) * V + v0 + vcol] = ov[r];
      }
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = w + 4 * i;
      if (blk >= NBLK) continue;
      const int kb = blk / NCB, cb = blk % NCB;
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sacc[i][r] * sm.gam[16 * kb + 4 * (lane >> 4) + r];
      if constexpr (F32) mma_f32<kTok>(acc, sm.keT + 16 * kb * 17, 17, sm.uT + cb * 16 * 17, 17, lane);
      else mma_tok_bf16(acc, sm.keT + 16 * kb * kCat, sm.uT + cb * 16 * kCat, lane);
      sacc[i] = acc;
    }
    write_state_operand();
    __syncthreads();
  }

  if (p.S_out) {
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int blk = w + 4 * i;
      if (blk >= NBLK) continue;
      const int kb = blk / NCB, cb = blk % NCB;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * kb + 4 * (lane >> 4) + r;
        p.S_out[((long)hd * K + c) * V + v0 + 16 * cb + (lane & 15)] = sacc[i][r];
      }
    }
  }
}

template <int K, typename T>
static hipError_t launch_chunk_kt(const ChunkParams& p, hipStream_t stream) {
  constexpr int BV = K < 32 ? K : 32;
  constexpr int NVT = K / BV;
  using Smem = typename std::conditional<std::is_same<T, float>::value, SmemF32<K, BV>,
                                         SmemBF16<K, BV>>::type;
  // More than half of the CU's 160 KiB of LDS per workgroup keeps one
  // workgroup per CU, so the B*HV*NVT workgroups spread over all CUs.
  size_t lds = sizeof(Smem);
  if (lds < 84 * 1024) lds = 84 * 1024;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<K, T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nheads = p.B * p.HV;
  const long blocks = (long)((nheads + 7) / 8) * 8 * NVT;
  hipLaunchKernelGGL((chunk_fwd_kernel<K, T>), dim3((unsigned)blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        float lower_bound, const float* S0, float* o, float* S_out, int B, int T,
                        int H, int HV, int K, hipStream_t stream) {
  ChunkParams p{q, k, v, g_raw, beta, A_log, dt_bias, S0, o, S_out, B, T, H, HV, kind, lower_bound};
#define KDA_CHUNK_CASE(KK)                                                  \
  if (K == KK)                                                              \
    return bf16 ? launch_chunk_kt<KK, uint16_t>(p, stream)                  \
                : launch_chunk_kt<KK, float>(p, stream);
  KDA_CHUNK_CASE(16) KDA_CHUNK_CASE(32) KDA_CHUNK_CASE(64) KDA_CHUNK_CASE(128)
#undef KDA_CHUNK_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
