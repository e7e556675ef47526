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
constexpr int kRS = 20;      // row stride of the fp32 R tile (16-byte rows, conflict-free stores)
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
  uint16_t uT[4][kTok * kCat];                  // U^T per wave, own column block [v][hi t | lo t]
  float r[kTok * kRS > (K / 16) * BV ? kTok * kRS : (K / 16) * BV];
  float gam[K];
  float beta[kTok];
  int flag[4];
};

template <int K, int BV>
struct SmemF32 {
  static constexpr int LD = K + 1;
  float qr[kTok * LD], qh[kTok * LD], kr[kTok * LD], kh[kTok * LD], ke[kTok * LD];
  float keT[K * 17];  // [c][t]
  float st[BV * LD];  // [v][c]
  float aqk[kTok * 17], akk[kTok * 17];
  float ebT[BV * 17], uT[4][kTok * 17];
  float r[kTok * kRS > (K / 16) * BV ? kTok * kRS : (K / 16) * BV];
  float gam[K];
  float beta[kTok];
  int flag[4];
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

template <int K, typename T, int GK>
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
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  const float* bias = (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias + (long)hv * K : nullptr;
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

  // ---- inputs of the next block, prefetched into registers one block ahead
  typedef typename In<T>::Raw4 Raw4;
  typedef typename In<T>::Raw1 Raw1;
  const int tp = tid & 7, c0 = (tid >> 3) * 4;  // prep thread: token pair, channel quad
  const int cbw = w - 2;                        // waves 2.. own value column block cbw
  const bool prep_thread = tid < 2 * K;
  const bool ebar_wave = w >= 2 && cbw < NCB;
  float bias4[4] = {0.f, 0.f, 0.f, 0.f};  // dt_bias of the prep thread's channels
  if (bias && prep_thread) {
#pragma unroll
    for (int c = 0; c < 4; ++c) bias4[c] = bias[c0 + c];
  }
  float4 pg[2];
  Raw4 pq[2], pk[2];
  Raw1 pv[4];
  float pbeta = 0.0f;
  // Loads past the end of the sequence read the last token instead (always a
  // valid address) and are replaced by padding values where they are used.
  auto fetch = [&](int tb) {
    if (prep_thread) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = min(tb + 2 * tp + j, T_ - 1);
        const long row = b * T_ + t;
        pg[j] = *reinterpret_cast<const float4*>(p.g_raw + (row * HV + hv) * K + c0);
        pq[j] = In<T>::raw4(qg, (row * H + h) * K + c0);
        pk[j] = In<T>::raw4(kg, (row * H + h) * K + c0);
      }
    }
    if (tid < kTok) {
      const float bt = p.beta[(b * T_ + min(tb + tid, T_ - 1)) * HV + hv];
      pbeta = tb + tid < T_ ? bt : 0.0f;
    }
  };
  auto fetch_v = [&](int tb) {
    if (ebar_wave) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tb + 4 * (lane >> 4) + r;
        const Raw1 x = vg[((b * T_ + min(t, T_ - 1)) * HV + hv) * V + v0 + 16 * cbw + (lane & 15)];
        pv[r] = t < T_ ? x : In<T>::zero1();
      }
    }
  };
  if (T_ > 0) {
    fetch(0);
    fetch_v(0);
  }

  for (int t0 = 0; t0 < T_; t0 += kTok) {
    // ------------------------------------------------------------ prep
    // thread (tp, cq): tokens 2tp, 2tp+1 of the block, channels c0 .. c0+3
    bool overflow = false;
    if (prep_thread) {
      float al[2][4], qv[2][4], kv[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool valid = t0 + 2 * tp + j < T_;  // padding: no decay, no write, no read
        const float gr[4] = {pg[j].x, pg[j].y, pg[j].z, pg[j].w};
        In<T>::unpack4(pq[j], qv[j]);
        In<T>::unpack4(pk[j], kv[j]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float a = exp_f(gate_log_decay_k<GK>(gr[c], bias4[c], rate, p.lower_bound));
          al[j][c] = valid ? a : 1.0f;
          qv[j][c] = valid ? qv[j][c] : 0.0f;
          kv[j][c] = valid ? kv[j][c] : 0.0f;
        }
      }
      float E0[4], E1[4], S0f[4], S1f[4], ig[4];
      uint16_t ke_h0[4], ke_l0[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // prefix products over the token pairs of an 8-lane segment (DPP row shifts)
        const float pair = al[0][c] * al[1][c];
        float x = pair, y;
        y = row_shr<1>(x); if (tp >= 1) x *= y;
        y = row_shr<2>(x); if (tp >= 2) x *= y;
        y = row_shr<4>(x); if (tp >= 4) x *= y;
        float ex = row_shr<1>(x);
        if (tp == 0) ex = 1.0f;
        E0[c] = ex * al[0][c];
        E1[c] = x;
        // suffix products, exclusive of the lane's own pair
        float z = pair;
        y = row_shl<1>(z); if (tp < 7) z *= y;
        y = row_shl<2>(z); if (tp < 6) z *= y;
        y = row_shl<4>(z); if (tp < 4) z *= y;
        float sx = row_shl<1>(z);
        if (tp == 7) sx = 1.0f;
        S1f[c] = sx;
        S0f[c] = al[1][c] * sx;
        const float gam = x * sx;  // decay over the whole block
        overflow |= !(gam >= kGammaMin && gam <= kGammaMax);
        ig[c] = __builtin_amdgcn_rcpf(gam);
        if (tp == 0) sm.gam[c0 + c] = gam;
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
          auto put = [&](uint16_t* dh, uint16_t* dl, const float* x, uint16_t* h4, uint16_t* l4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) split_bf16(x[c], h4[c], l4[c]);
            *reinterpret_cast<uint2*>(dh + t * LD + c0) = uint2{pack2(h4[0], h4[1]), pack2(h4[2], h4[3])};
            *reinterpret_cast<uint2*>(dl + t * LD + c0) = uint2{pack2(l4[0], l4[1]), pack2(l4[2], l4[3])};
          };
          uint16_t h4[4], l4[4];
          put(sm.qr_hi, sm.qr_lo, qr, h4, l4);
          put(sm.qh_hi, sm.qh_lo, qh, h4, l4);
          put(sm.kr_hi, sm.kr_lo, kr, h4, l4);
          put(sm.kh_hi, sm.kh_lo, kh, h4, l4);
          put(sm.ke_hi, sm.ke_lo, ke, h4, l4);
          // (k Suf)^T: the lane's two tokens are adjacent, one 32-bit store per channel
          if (j == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) ke_h0[c] = h4[c], ke_l0[c] = l4[c];
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              *reinterpret_cast<uint32_t*>(sm.keT + (c0 + c) * kCat + t - 1) = pack2(ke_h0[c], h4[c]);
              *reinterpret_cast<uint32_t*>(sm.keT + (c0 + c) * kCat + 16 + t - 1) = pack2(ke_l0[c], l4[c]);
            }
          }
        }
      }
    }
    if (tid < kTok) sm.beta[tid] = pbeta;
    const bool ov_wave = __any(overflow);
    if (lane == 0) sm.flag[w] = ov_wave ? 1 : 0;
    if (t0 + kTok < T_) fetch(t0 + kTok);  // next block's inputs travel while this one computes
    __syncthreads();
    const int fallback = sm.flag[0] | sm.flag[1] | sm.flag[2] | sm.flag[3];

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
            const float a = exp_f(gate_log_decay_k<GK>(p.g_raw[(row * HV + hv) * K + c],
                                                       bias ? bias[c] : 0.0f, rate, p.lower_bound));
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
      if (t0 + kTok < T_) fetch_v(t0 + kTok);
      write_state_operand();
      __syncthreads();
      continue;
    }

    // -------------------------------------------------------------- B
    // wave 0: A;  wave 1: R, then (I + R)^{-1};  waves 2..: K_hat S, Q_hat S, Ebar
    f32x4 qs = {0.f, 0.f, 0.f, 0.f};
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
        sm.r[i * kRS + j] = j < i ? sm.beta[i] * acc[r] : 0.0f;
      }
      // The same wave reads R back: LDS requests of one wave complete in
      // order; the fences keep the compiler from reordering around them.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < 16) {
        // (I + R)^{-1}, column c = lane, by forward substitution in fp32:
        // X[i] = delta_ic - sum_{m<i} R[i][m] X[m], four partial sums per row
        const int c = lane;
        // all 40 row segments of the strict lower triangle are read up front
        // (broadcast reads), so LDS latency is paid once, not per row
        float4 Rr[40];
        {
          int n = 0;
#pragma unroll
          for (int i = 1; i < kTok; ++i)
#pragma unroll
            for (int m4 = 0; m4 < i; m4 += 4) Rr[n++] = *reinterpret_cast<const float4*>(&sm.r[i * kRS + m4]);
        }
        float X[kTok];
        int n = 0;
#pragma unroll
        for (int i = 0; i < kTok; ++i) {
          float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m4 = 0; m4 < i; m4 += 4) {
            const float4 rr = Rr[n++];
            const float rv[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (m4 + u < i) part[u] += rv[u] * X[m4 + u];
          }
          X[i] = ((i == c) ? 1.0f : 0.0f) - ((part[0] + part[1]) + (part[2] + part[3]));
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
    } else if (ebar_wave) {
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
        const float e = sm.beta[t] * (In<T>::widen(pv[r]) - pk[r]);
        if constexpr (F32) {
          sm.ebT[vcol * 17 + t] = e;
        } else {
          uint16_t hi, lo;
          split_bf16(e, hi, lo);
          sm.ebT[vcol * kCat + t] = hi;
          sm.ebT[vcol * kCat + 16 + t] = lo;
        }
      }
      if (t0 + kTok < T_) fetch_v(t0 + kTok);
    }
    __syncthreads();

    // -------------------------------------------------------------- D
    // Every wave owns one value column block (cb = w % NCB): it resolves
    // U = (I + R)^{-1} Ebar for that block itself (a private copy, so no
    // further barrier), then waves 2.. form the outputs and every wave updates
    // its own state blocks.
    const int cbo = w % NCB;
    {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) mma_f32<kTok>(u, sm.akk, 17, sm.ebT + cbo * 16 * 17, 17, lane);
      else mma_tok_bf16(u, sm.akk, sm.ebT + cbo * 16 * kCat, lane);
      const int vl = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (lane >> 4) + r;
        if constexpr (F32) {
          sm.uT[w][vl * 17 + t] = u[r];
        } else {
          uint16_t hi, lo;
          split_bf16(u[r], hi, lo);
          sm.uT[w][vl * kCat + t] = hi;
          sm.uT[w][vl * kCat + 16 + t] = lo;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (ebar_wave) {
      f32x4 ov = qs * scale;
      if constexpr (F32) mma_f32<kTok>(ov, sm.aqk, 17, sm.uT[w], 17, lane);
      else mma_tok_bf16(ov, sm.aqk, sm.uT[w], lane);
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
      const int kb = blk / NCB;
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = sacc[i][r] * sm.gam[16 * kb + 4 * (lane >> 4) + r];
      if constexpr (F32) mma_f32<kTok>(acc, sm.keT + 16 * kb * 17, 17, sm.uT[w], 17, lane);
      else mma_tok_bf16(acc, sm.keT + 16 * kb * kCat, sm.uT[w], lane);
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

template <int K, typename T, int GK>
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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<K, T, GK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int nheads = p.B * p.HV;
  const long blocks = (long)((nheads + 7) / 8) * 8 * NVT;
  hipLaunchKernelGGL((chunk_fwd_kernel<K, T, GK>), dim3((unsigned)blocks), dim3(256), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        float lower_bound, const float* S0, float* o, float* S_out, int B, int T,
                        int H, int HV, int K, hipStream_t stream) {
  ChunkParams p{q, k, v, g_raw, beta, A_log, dt_bias, S0, o, S_out, B, T, H, HV, kind, lower_bound};
#define KDA_CHUNK_GATE(KK, TT)                                                   \
  switch (kind) {                                                                \
    case KDA_GATE_SAFE: return launch_chunk_kt<KK, TT, KDA_GATE_SAFE>(p, stream);         \
    case KDA_GATE_STANDARD: return launch_chunk_kt<KK, TT, KDA_GATE_STANDARD>(p, stream); \
    default: return launch_chunk_kt<KK, TT, KDA_GATE_NONE>(p, stream);                    \
  }
#define KDA_CHUNK_CASE(KK)                                  \
  if (K == KK) {                                            \
    if (bf16) { KDA_CHUNK_GATE(KK, uint16_t) }              \
    else { KDA_CHUNK_GATE(KK, float) }                      \
  }
  KDA_CHUNK_CASE(16) KDA_CHUNK_CASE(32) KDA_CHUNK_CASE(64) KDA_CHUNK_CASE(128)
#undef KDA_CHUNK_CASE
#undef KDA_CHUNK_GATE
  return hipErrorInvalidValue;
}

}  // namespace kda
