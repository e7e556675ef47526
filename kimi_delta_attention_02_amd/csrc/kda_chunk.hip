// Chunkwise KDA forward: gate, intra-chunk triangular solve and inter-chunk
// state propagation fused in one kernel.
//
// Algebra (the "DeltaNet family" page, section "Chunkwise KDA", written in the
// K x V state layout of the "K3 notes").  For a block of n = 16 tokens entering
// with state S, with E_i = prod_{m<=i} alpha_m (alpha = exp(g), per key
// channel), gamma = E_{n-1} and Suf_j = prod_{m>j} alpha_m = gamma / E_j:
//
//   temporary errors   Ebar_i = beta_i (v_i - (k_i * E_i) . S)
//   coupling           R_ij   = beta_i sum_c (k_ic E_ic) (k_jc / E_jc)    (j < i)
//   resolved errors    U      = (I + R)^{-1} Ebar        (causal triangular solve)
//   outputs            O_i    = s (q_i * E_i) . S + sum_{j<=i} A_ij U_j,
//                      A_ij   = s sum_c (q_ic E_ic) (k_jc / E_jc)         (j <= i)
//   block-end state    S'     = diag(gamma) S + (k * Suf)^T U
//
// with s = 1/sqrt(K).  Every factor is bounded: for the safe and standard
// gates (log-decay g <= 0) E and Suf lie in [gamma, 1] and k / E in [|k|,
// |k| / gamma], finite as long as gamma >= 2^-100 in every channel (69 nats
// of decay inside 16 tokens; the safe gate with lower bound -5 stays under 80
// nats, and real data far less).  With a caller-supplied log-decay of either
// sign (gate none) gamma, E and Suf are each held to [2^-100, 2^100].  A block
// that breaks a bound is run token by token instead (the recurrence itself, no
// factorisation), so every input is handled exactly.  Across blocks the state
// carries the coupling between earlier and later tokens, which makes the
// 16-token blocks the diagonal blocks of the chunk's triangular system.
//
// Schedule.  One workgroup owns one (sequence b, value head hv, 32-wide value
// tile); the four value tiles of a head share blockIdx % 8 and so an XCD (and
// its L2, which serves their common q, k, g_raw reads).  Its eight wavefronts
// form a four-stage pipeline over 16-token blocks, one barrier per step; each
// role runs its own loop over the NT + 3 steps:
//   waves 0-3  prep of block n+3: gate, cumulative products, scaled operands
//              (hi/lo words) and the block's v tile into a triple-buffered LDS
//              slot, with the next block's HBM inputs loaded a step ahead
//   wave 4     A^T of block n+2 (kept in registers) and O = s Q_hat S + A U of
//              block n with Q_hat S and U handed over by the chain, then the
//              o stores (K not a multiple of 32: it forms s Q_hat S of block
//              n+1 itself from the chain's LDS copy of the state)
//   wave 5     R of block n+2 (MFMA), then (I + R)^{-1} = X_d - X_d N X_d
//              (X_d: the two 8x8 diagonal inverses by substitution, N: the
//              lower-left 8x8 block of R), on fp32 MFMA
//   waves 6-7  the state chain of block n+1, one 16-wide value column block
//              each, with that column block of the fp32 state held in
//              registers for the whole sequence: diag(gamma) S, K_hat S and
//              Q_hat S (from the hi/lo state in its registers), Ebar, U and the
//              state update; Q_hat S and U go to wave 4 (K not a multiple of
//              32: K_hat S against a hi/lo copy of the state in a
//              double-buffered LDS slot, which wave 4 also reads)
// Issue priority: the chain waves win their SIMD's arbitration from K_hat S
// to U and yield it for the state update and its split, which only the next
// step needs; wave 4 wins it over the prep wave on its SIMD.
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
  // checkpoint mode (the backward's forward pass; no o): the state entering
  // every 16-token block, [B, HV, NC, K / 4, V, 4] (each state by key quads:
  // keys 4 i .. 4 i + 3 of every column together), and
  // U = beta r of every block, [B, HV, NC, V / 16, 64, 4] (per 16-wide column
  // block, lane l of 64 holding rows 4 (l / 16) .. + 3 of column l % 16)
  float* ckpt;
  float* u_out;
  // checkpoint mode, also: the backward's value-independent operands of every
  // block, written by the workgroup of the head's first value tile:
  //   eseg   [B, HV, NC, 16, K]  E = prod_{m <= t} alpha_m from the block start
  //                              (row-major; past the end it stays at the last token's)
  //   ops    [B, HV, NC, 3, 64, 4]: lane (c, g) = (l % 16, l / 16), entry r, of
  //            0: P[c][4 g + r] if 4 g + r < c, else 0, P = (k E)(k / E)^T
  //            1: s ((q E)(k / E)^T)[4 g + r][c] if 4 g + r >= c, else 0 (A^T)
  //            2: (I + R)^{-1}[4 g + r][c], R = diag(beta) strictly-lower[P]
  //   segbad [B, HV, NC]  nonzero where the block runs token by token (its
  //                        ops are then not written)
  float* eseg;
  float* ops;
  int* segbad;
  int B, T, H, HV, kind;
  int G;  // value heads per XCD group (a divisor of HV / H)
  float lower_bound;
  // checkpoint mode, also: the backward's summed gradients, zeroed here so
  // that no separate launch has to (each may be null): dq, dk [B, T, H, K],
  // dbeta [B, T, HV], dg [B, T, HV, K] ([B, T, HV] with a per-head gate),
  // dA_log [HV], ddt_bias [HV, K] ([HV] per head).  The workgroup of each
  // head's first value tile zeroes its rows, that of the first value head of
  // a query/key group the dq and dk rows.
  float *zdq, *zdk, *zdb, *zdg, *zdA, *zddt;
};

constexpr int kTok = 16;      // tokens per block
constexpr int kCat = 40;      // row stride of [hi t0..15 | lo t0..15] operands (+8 pad)
constexpr int kRS = 20;       // row stride of the fp32 R tile (16-byte rows, conflict-free stores)
constexpr int kThreads = 512;  // eight wavefronts
constexpr int kPrepWaves = 4, kAqkWave = 4, kInvWave = 5, kChainWave0 = 6;
constexpr float kGammaMin = 7.888609052210118e-31f;  // 2^-100
constexpr float kGammaMax = 1.2676506002282294e30f;  // 2^100 (only a positive log-decay can get here)

// A decay factor the factorised block form can use as it is (NaN fails).
__device__ __forceinline__ bool in_bounds(float x) { return x >= kGammaMin && x <= kGammaMax; }

// ------------------------------------------------------------------ LDS
// ROWS x K operand with the key axis contiguous (bf16: hi and lo words).
// bf16 rows with K a multiple of 32 are unpadded and swizzled: the 16-byte
// chunk j of row r (key channels 8j .. 8j+7) sits at chunk position
// j ^ (r mod K/8).  An MFMA operand read (lane l: row l % 16, one chunk) then
// spreads every group of lanes that the LDS serves together over distinct
// banks, and the prep's row writes keep their cost; padded rows of 272 bytes
// cost half as much again per read.  Rows must start at multiples of 16.
template <bool F32, int ROWS, int K>
struct alignas(16) RowOp;
template <int ROWS, int K>
struct alignas(16) RowOp<false, ROWS, K> {
  static constexpr bool kSwz = K % 32 == 0;
  static constexpr int LD = kSwz ? K : K + 8;
  uint16_t hi[ROWS * LD], lo[ROWS * LD];
};

// position in its row of key channel c (c % 4 == 0: four channels stay together)
// Position of the four keys c .. c+3 (c a multiple of 4) in a bf16 operand
// row: inside each 32-key slice, key e goes to 8 ((e mod 16) / 4) + 4 (e / 16)
// + e mod 4, so that an MFMA lane's eight positions 8 g .. 8 g + 7 hold keys
// 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3, the rows a 16 x 16 accumulator
// fragment pair gives that lane.  Products over the keys do not depend on the
// order, since both operands of each use it.
template <int K>
__device__ __forceinline__ int key_pos(int c) {
  if constexpr (K % 32 == 0) return (c & ~31) | (((c & 15) >> 2) << 3) | (((c >> 4) & 1) << 2);
  else return c;
}

template <int K>
__device__ __forceinline__ int row_pos(int r, int c) {
  if constexpr (K % 32 == 0)
    return (((c >> 3) ^ (r & (K / 8 - 1))) << 3) | (c & 7);
  else
    return c;
}
template <int ROWS, int K>
struct alignas(16) RowOp<true, ROWS, K> {
  static constexpr int LD = K + 1;
  float f[ROWS * LD];
};

// ROWS x 16-token operand with the token axis contiguous: bf16 rows are
// [hi t0..15 | lo t0..15].
template <bool F32, int ROWS>
struct alignas(16) TokOp;
template <int ROWS>
struct alignas(16) TokOp<false, ROWS> {
  uint16_t c[ROWS * kCat];
};
template <int ROWS>
struct alignas(16) TokOp<true, ROWS> {
  float c[ROWS * 17 + 3];
};

// Operands of one 16-token block, written by the prep stage.
template <bool F32, int K, int BV>
struct alignas(16) BlockOps {
  RowOp<F32, kTok, K> qh, kh, ki;  // q E, k E, k / E  (rows = tokens)
  TokOp<F32, K> keT;               // (k Suf)^T        (rows = key channels)
  float gam[K];                    // gamma per key channel
  float beta[kTok];
  int flag[4];                     // per prep wave: a channel broke the gamma bound
  alignas(16) typename std::conditional<F32, float, uint16_t>::type vT[BV][kTok];  // v tile, [column][t]
};

// Per chain wave: scratch of the fp32-input path (Ebar^T, U^T  [v][t]).
template <bool F32>
struct ChainScratch {
  TokOp<true, 16> eb, u;
};
template <>
struct ChainScratch<false> {};

// bf16 inputs: U of one column block handed from the chain to the output
// wave, per lane the hi and lo words of its four accumulator-layout values.
template <bool F32, int NCB>
struct UHandoff {
  uint4 u[NCB][2][64];   // U hi/lo: [column block][block parity][lane]
  f32x4 qs[NCB][2][64];  // Q_hat S of the block (K a multiple of 32), likewise
};
template <int NCB>
struct UHandoff<true, NCB> {};

template <bool F32, int K, int BV>
struct alignas(16) Smem {
  BlockOps<F32, K, BV> blk[3];
  TokOp<F32, kTok> akk[2];           // (I + R)^{-1} of the next two blocks
  TokOp<F32, kTok> aqk[F32 ? 2 : 1];  // A (fp32 inputs; bf16 keeps it in registers)
  alignas(16) float r[kTok * kRS];
  alignas(16) float xd[kTok * kRS];  // inverse of I + R's diagonal 8 x 8 blocks (zero elsewhere)
  alignas(16) float pt[kTok * kRS];
  struct alignas(16) Chain {
    RowOp<F32, 16, K> st[2];         // S^T of its column block [v][c], by block parity
    ChainScratch<F32> f;
  } chain[BV / 16];
  UHandoff<F32, BV / 16> uo;
  // checkpoint mode: the unscaled coupling P of the last two blocks (masked
  // strictly lower), handed from the inverse wave to the A wave
  alignas(16) float pl[F32 ? 2 : 1][F32 ? kTok * kRS : 4];
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
#pragma unroll
    for (int s = 0; s < K; s += 32) {
      const int o = row * ld + row_pos<K>(row, s + (lane >> 4) * 8);  // swizzled rows
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ah + o);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Bh + o);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
      if constexpr (HL == 3) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(Al + o);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Bl + o);
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

// Retain factor exp(g) for the token-by-token path, kept out of line: that
// rare path then does not raise the register allocation of the main one.
// The prep's retain factor alpha = exp(g) from g_raw and the per-head
// constants, with the bias pre-folded by prep_bias_pre.  Safe and none: the
// shared gate formulas.  Standard (g = -rate softplus(x)): in base 2,
// alpha = 2^(-rate l), l = log2(1 + 2^y) = max(y, 0) + log2(1 + 2^-|y|),
// y = x log2(e).  The log of a number in (1, 2] is exact to fp32 rounding in
// absolute terms, and alpha's relative error is the absolute error of its
// exponent, so this is as accurate as the log1p form (~3e-6 relative at
// worst over x in N(-4, 3), rate 4, both ways) in five VALU instructions and
// three transcendentals instead of eleven and three.  NaN propagates through
// the log term; x = +inf gives alpha = 0, x = -inf alpha = 1.
template <int GK>
__device__ __forceinline__ float prep_bias_pre(float bias, GateConsts gc) {
  return GK == KDA_GATE_STANDARD ? bias * kLog2e : gate_bias_pre<GK>(bias, gc);
}
template <int GK>
__device__ __forceinline__ float prep_alpha(float graw, float pre, GateConsts gc, float nrate) {
  if constexpr (GK == KDA_GATE_STANDARD) {
    const float y = __builtin_fmaf(graw, kLog2e, pre);
    const float l = fmaxf(y, 0.0f) + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(y)));
    return __builtin_amdgcn_exp2f(nrate * l);
  } else {
    return gate_alpha_pre<GK>(graw, pre, gc);
  }
}

template <int GK>
__device__ __noinline__ float slow_path_alpha(float graw, float bias, float rate, float L) {
  return exp_f(gate_log_decay_k<GK>(graw, bias, rate, L));
}

__device__ __forceinline__ void wave_lds_sync() {
  // One wavefront's LDS requests complete in order; the fences keep the
  // compiler from moving its LDS accesses across this point.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// four consecutive key-axis values of one row
template <bool F32, int ROWS, int K>
__device__ __forceinline__ void put4(RowOp<F32, ROWS, K>& op, int row, int c0, const float x[4]) {
  constexpr int LD = RowOp<F32, ROWS, K>::LD;
  if constexpr (F32) {
#pragma unroll
    for (int c = 0; c < 4; ++c) op.f[row * LD + c0 + c] = x[c];
  } else {
    uint2 h, l;
    split2_bf16(x[0], x[1], h.x, l.x);
    split2_bf16(x[2], x[3], h.y, l.y);
    const int o = row * LD + row_pos<K>(row, key_pos<K>(c0));
    *reinterpret_cast<uint2*>(op.hi + o) = h;
    *reinterpret_cast<uint2*>(op.lo + o) = l;
  }
}

// one value at (row, token t)
template <bool F32, int ROWS>
__device__ __forceinline__ void put_tok(TokOp<F32, ROWS>& op, int row, int t, float x) {
  if constexpr (F32) {
    op.c[row * 17 + t] = x;
  } else {
    uint16_t h, l;
    split_bf16(x, h, l);
    op.c[row * kCat + t] = h;
    op.c[row * kCat + 16 + t] = l;
  }
}

// two adjacent tokens t (even) and t + 1 of one row
template <bool F32, int ROWS>
__device__ __forceinline__ void put_tok2(TokOp<F32, ROWS>& op, int row, int t, float x0, float x1) {
  if constexpr (F32) {
    op.c[row * 17 + t] = x0;
    op.c[row * 17 + t + 1] = x1;
  } else {
    uint32_t h, l;
    split2_bf16(x0, x1, h, l);
    *reinterpret_cast<uint32_t*>(op.c + row * kCat + t) = h;
    *reinterpret_cast<uint32_t*>(op.c + row * kCat + 16 + t) = l;
  }
}

// acc += A[arow0 .. +16) x B[brow0 .. +16)^T over the key axis
template <bool F32, int K, int RA, int RB>
__device__ __forceinline__ void kprod(f32x4& acc, const RowOp<F32, RA, K>& A, int arow0,
                                      const RowOp<F32, RB, K>& B, int brow0, int lane) {
  constexpr int LD = RowOp<F32, RA, K>::LD;
  if constexpr (F32)
    mma_f32<K>(acc, A.f + arow0 * LD, LD, B.f + brow0 * LD, LD, lane);
  else
    mma_kappa_bf16<K, 3>(acc, A.hi + arow0 * LD, A.lo + arow0 * LD, B.hi + brow0 * LD,
                         B.lo + brow0 * LD, LD, lane);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 16x16x16 bf16 MFMA: the B operand layout (lane l holds k = 4 (l/16) .. +3 of
// column l % 16) equals the accumulator layout, so a product's result can feed
// the next product over the token axis straight from registers.
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split4(const float x[4], bf16x4& hi, bf16x4& lo) {
  uint2 h, l;
  split2_bf16(x[0], x[1], h.x, l.x);
  split2_bf16(x[2], x[3], h.y, l.y);
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, l);
}

// acc += A (16 x 16 tokens, rows [hi | lo] at `row`) * B (accumulator layout,
// given as hi and lo words): hi*hi + hi*lo + lo*hi.
__device__ __forceinline__ void tprod_reg(f32x4& acc, const uint16_t* Acat, bf16x4 bh, bf16x4 bl,
                                          int lane) {
  const uint16_t* a = Acat + (lane & 15) * kCat + 4 * (lane >> 4);
  const bf16x4 ah = *reinterpret_cast<const bf16x4*>(a);
  const bf16x4 al = *reinterpret_cast<const bf16x4*>(a + 16);
  acc = mfma16(ah, bh, acc);
  acc = mfma16(ah, bl, acc);
  acc = mfma16(al, bh, acc);
}

// fp32 inputs: acc1 += A1 x B^T and acc2 += A2 x B^T over the key axis
template <int K, int RB>
__device__ __forceinline__ void kprod2(f32x4& acc1, f32x4& acc2, const RowOp<true, kTok, K>& A1,
                                       const RowOp<true, kTok, K>& A2, const RowOp<true, RB, K>& B,
                                       int lane) {
  kprod(acc1, A1, 0, B, 0, lane);
  kprod(acc2, A2, 0, B, 0, lane);
}

// acc += A[arow0 .. +16) (16 tokens) x B (16 tokens x 16, given by its columns)
template <bool F32, int RA, int RB>
__device__ __forceinline__ void tprod(f32x4& acc, const TokOp<F32, RA>& A, int arow0,
                                      const TokOp<F32, RB>& B, int lane) {
  if constexpr (F32)
    mma_f32<kTok>(acc, A.c + arow0 * 17, 17, B.c, 17, lane);
  else
    mma_tok_bf16(acc, A.c + arow0 * kCat, B.c, lane);
}

// raw buffer loads of four q / k elements and of a thread's v values
template <typename T>
__device__ __forceinline__ typename In<T>::Raw4 buffer_load_raw4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (std::is_same<T, float>::value)
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  else
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <typename VR>
__device__ __forceinline__ VR buffer_load_v(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(VR) == 2)
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  else if constexpr (sizeof(VR) == 4)
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  else
    return __builtin_bit_cast(VR, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// One level of the products over the token pairs of a 16-lane row (lanes
// 2 tp + parity hold token pair tp of two channel groups): each prefix value
// x[c] takes the product with the value SH lanes below, each suffix value
// z[c] with the value SH lanes above (SH = 2, 4, 8: one, two, four pairs).  A lane whose partner falls outside its
// row is not written by the DPP instruction and keeps its value, so no lane
// select is needed.  The s_nop gives the two wait states a DPP read of a VGPR
// needs after a VALU write of it.
#define KDA_PAIR_SCAN(SH, NCH_)                                                                  \
  if constexpr (NCH_ == 4) {                                                                     \
    asm("s_nop 1\n\t"                                                                            \
        "v_mul_f32_dpp %0, %0, %0 row_shr:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %1, %1, %1 row_shr:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %2, %2, %2 row_shr:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %3, %3, %3 row_shr:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %4, %4, %4 row_shl:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %5, %5, %5 row_shl:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %6, %6, %6 row_shl:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %7, %7, %7 row_shl:" #SH " row_mask:0xf bank_mask:0xf"                    \
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(z[0]), "+v"(z[1]), "+v"(z[2]),    \
          "+v"(z[3]));                                                                           \
  } else {                                                                                       \
    asm("s_nop 1\n\t"                                                                            \
        "v_mul_f32_dpp %0, %0, %0 row_shr:" #SH " row_mask:0xf bank_mask:0xf\n\t"                \
        "v_mul_f32_dpp %1, %1, %1 row_shl:" #SH " row_mask:0xf bank_mask:0xf"                    \
        : "+v"(x[0]), "+v"(z[0]));                                                               \
  }

// ----------------------------------------------------------------- kernel

// GS: per-head gate (g_raw [B, T, HV], dt_bias [HV]), one decay shared by all
// key channels, so the prep computes one gate and one product scan per token
// pair instead of four.
template <int K, typename T, int GK, bool GS, bool CK>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(ChunkParams p) {
  // F32: every product on fp32 MFMA (fp32 inputs, and checkpoint mode, whose
  // states feed the backward's fp32 arithmetic); otherwise hi/lo bf16 operands
  constexpr bool F32IN = std::is_same<T, float>::value;
  constexpr bool F32 = F32IN || CK;
  constexpr int V = K;
  constexpr int BV = V < 32 ? V : 32;
  constexpr int NCB = BV / 16, NKB = K / 16, NVT = V / BV;
  // bf16 with K a multiple of 32: the chain forms Q_hat S beside K_hat S from
  // the hi/lo state in its registers and hands it to the A wave, so no copy
  // of the state goes through LDS
  constexpr bool kChainQS = !F32 && K % 32 == 0;
  using SM = Smem<F32, K, BV>;
  using Ops = BlockOps<F32, K, BV>;
  typedef typename In<T>::Raw4 Raw4;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T_ = p.T, HV = p.HV, H = p.H;
  const int NT = (T_ + kTok - 1) / kTok;

  // workgroup -> (head, value tile).  blockIdx % 8 picks the XCD (workgroups
  // are dispatched to the eight XCDs in turn); the NVT tiles of a head, and
  // the p.G value heads of one query/key group, share it and so its L2.
  const int nheads = p.B * HV;
  const int x8 = blockIdx.x & 7, y8 = blockIdx.x >> 3;
  const int m8 = y8 / NVT, vt = y8 % NVT;
  const int hd = ((m8 / p.G) * 8 + x8) * p.G + m8 % p.G;
  if (hd >= nheads) return;
  const long b = hd / HV;
  const int hv = hd % HV;
  const int h = hv / (HV / H);
  const int v0 = vt * BV;
  const float scale = 1.0f / __builtin_sqrtf((float)K);
  const float rate = GK != KDA_GATE_NONE ? exp_f(p.A_log[hv]) : 1.0f;
  constexpr int GKD = GS ? 1 : K;  // gate elements per (token, value head)
  const float* bias = (p.dt_bias && GK != KDA_GATE_NONE) ? p.dt_bias + (long)hv * GKD : nullptr;
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);

  // Each role runs its own loop over the pipeline steps; every loop executes
  // the same NT + 3 barriers, and registers are allocated per role.
  if (w < kPrepWaves) {
    // ---- prep threads: token pair tp (tokens 2tp, 2tp+1), key channels c0 .. c0+3;
    // a 16-lane row holds the eight token pairs of two channel groups, interleaved
    const bool prep_thread = tid < 2 * K;
    // v of the workgroup's value tile, spread over all prep threads:
    // thread -> token vtt, columns vc .. vc + VPT - 1
    constexpr int VPT = kTok * BV / (64 * kPrepWaves);
    static_assert(VPT == 1 || VPT == 2, "value tile / prep thread split");
    typedef typename std::conditional<VPT * sizeof(T) == 2, uint16_t,
            typename std::conditional<VPT * sizeof(T) == 4, uint32_t, uint2>::type>::type VRaw;
    const int vtt = tid / (BV / VPT), vc = (tid % (BV / VPT)) * VPT;
    const int tp = (tid >> 1) & 7, c0 = ((tid >> 4) * 2 + (tid & 1)) * 4;
    float bias4[4] = {0.f, 0.f, 0.f, 0.f};
    if (bias && prep_thread) {
  #pragma unroll
      for (int c = 0; c < 4; ++c) bias4[c] = bias[GS ? 0 : c0 + c];
    }
    const GateConsts gc = gate_consts(rate, p.lower_bound);
  #pragma unroll
    for (int c = 0; c < 4; ++c) bias4[c] = prep_bias_pre<GK>(bias4[c], gc);
    const float nrate = -rate;
    // One block's inputs as loaded.  Two sets alternate between the steps of
    // the loop below (unrolled by two), so the loads of block n + 1 land in
    // the set not being read for block n and nothing is copied between them.
    struct PrepIn {
      float4 g[2];
      Raw4 q[2], k[2];
      VRaw v;
      float beta;
    };
    // Token rows of this sequence and head; a block's rows sit at fixed
    // per-thread byte offsets from a block base that is uniform over the
    // workgroup, so a full block's loads need no per-step address arithmetic.
    const long gs = (long)HV * GKD, qs = (long)H * K, vs = (long)HV * V;
    const float* g_seq = p.g_raw + (b * T_ * HV + hv) * (long)GKD;
    const T* q_seq = qg + (b * T_ * H + h) * (long)K;
    const T* k_seq = kg + (b * T_ * H + h) * (long)K;
    const T* v_seq = vg + (b * T_ * HV + hv) * (long)V + v0;
    const float* beta_seq = p.beta + b * T_ * HV + hv;
    // threads without a row (K < 128) take an offset beyond every range, so
    // their loads return zero without touching memory
    constexpr uint32_t kNoRow = 0x80000000u;
    uint32_t og[2], oq[2];
  #pragma unroll
    for (int j = 0; j < 2; ++j) {
      og[j] = prep_thread ? (uint32_t)(((2 * tp + j) * gs + (GS ? 0 : c0)) * sizeof(float)) : kNoRow;
      oq[j] = prep_thread ? (uint32_t)(((2 * tp + j) * qs + c0) * sizeof(T)) : kNoRow;
    }
    const uint32_t ov = (uint32_t)((vtt * vs + vc) * sizeof(T));
    // threads 16 and up repeat the beta of tokens 0..15
    const uint32_t ob = (uint32_t)((tid & (kTok - 1)) * HV * sizeof(float));
    // A block's rows are read as raw buffer loads: a descriptor on the block
    // base (scalar registers, formed per step) plus each thread's fixed 32-bit
    // byte offset, so no address is formed in vector registers.  The
    // descriptor's range ends at the sequence's last token, so rows past the
    // end of a ragged last block read as zero (and are replaced by padding
    // values where they are used).  Every load is unconditional: results
    // merged from two paths would be copied, and each copy waits for every
    // load in flight, the next block's included.
    auto rsrc = [](const void* base, uint32_t bytes) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                               0x00020000);
    };
    auto fetch = [&](int blk, PrepIn& in) {
      // a block past the end gets an empty range: its loads touch no memory
      // (the clamp is read back as a scalar: the descriptor must be uniform)
      const int rows_i = __builtin_amdgcn_readfirstlane(max(0, min(kTok, T_ - blk * kTok)));
      const int tb = rows_i > 0 ? blk * kTok : 0;
      const uint32_t rows = (uint32_t)rows_i;
      const auto rg = rsrc(g_seq + tb * gs, rows * (uint32_t)(gs * sizeof(float)));
      const auto rq = rsrc(q_seq + tb * qs, rows * (uint32_t)(qs * sizeof(T)));
      const auto rk = rsrc(k_seq + tb * qs, rows * (uint32_t)(qs * sizeof(T)));
      const auto rv = rsrc(v_seq + tb * vs, rows * (uint32_t)(vs * sizeof(T)));
      const auto rb = rsrc(beta_seq + (long)tb * HV, rows * (uint32_t)(HV * sizeof(float)));
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (GS) {
          const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, og[j], 0, 0));
          in.g[j] = float4{x, x, x, x};
        } else {
          in.g[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, og[j], 0, 0));
        }
        in.q[j] = buffer_load_raw4<T>(rq, oq[j]);
        in.k[j] = buffer_load_raw4<T>(rk, oq[j]);
      }
      in.v = buffer_load_v<VRaw>(rv, ov);
      in.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, ob, 0, 0));
    };
    PrepIn in0, in1;
    fetch(0, in0);
    // one pipeline step: prep of block it from `cur`, loads of block it + 1 into `nxt`
    auto step = [&](int it, const PrepIn& cur, PrepIn& nxt) {
      fetch(it + 1, nxt);  // the next block's inputs travel during this step
      if (it < NT) {
        // the slot as one scalar, so that each LDS address is one add to it
        Ops& B = sm.blk[__builtin_amdgcn_readfirstlane(it % 3)];
        bool overflow = false;
        // Full blocks (all but possibly the last) skip the padding selects.
        auto prep_block = [&](auto full) {
          constexpr bool kFull = decltype(full)::value;
          const int t0 = it * kTok;
          const float4* g_in = cur.g;
          const Raw4 *q_in = cur.q, *k_in = cur.k;
          constexpr int NCH = GS ? 1 : 4;  // distinct decays among the four channels
          float al[2][4], qv[2][4], kv[2][4];
  #pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bool valid = kFull || t0 + 2 * tp + j < T_;  // padding: no decay, no write, no read
            const float gr[4] = {g_in[j].x, g_in[j].y, g_in[j].z, g_in[j].w};
            In<T>::unpack4(q_in[j], qv[j]);
            In<T>::unpack4(k_in[j], kv[j]);
  #pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float a = c < NCH ? prep_alpha<GK>(gr[c], bias4[c], gc, nrate) : al[j][0];
              al[j][c] = valid ? a : 1.0f;
              qv[j][c] = valid ? qv[j][c] : 0.0f;
              kv[j][c] = valid ? kv[j][c] : 0.0f;
            }
          }
          // Products over the token pairs of a 16-lane row by DPP row shifts,
          // each level applied to the four channels together: inclusive prefix
          // x and suffix z of the pair products.
          float x[4], z[4];
  #pragma unroll
          for (int c = 0; c < NCH; ++c) x[c] = z[c] = al[0][c] * al[1][c];
          KDA_PAIR_SCAN(2, NCH)
          KDA_PAIR_SCAN(4, NCH)
          KDA_PAIR_SCAN(8, NCH)
          float E[2][4], Sf[2][4], ig[4], gam[4];
  #pragma unroll
          for (int c = 0; c < NCH; ++c) {
            // exclusive prefix and suffix: the lanes of the row's first and last
            // token pair have no partner and read 1
            const float ex = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, x[c]), 0x112, 0xF, 0xF, false));
            const float sx = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, z[c]), 0x102, 0xF, 0xF, false));
            E[0][c] = ex * al[0][c];
            E[1][c] = x[c];
            Sf[1][c] = sx;
            Sf[0][c] = al[1][c] * sx;
            gam[c] = x[c] * sx;  // decay over the whole block
            // the safe and standard gates give g <= 0, so E, Suf in [gamma, 1]: gamma
            // bounds them all; NaN fails too
            overflow |= !(gam[c] >= kGammaMin);
            if constexpr (GK == KDA_GATE_NONE)  // any sign: every factor on its own
              overflow |= !(gam[c] <= kGammaMax) | !in_bounds(E[0][c]) | !in_bounds(E[1][c]) |
                          !in_bounds(Sf[0][c]) | !in_bounds(Sf[1][c]);
            ig[c] = __builtin_amdgcn_rcpf(gam[c]);
          }
  #pragma unroll
          for (int c = NCH; c < 4; ++c) {  // per-head gate: the other channels share channel 0's
            E[0][c] = E[0][0];
            E[1][c] = E[1][0];
            Sf[0][c] = Sf[0][0];
            Sf[1][c] = Sf[1][0];
            gam[c] = gam[0];
            ig[c] = ig[0];
          }
          if (tp == 0) *reinterpret_cast<float4*>(&B.gam[c0]) = float4{gam[0], gam[1], gam[2], gam[3]};
          if constexpr (CK) {  // the head's first value tile hands E to the backward
            if (v0 == 0) {
              float* eb = p.eseg + ((long)hd * NT + it) * (kTok * K) + c0;
  #pragma unroll
              for (int j = 0; j < 2; ++j)
                *reinterpret_cast<float4*>(eb + (2 * tp + j) * K) = float4{E[j][0], E[j][1], E[j][2], E[j][3]};
              // and zeroes the gradient rows of its tokens and channels
              const float4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
              for (int j = 0; j < 2; ++j) {
                const long t = t0 + 2 * tp + j;
                if (t < T_) {
                  if (!GS && p.zdg) *reinterpret_cast<float4*>(p.zdg + ((b * T_ + t) * HV + hv) * (long)K + c0) = z4;
                  if (hv % (HV / H) == 0) {
                    const long qo = ((b * T_ + t) * H + h) * (long)K + c0;
                    if (p.zdq) *reinterpret_cast<float4*>(p.zdq + qo) = z4;
                    if (p.zdk) *reinterpret_cast<float4*>(p.zdk + qo) = z4;
                  }
                }
              }
            }
          }
          float ke[2][4];
  #pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int t = 2 * tp + j;
            float qh[4], kh[4], ki[4];
  #pragma unroll
            for (int c = 0; c < 4; ++c) {
              qh[c] = qv[j][c] * E[j][c];
              kh[c] = kv[j][c] * E[j][c];
              ke[j][c] = kv[j][c] * Sf[j][c];
              ki[c] = ke[j][c] * ig[c];  // k / E = k Suf / gamma
            }
            put4(B.qh, t, c0, qh);
            put4(B.kh, t, c0, kh);
            put4(B.ki, t, c0, ki);
          }
  #pragma unroll
          for (int c = 0; c < 4; ++c) put_tok2(B.keT, c0 + c, 2 * tp, ke[0][c], ke[1][c]);
        };
        {  // v tile, transposed for the chain waves (padding rows: 0)
          const VRaw x = it * kTok + vtt < T_ ? cur.v : VRaw{};
          if constexpr (F32IN && VPT == 1) {
            B.vT[vc][vtt] = __uint_as_float(x);
          } else if constexpr (F32IN) {
            B.vT[vc][vtt] = __uint_as_float(x.x);
            B.vT[vc + 1][vtt] = __uint_as_float(x.y);
          } else if constexpr (F32 && VPT == 1) {  // bf16 inputs on the fp32 path: widened
            B.vT[vc][vtt] = bf16_bits_to_f32((uint16_t)x);
          } else if constexpr (F32) {
            B.vT[vc][vtt] = bf16_bits_to_f32((uint16_t)(x & 0xffffu));
            B.vT[vc + 1][vtt] = bf16_bits_to_f32((uint16_t)(x >> 16));
          } else if constexpr (VPT == 1) {
            B.vT[vc][vtt] = x;
          } else {
            B.vT[vc][vtt] = (uint16_t)(x & 0xffffu);
            B.vT[vc + 1][vtt] = (uint16_t)(x >> 16);
          }
          if (tid < kTok) B.beta[tid] = it * kTok + tid < T_ ? cur.beta : 0.0f;
          if constexpr (CK) {  // the backward's per-token gradients, zeroed (see ChunkParams)
            if (v0 == 0 && tid < kTok && it * kTok + tid < T_) {
              const long row = (b * T_ + it * kTok + tid) * HV + hv;
              if (p.zdb) p.zdb[row] = 0.0f;
              if (GS && p.zdg) p.zdg[row] = 0.0f;
            }
            if (v0 == 0 && it == 0) {  // and the per-head sums (every sequence writes the same zeros)
              if (p.zddt && tid < GKD) p.zddt[(long)hv * GKD + tid] = 0.0f;
              if (p.zdA && tid == 0) p.zdA[hv] = 0.0f;
            }
          }
        }
        if (prep_thread) {
          if ((it + 1) * kTok <= T_) prep_block(std::true_type{});
          else prep_block(std::false_type{});
        }
        const bool ov = __any(overflow);
        if (lane == 0) B.flag[w] = ov ? 1 : 0;
      }
      __syncthreads();
    };
    int it = 0;
    for (; it + 1 < NT + 3; it += 2) {
      step(it, in0, in1);
      step(it + 1, in1, in0);
    }
    if (it < NT + 3) step(it, in0, in1);
  } else if (w == kAqkWave || w == kInvWave) {
    // The A wave (A, then the outputs) shares its SIMD with a prep wave that
    // has slack; it takes the issue arbitration, the prep wave absorbs the wait.
    if (w == kAqkWave) __builtin_amdgcn_s_setprio(1);
    // bf16 inputs: the A wave also forms the outputs, one step behind the
    // chain: O = s Q_hat S + A U for the block whose U the chain produced last
    // step.  A is computed as A^T = (k / E)(q E)^T, whose accumulator layout is
    // A's MFMA operand layout, and stays in registers; Q_hat S (formed by the
    // chain when K is a multiple of 32, else here from the chain's LDS copy
    // of the state) and U arrive from the chain through LDS.
    bf16x4 ah_n = {}, al_n = {}, ah_o = {}, al_o = {};  // A of blocks it-2 (n), it-3 (o)
    bool skip_n = true, skip_o = true;  // block absent or run token by token
    f32x4 qsv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) qsv[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (w == kInvWave)  // the off-diagonal blocks of xd stay zero
      for (int e = lane; e < kTok * kRS; e += 64) sm.xd[e] = 0.0f;
    for (int it = 0; it < NT + 3; ++it) {
      const int ti = it - 1;
      if constexpr (!F32 && !CK) {
        if (w == kAqkWave) {
          const int g = lane >> 4;
          if (!skip_o) {  // O of block it - 3
            const int t0 = (it - 3) * kTok;
            float* orow = p.o + ((b * T_ + t0 + 4 * g) * HV + hv) * (long)V + v0 + (lane & 15);
  #pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const uint4 uu = sm.uo.u[cb][(it - 3) & 1][lane];
              const bf16x4 uh = __builtin_bit_cast(bf16x4, uint2{uu.x, uu.y});
              const bf16x4 ul = __builtin_bit_cast(bf16x4, uint2{uu.z, uu.w});
              f32x4 acc = kChainQS ? sm.uo.qs[cb][(it - 3) & 1][lane] * scale : qsv[cb];
              acc = mfma16(ah_o, uh, acc);
              acc = mfma16(ah_o, ul, acc);
              acc = mfma16(al_o, uh, acc);
  #pragma unroll
              for (int r = 0; r < 4; ++r)
                if (t0 + 4 * g + r < T_) orow[(long)r * HV * V + 16 * cb] = acc[r];
            }
          }
          ah_o = ah_n;
          al_o = al_n;
          skip_o = skip_n;
          if (!kChainQS && !skip_o) {  // s Q_hat S of block it - 2 (otherwise the chain's)
            const Ops& B2 = sm.blk[(it - 2) % 3];
  #pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
              kprod(acc, B2.qh, 0, sm.chain[cb].st[(it - 2) & 1], 0, lane);
              qsv[cb] = acc * scale;
            }
          }
          skip_n = true;
          if (ti >= 0 && ti < NT) {  // A of block it - 1
            const Ops& B = sm.blk[ti % 3];
            skip_n = (B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3]) != 0;
            if (!skip_n) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
              kprod(acc, B.ki, 0, B.qh, 0, lane);  // lane l, r: A[l % 16][4 g + r] / s
              float a[4];
  #pragma unroll
              for (int r = 0; r < 4; ++r) a[r] = 4 * g + r <= (lane & 15) ? scale * acc[r] : 0.0f;
              split4(a, ah_n, al_n);
            }
          }
        }
      }
      if (ti >= 0 && ti < NT && (F32 || w == kInvWave)) {
        const Ops& B = sm.blk[ti % 3];
        if (!(B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3])) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const int j = lane & 15;
          if (w == kAqkWave) {
            if constexpr (F32 && !CK) {
              kprod(acc, B.qh, 0, B.ki, 0, lane);
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int i = 4 * (lane >> 4) + r;
                put_tok(sm.aqk[ti & 1], i, j, j <= i ? scale * acc[r] : 0.0f);
              }
            }
          } else {
            kprod(acc, B.kh, 0, B.ki, 0, lane);
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * (lane >> 4) + r;
              sm.r[i * kRS + j] = j < i ? B.beta[i] * acc[r] : 0.0f;
            }
            if constexpr (CK) {  // P itself, for the backward's operands (the A wave writes them)
              if (v0 == 0) {
  #pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const int i = 4 * (lane >> 4) + r;
                  sm.pl[ti & 1][i * kRS + j] = j < i ? acc[r] : 0.0f;
                }
              }
            }
            wave_lds_sync();
            // (I + R)^{-1} in fp32.  With X_d the inverse of I + R's two 8 x 8
            // diagonal blocks and N = R's lower-left 8 x 8 block,
            // (I + R)^{-1} = X_d - X_d N X_d, since (X_d N)^2 = 0.
            {  // X_d by forward substitution, one column c per lane (lanes >= 16 repeat)
              const int c = lane & 15, bo = c & 8;  // bo: first row of c's diagonal block
              float X[8];
  #pragma unroll
              for (int ii = 0; ii < 8; ++ii) {
                const float* rrow = &sm.r[(bo + ii) * kRS + bo];
                float part[2] = {0.f, 0.f};
  #pragma unroll
                for (int m = 0; m < ii; ++m) part[m & 1] += rrow[m] * X[m];
                X[ii] = ((ii == (c & 7)) ? 1.0f : 0.0f) - (part[0] + part[1]);
              }
              if (lane < 16) {
  #pragma unroll
                for (int ii = 0; ii < 8; ++ii) sm.xd[(bo + ii) * kRS + c] = X[ii];
              }
            }
            wave_lds_sync();
            {  // Y = X^T = Y_d - Y_d P, P = N^T Y_d, on the 16x16x4 fp32 MFMA
              const int row = lane & 15, kk = lane >> 4;
              f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
              for (int s4 = 8; s4 < 16; s4 += 4) {  // N^T is zero outside k = 8..15, rows 0..7
                const float a = row < 8 ? sm.r[(s4 + kk) * kRS + row] : 0.0f;
                pacc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sm.xd[row * kRS + s4 + kk], pacc, 0, 0, 0);
              }
              *reinterpret_cast<f32x4*>(&sm.pt[row * kRS + 4 * kk]) = pacc;  // P^T, [column][row]
              wave_lds_sync();
              const float4 yd = *reinterpret_cast<const float4*>(&sm.xd[row * kRS + 4 * kk]);
              f32x4 y = {yd.x, yd.y, yd.z, yd.w};
  #pragma unroll
              for (int s4 = 0; s4 < 8; s4 += 4)  // P is zero outside rows 0..7
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(-sm.xd[(s4 + kk) * kRS + row],
                                                         sm.pt[row * kRS + s4 + kk], y, 0, 0, 0);
              // lane l, r: Y[4 kk + r][row] = X[row][4 kk + r], X's MFMA operand layout
              if constexpr (F32) {
  #pragma unroll
                for (int r = 0; r < 4; ++r) sm.akk[ti & 1].c[row * 17 + 4 * kk + r] = y[r];
              } else {
                const float yy[4] = {y[0], y[1], y[2], y[3]};
                bf16x4 yh, yl;
                split4(yy, yh, yl);
                *reinterpret_cast<bf16x4*>(&sm.akk[ti & 1].c[row * kCat + 4 * kk]) = yh;
                *reinterpret_cast<bf16x4*>(&sm.akk[ti & 1].c[row * kCat + 16 + 4 * kk]) = yl;
              }
            }
          }
        }
      }
      if constexpr (CK) {
        // The A wave of the head's first value tile writes the backward's
        // operands of the chain's block (its E came from the prep, P and the
        // inverse from the inverse wave, one step earlier), and whether the
        // block runs token by token.
        const int tc = it - 2;
        if (w == kAqkWave && v0 == 0 && tc >= 0 && tc < NT) {
          const Ops& B = sm.blk[tc % 3];
          const bool bad = (B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3]) != 0;
          const long blk = (long)hd * NT + tc;
          if (lane == 0) p.segbad[blk] = bad ? 1 : 0;
          if (!bad) {
            const int c = lane & 15, g = lane >> 4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            kprod(acc, B.qh, 0, B.ki, 0, lane);  // lane l, r: ((q E)(k / E)^T)[4 g + r][c]
            float4* ob = reinterpret_cast<float4*>(p.ops + blk * (3 * 64 * 4)) + lane;
            ob[0] = *reinterpret_cast<const float4*>(&sm.pl[tc & 1][c * kRS + 4 * g]);
            float m[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) m[r] = 4 * g + r >= c ? scale * acc[r] : 0.0f;
            ob[64] = float4{m[0], m[1], m[2], m[3]};
            const float* X = sm.akk[tc & 1].c;  // X[i][j] at i * 17 + j
            ob[128] = float4{X[(4 * g) * 17 + c], X[(4 * g + 1) * 17 + c], X[(4 * g + 2) * 17 + c],
                             X[(4 * g + 3) * 17 + c]};
          }
        }
      }
      __syncthreads();
    }
  } else {
    // ---- chain waves: value column block cb, state rows 16 kb + 4 (lane/16) + r
    const int cb = w - kChainWave0;
    // The chain is the pipeline's critical path and shares its SIMD with a
    // VALU-heavy prep wave: its instructions win the issue arbitration.
    __builtin_amdgcn_s_setprio(2);
    const bool chain = cb >= 0 && cb < NCB;
    const int vcol = v0 + 16 * cb + (lane & 15);
    f32x4 sacc[NKB];
    // bf16, K a multiple of 32: the hi/lo words of the state by 32-key slice,
    // kept for the next step's K_hat S.  With the key order that key_pos gives
    // the rows, positions 8 (l/16) .. +7 of slice s hold keys 32 s + 4 (l/16)
    // + 0..3 and 32 s + 16 + 4 (l/16) + 0..3: fragments 2s and 2s+1 as they are.
    constexpr bool kRegB = !F32 && K % 32 == 0;
    constexpr int NSL = kRegB ? K / 32 : 1;
    bf16x8 sh[NSL], sl[NSL];
    auto write_state_operand = [&](RowOp<F32, 16, K>& st) {
      if constexpr (kRegB) {
        const int row = lane & 15;
  #pragma unroll
        for (int q = 0; q < NSL; ++q) {
          uint4 h, l;
          split2_bf16(sacc[2 * q][0], sacc[2 * q][1], h.x, l.x);
          split2_bf16(sacc[2 * q][2], sacc[2 * q][3], h.y, l.y);
          split2_bf16(sacc[2 * q + 1][0], sacc[2 * q + 1][1], h.z, l.z);
          split2_bf16(sacc[2 * q + 1][2], sacc[2 * q + 1][3], h.w, l.w);
          sh[q] = __builtin_bit_cast(bf16x8, h);
          sl[q] = __builtin_bit_cast(bf16x8, l);
          (void)row;
          (void)st;  // the state's only readers are this wave's registers
        }
      } else {
  #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const float x[4] = {sacc[kb][0], sacc[kb][1], sacc[kb][2], sacc[kb][3]};
          put4(st, lane & 15, 16 * kb + 4 * (lane >> 4), x);
        }
      }
    };
    if (chain) {
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * kb + 4 * (lane >> 4) + r;
          sacc[kb][r] = p.S0 ? p.S0[((long)hd * K + c) * V + vcol] : 0.0f;
        }
      }
      write_state_operand(sm.chain[cb].st[0]);
      wave_lds_sync();
    }
    for (int it = 0; it < NT + 3; ++it) {
      __builtin_amdgcn_s_setprio(2);  // the critical part: K_hat S to U
      const int tc = it - 2;
      if (tc >= 0 && tc < NT && chain) {
        const Ops& B = sm.blk[tc % 3];
        typename SM::Chain& C = sm.chain[cb];
        const int t0 = tc * kTok;
        // checkpoint mode: this block's entry state (column vcol, keys
        // 16 kb + 4 (lane / 16) .. + 3), stored by key quads ([K / 4][V][4]:
        // the 16 columns of a row group are 256 contiguous bytes), and where
        // its U goes
        float* ublk = nullptr;
        if constexpr (CK) {
          const long blk = (long)hd * NT + tc;
          float* ck = p.ckpt + blk * K * V + ((lane >> 4) * V + vcol) * 4;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            *reinterpret_cast<float4*>(ck + 16 * kb * V) =
                float4{sacc[kb][0], sacc[kb][1], sacc[kb][2], sacc[kb][3]};
          ublk = p.u_out + ((blk * (V / 16) + vcol / 16) * 64 + lane) * 4;
        }
        if (B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3]) {
          // ---- token-by-token recurrence (exact, slow path); the wave owns all
          // key rows of its columns, so both reductions stay in the wavefront
          for (int tt = 0; tt < kTok && t0 + tt < T_; ++tt) {
            const long row = b * T_ + t0 + tt;
            const float* grow = p.g_raw + (row * HV + hv) * GKD;
            const float a_head = GS ? slow_path_alpha<GK>(grow[0], bias ? bias[0] : 0.0f, rate,
                                                          p.lower_bound) : 0.0f;
            const T* krow = kg + (row * H + h) * K;
            const T* qrow = qg + (row * H + h) * K;
            float part = 0.0f;
  #pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int c = 16 * kb + 4 * (lane >> 4) + r;
                sacc[kb][r] *= GS ? a_head : slow_path_alpha<GK>(grow[c], bias ? bias[c] : 0.0f, rate,
                                                                 p.lower_bound);
                part += In<T>::at(krow, c) * sacc[kb][r];
              }
              // one key block at a time: keeps this rare path's registers bounded
              __builtin_amdgcn_sched_barrier(0);
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            const float rr = p.beta[row * HV + hv] * (In<T>::at(vg, (row * HV + hv) * V + vcol) - part);
            if constexpr (CK)  // U of token tt: row tt of the block, lane (tt / 4) * 16 + column
              if ((lane >> 4) == (tt >> 2)) ublk[tt & 3] = rr;
            float op = 0.0f;
  #pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int c = 16 * kb + 4 * (lane >> 4) + r;
                sacc[kb][r] += In<T>::at(krow, c) * rr;
                op += In<T>::at(qrow, c) * sacc[kb][r];
              }
              __builtin_amdgcn_sched_barrier(0);
            }
            op += __shfl_xor(op, 16);
            op += __shfl_xor(op, 32);
            if (!CK && lane < 16) p.o[(row * HV + hv) * V + vcol] = scale * op;
          }
        } else {
          const int g = lane >> 4;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {  // diag(gamma) S first: needs nothing below
            const float4 gm = *reinterpret_cast<const float4*>(&B.gam[16 * kb + 4 * g]);
            sacc[kb] *= f32x4{gm.x, gm.y, gm.z, gm.w};
          }
          // bf16: the (k Suf)^T operands of the state update, read now so that
          // their LDS latency passes under K_hat S and U
          bf16x4 kth[F32 ? 1 : NKB], ktl[F32 ? 1 : NKB];
          if constexpr (!F32) {
            const uint16_t* a = B.keT.c + (lane & 15) * kCat + 4 * (lane >> 4);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              kth[kb] = *reinterpret_cast<const bf16x4*>(a + 16 * kb * kCat);
              ktl[kb] = *reinterpret_cast<const bf16x4*>(a + 16 * kb * kCat + 16);
            }
          }
          f32x4 pk = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
          if constexpr (F32 && CK)
            kprod(pk, B.kh, 0, C.st[tc & 1], 0, lane);        // K_hat S (no output)
          else if constexpr (F32)
            kprod2(pk, qs, B.kh, B.qh, C.st[tc & 1], lane);  // K_hat S and Q_hat S
          else if constexpr (kRegB) {  // K_hat S, the state from registers
            const int row = lane & 15;
  #pragma unroll
            for (int q = 0; q < NSL; ++q) {
              const int o = row * RowOp<F32, kTok, K>::LD + row_pos<K>(row, 32 * q + 8 * (lane >> 4));
              const bf16x8 ah = *reinterpret_cast<const bf16x8*>(B.kh.hi + o);
              const bf16x8 al = *reinterpret_cast<const bf16x8*>(B.kh.lo + o);
              const bf16x8 qh = *reinterpret_cast<const bf16x8*>(B.qh.hi + o);
              const bf16x8 ql = *reinterpret_cast<const bf16x8*>(B.qh.lo + o);
              pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sh[q], pk, 0, 0, 0);
              qs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, sh[q], qs, 0, 0, 0);
              pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, sl[q], pk, 0, 0, 0);
              qs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, sl[q], qs, 0, 0, 0);
              pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, sh[q], pk, 0, 0, 0);
              qs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, sh[q], qs, 0, 0, 0);
            }
            // Q_hat S goes to the A wave, which forms this block's outputs next step
            if constexpr (!CK) sm.uo.qs[cb][tc & 1][lane] = qs;
          } else
            kprod(pk, B.kh, 0, C.st[tc & 1], 0, lane);        // K_hat S
          const float4 bt4 = *reinterpret_cast<const float4*>(&B.beta[4 * g]);
          float vv[4];  // v of tokens 4g .. 4g+3 in this lane's column (padding: 0)
          if constexpr (F32) {
            const float4 x = *reinterpret_cast<const float4*>(&B.vT[16 * cb + (lane & 15)][4 * g]);
            vv[0] = x.x; vv[1] = x.y; vv[2] = x.z; vv[3] = x.w;
          } else {
            In<T>::unpack4(*reinterpret_cast<const uint2*>(&B.vT[16 * cb + (lane & 15)][4 * g]), vv);
          }
          const float e[4] = {bt4.x * (vv[0] - pk[0]), bt4.y * (vv[1] - pk[1]),
                              bt4.z * (vv[2] - pk[2]), bt4.w * (vv[3] - pk[3])};
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
          if constexpr (F32) {
            f32x4 ov = qs * scale;
#pragma unroll
            for (int r = 0; r < 4; ++r) put_tok(C.f.eb, lane & 15, 4 * g + r, e[r]);
            wave_lds_sync();
            tprod(u, sm.akk[tc & 1], 0, C.f.eb, lane);
            if constexpr (CK) *reinterpret_cast<float4*>(ublk) = float4{u[0], u[1], u[2], u[3]};
#pragma unroll
            for (int r = 0; r < 4; ++r) put_tok(C.f.u, lane & 15, 4 * g + r, u[r]);
            wave_lds_sync();
            if constexpr (!CK) tprod(ov, sm.aqk[tc & 1], 0, C.f.u, lane);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) tprod(sacc[kb], B.keT, 16 * kb, C.f.u, lane);
            if constexpr (!CK) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int t = t0 + 4 * g + r;
                if (t < T_) p.o[((b * T_ + t) * HV + hv) * V + vcol] = ov[r];
              }
            }
          } else {
            // Ebar, U stay in registers: accumulator layout = B operand layout
            bf16x4 eh, el, uh, ul;
            split4(e, eh, el);
            tprod_reg(u, sm.akk[tc & 1].c, eh, el, lane);  // U = (I + R)^{-1} Ebar
            if constexpr (CK) *reinterpret_cast<float4*>(ublk) = float4{u[0], u[1], u[2], u[3]};
            const float uu[4] = {u[0], u[1], u[2], u[3]};
            split4(uu, uh, ul);
            {  // U to the output wave
              const uint2 h2 = __builtin_bit_cast(uint2, uh), l2 = __builtin_bit_cast(uint2, ul);
              sm.uo.u[cb][tc & 1][lane] = uint4{h2.x, h2.y, l2.x, l2.y};
            }
            // The update and split feed only the next step, after the barrier,
            // and the chain has slack: the prep wave on this SIMD issues first.
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {  // S = gamma S + (k Suf)^T U
              sacc[kb] = mfma16(kth[kb], uh, sacc[kb]);
              sacc[kb] = mfma16(kth[kb], ul, sacc[kb]);
              sacc[kb] = mfma16(ktl[kb], uh, sacc[kb]);
            }
          }
        }
        write_state_operand(C.st[(tc + 1) & 1]);
        wave_lds_sync();
      }
      __syncthreads();
    }
    if (chain && p.S_out) {
  #pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * kb + 4 * (lane >> 4) + r;
          p.S_out[((long)hd * K + c) * V + vcol] = sacc[kb][r];
        }
      }
    }
  }
}

template <int K, typename T, int GK, bool GS, bool CK = false>
static hipError_t launch_chunk_kt(const ChunkParams& p, hipStream_t stream) {
  constexpr int BV = K < 32 ? K : 32;
  constexpr int NVT = K / BV;
  using SM = Smem<std::is_same<T, float>::value || CK, K, BV>;  // the kernel's own layout
  // More than half of the CU's 160 KiB of LDS per workgroup keeps one
  // workgroup per CU, so the B*HV*NVT workgroups spread over all CUs.
  size_t lds = sizeof(SM);
  if (lds < 84 * 1024) lds = 84 * 1024;
  // the dynamic LDS limit above 64 KiB is raised on every launch (a host-side
  // attribute of the function: cheap, and it leaves the library stateless)
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_kernel<K, T, GK, GS, CK>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nheads = p.B * p.HV;
  const long blocks = (long)((nheads / p.G + 7) / 8) * 8 * p.G * NVT;
  hipLaunchKernelGGL((chunk_fwd_kernel<K, T, GK, GS, CK>), dim3((unsigned)blocks), dim3(kThreads), lds,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                        const float* beta, const float* A_log, const float* dt_bias, int kind,
                        int per_head, float lower_bound, const float* S0, float* o, float* S_out,
                        int B, int T, int H, int HV, int K, hipStream_t stream) {
  ChunkParams p{q, k, v, g_raw, beta, A_log, dt_bias, S0, o, S_out, nullptr, nullptr, nullptr, nullptr,
                nullptr, B, T, H, HV,
                kind, 1, lower_bound};
  // The value heads of one query/key head share an XCD (and their q, k reads
  // its L2) when that keeps the eight XCDs evenly loaded.
  const int Gq = HV / H;
  p.G = (B * HV / Gq) % 8 == 0 ? Gq : 1;
#define KDA_CHUNK_GS(KK, TT, GG)                                     \
  return per_head ? launch_chunk_kt<KK, TT, GG, true>(p, stream)     \
                  : launch_chunk_kt<KK, TT, GG, false>(p, stream);
#define KDA_CHUNK_GATE(KK, TT)                                      \
  switch (kind) {                                                   \
    case KDA_GATE_SAFE: KDA_CHUNK_GS(KK, TT, KDA_GATE_SAFE)         \
    case KDA_GATE_STANDARD: KDA_CHUNK_GS(KK, TT, KDA_GATE_STANDARD) \
    default: KDA_CHUNK_GS(KK, TT, KDA_GATE_NONE)                    \
  }
#define KDA_CHUNK_CASE(KK)                     \
  if (K == KK) {                               \
    if (bf16) { KDA_CHUNK_GATE(KK, uint16_t) } \
    else { KDA_CHUNK_GATE(KK, float) }         \
  }
  KDA_CHUNK_CASE(16) KDA_CHUNK_CASE(32) KDA_CHUNK_CASE(64) KDA_CHUNK_CASE(128)
#undef KDA_CHUNK_CASE
#undef KDA_CHUNK_GATE
#undef KDA_CHUNK_GS
  return hipErrorInvalidValue;
}

// The forward pass of the backward: the same kernel in checkpoint mode, which
// writes the state entering every 16-token block, U of every block and the
// backward's per-block operands (see ChunkParams) instead of o; K in
// {32, 64, 128}.
hipError_t launch_chunk_ckpt(const void* q, const void* k, const void* v, int bf16, const float* g_raw,
                             const float* beta, const float* A_log, const float* dt_bias, int kind,
                             int per_head, float lower_bound, const float* S0, float* ckpt,
                             float* u_out, float* eseg, float* ops, int* segbad, int B, int T, int H,
                             int HV, int K, float* const zero[6], hipStream_t stream) {
  ChunkParams p{q, k, v, g_raw, beta, A_log, dt_bias, S0, nullptr, nullptr, ckpt, u_out, eseg, ops,
                segbad, B, T, H, HV,
                kind, 1, lower_bound, zero[0], zero[1], zero[2], zero[3], zero[4], zero[5]};
  const int Gq = HV / H;
  p.G = (B * HV / Gq) % 8 == 0 ? Gq : 1;
#define KDA_CKPT_GS(KK, TT, GG)                                            \
  return per_head ? launch_chunk_kt<KK, TT, GG, true, true>(p, stream)     \
                  : launch_chunk_kt<KK, TT, GG, false, true>(p, stream);
#define KDA_CKPT_GATE(KK, TT)                                      \
  switch (kind) {                                                  \
    case KDA_GATE_SAFE: KDA_CKPT_GS(KK, TT, KDA_GATE_SAFE)         \
    case KDA_GATE_STANDARD: KDA_CKPT_GS(KK, TT, KDA_GATE_STANDARD) \
    default: KDA_CKPT_GS(KK, TT, KDA_GATE_NONE)                    \
  }
#define KDA_CKPT_CASE(KK)                     \
  if (K == KK) {                              \
    if (bf16) { KDA_CKPT_GATE(KK, uint16_t) } \
    else { KDA_CKPT_GATE(KK, float) }         \
  }
  KDA_CKPT_CASE(32) KDA_CKPT_CASE(64) KDA_CKPT_CASE(128)
#undef KDA_CKPT_CASE
#undef KDA_CKPT_GATE
#undef KDA_CKPT_GS
  return hipErrorInvalidValue;
}

}  // namespace kda
