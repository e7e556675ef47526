// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // round to nearest even
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  __bf16 h = static_cast<__bf16>(x);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = f32_to_bf16_bits(x - static_cast<float>(h));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The same split for two values at once, packed: hi = the bf16 pair of x0, x1
// (round to nearest even) and lo = the bf16 pair of the remainders x - hi.
// The remainders come from v_dot2c_f32_bf16 as x + hi . m with m = (-1, 0)
// or (0, -1): the products are exact and x - hi is representable, so the one
// rounding of the dot product is exact.  The masks live in scalar registers
// behind an empty asm, which keeps the compiler from encoding (-1, 0) as the
// inline constant -1.0 (the hardware reads that constant as the f32 bit
// pattern 0xbf800000, i.e. the pair (0, -1)).
__device__ __forceinline__ void split2_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  uint32_t m0 = 0x0000bf80u, m1 = 0xbf800000u;
  asm("" : "+s"(m0), "+s"(m1));
  const bf16x2 h = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
  const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m0), x0, false);
  const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1), x1, false);
  const bf16x2 l = {static_cast<__bf16>(l0), static_cast<__bf16>(l1)};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// log(1 + e) for e in [0, 1]; a short series where 1 + e would round.
__device__ __forceinline__ float log1p_small(float e) {
  if (e < 0.0009765625f) return e * (1.0f - e * (0.5f - e * (1.0f / 3.0f)));
  return __builtin_amdgcn_logf(1.0f + e) * kLn2;
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log(1 + e^-|x|); NaN propagates
// through e, and softplus(+inf) = +inf.
__device__ __forceinline__ float softplus_f(float x) {
  float e = exp_f(-fabsf(x));
  return fmaxf(x, 0.0f) + log1p_small(e);
}

// Gate activation: log-decay g for one element ("K3 notes", "Gate 激活").
//   safe     : g = L * sigmoid(rate * (g_raw + bias))
//   standard : g = -rate * softplus(g_raw + bias)
//   none     : g = g_raw
__device__ __forceinline__ float gate_log_decay(float graw, float bias, float rate, int kind,
                                                float L) {
  if (kind == KDA_GATE_SAFE) {
    float z = rate * (graw + bias);
    float e = __builtin_amdgcn_exp2f(-z * kLog2e);  // +inf for very negative z -> sigmoid 0
    return L * __builtin_amdgcn_rcpf(1.0f + e);
  }
  if (kind == KDA_GATE_STANDARD) return -rate * softplus_f(graw + bias);
  return graw;
}

// DPP lane shifts inside rows of 16 lanes (lanes whose source falls outside
// the row keep 0); VALU-speed alternatives to LDS-routed shuffles.
template <int N>
__device__ __forceinline__ float row_shr(float x) {  // lane p reads lane p - N
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x110 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float row_shl(float x) {  // lane p reads lane p + N
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x100 + N, 0xF, 0xF, false));
}

// x + x[lane ^ M] in every lane.  For M = 16 and 32 this uses the gfx950 row
// swaps (VALU, no LDS round trip): v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second, and
// v_permlane32_swap the upper half of the first with the lower half of the
// second, so with x in both operands the two results add up to x plus its
// partner in every lane.  They are written in asm because the compiler at hand
// reads both results of the builtin from one register.  The nop gives the two
// wait states the compiler itself places between a VALU write and the swap.
template <int M>
__device__ __forceinline__ float xor_sum(float x) {
  if constexpr (M == 16 || M == 32) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    if constexpr (M == 16)
      asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    else
      asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
  } else {
    return x + __shfl_xor(x, M);
  }
}

// The same gate with its kind fixed at compile time (no branch per element).
template <int GK>
__device__ __forceinline__ float gate_log_decay_k(float graw, float bias, float rate, float L) {
  if constexpr (GK == KDA_GATE_SAFE) {
    const float z = rate * (graw + bias);
    return L * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
  } else if constexpr (GK == KDA_GATE_STANDARD) {
    return -rate * softplus_f(graw + bias);
  } else {
    return graw;
  }
}

// Retain factor alpha = exp(g) of the same gate, with the per-head constants
// folded into cr = -rate log2(e) and cl = L log2(e):
//   safe     : alpha = 2^(cl / (1 + 2^(cr (g_raw + bias))))
//   standard : alpha = 2^(cr softplus(g_raw + bias))
//   none     : alpha = 2^(g_raw log2(e))
struct GateConsts {
  float cr, cl;
};
__device__ __forceinline__ GateConsts gate_consts(float rate, float L) {
  return GateConsts{-rate * kLog2e, L * kLog2e};
}
template <int GK>
__device__ __forceinline__ float gate_alpha(float graw, float bias, GateConsts gc) {
  if constexpr (GK == KDA_GATE_SAFE) {
    return __builtin_amdgcn_exp2f(
        gc.cl * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(gc.cr * (graw + bias))));
  } else if constexpr (GK == KDA_GATE_STANDARD) {
    return __builtin_amdgcn_exp2f(gc.cr * softplus_f(graw + bias));
  } else {
    return __builtin_amdgcn_exp2f(graw * kLog2e);
  }
}

// gate_alpha with the bias pre-folded: pass gate_bias_pre<GK>(bias, gc) as
// `pre`, so the safe gate's argument cr (g_raw + bias) is one fma.
template <int GK>
__device__ __forceinline__ float gate_bias_pre(float bias, GateConsts gc) {
  return GK == KDA_GATE_SAFE ? gc.cr * bias : bias;
}
template <int GK>
__device__ __forceinline__ float gate_alpha_pre(float graw, float pre, GateConsts gc) {
  if constexpr (GK == KDA_GATE_SAFE) {
    return __builtin_amdgcn_exp2f(
        gc.cl * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(graw, gc.cr, pre))));
  } else {
    return gate_alpha<GK>(graw, pre, gc);
  }
}

// ------------------------------------------------------------ load helpers

template <typename T>
struct In;  // element type of q / k / v

template <>
struct In<float> {
  typedef float4 Raw4;  // four elements as loaded, before widening
  typedef float Raw1;
  static __device__ __forceinline__ Raw4 raw4(const float* p, long i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  static __device__ __forceinline__ void unpack4(Raw4 v, float out[4]) {
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  static __device__ __forceinline__ float widen(Raw1 v) { return v; }
  static __device__ __forceinline__ Raw1 zero1() { return 0.0f; }
  static __device__ __forceinline__ float at(const float* p, long i) { return p[i]; }
  // four consecutive elements
  static __device__ __forceinline__ void load4(const float* p, long i, float out[4]) {
    float4 v = *reinterpret_cast<const float4*>(p + i);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};

template <>
struct In<uint16_t> {  // bfloat16 bits
  typedef uint2 Raw4;
  typedef uint16_t Raw1;
  static __device__ __forceinline__ Raw4 raw4(const uint16_t* p, long i) {
    return *reinterpret_cast<const uint2*>(p + i);
  }
  static __device__ __forceinline__ void unpack4(Raw4 v, float out[4]) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  static __device__ __forceinline__ float widen(Raw1 v) { return bf16_bits_to_f32(v); }
  static __device__ __forceinline__ Raw1 zero1() { return 0; }
  static __device__ __forceinline__ float at(const uint16_t* p, long i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void load4(const uint16_t* p, long i, float out[4]) {
    uint2 v = *reinterpret_cast<const uint2*>(p + i);
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xffff0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

}  // namespace kda
