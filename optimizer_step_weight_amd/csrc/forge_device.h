// forge_device.h -- device helpers shared by the fused and the unfused kernels:
// the element-wise update rules, stochastic rounding of the weight to bf16,
// the block-64 int8 moment codec, and Philox4x64-10.
//
// FORGE explainer (gist.science), Technical Summary section 2 "Core Mechanism"
// (the optimizer runs on the gradient tile held in registers) and "Precision and
// Fidelity" (fp32 gradient, stochastic rounding of the bf16 weight write-back,
// int8 states in blocks of 64); section 3 "Key Contributions" (the eight rules).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "forge_internal.h"

namespace forge {

// ------------------------------------------------------------------ Philox4x64-10
// Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds
// on a 256-bit counter; each round forms the 128-bit products of words 0 and 2 with
// two odd constants and mixes the halves with words 1, 3 and the key; the key moves
// by two Weyl constants between rounds.
struct U64x4 {
  uint64_t w[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                               uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t lo0 = kM0 * c0, hi0 = __umul64hi(kM0, c0);
    const uint64_t lo1 = kM1 * c2, hi1 = __umul64hi(kM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U64x4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// 16 random bits for element j (0..15) of the 16-element block whose Philox output is `o`:
// field (j & 3) of word j >> 2.
__device__ __forceinline__ uint32_t sr_field(const U64x4& o, int j) {
  return (uint32_t)(o.w[j >> 2] >> (16 * (j & 3))) & 0xFFFFu;
}

// ------------------------------------------------------------------ bf16 conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Stochastic rounding: (bits + r) >> 16 rounds the magnitude up with probability
// (bits mod 2^16) / 2^16; a NaN keeps its sign and becomes quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_sr(float x, uint32_t r16) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t q = (u + r16) >> 16;
  return (x != x) ? ((u >> 16) | 0x40u) : q;
}

// Round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t q = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (x != x) ? ((u >> 16) | 0x40u) : q;
}

// ------------------------------------------------------------------ update rules (fp32)
// One step of rule OPT for one element.  g: full gradient, w: weight before the step,
// m / v: moments before the step (updated in place), returns the new fp32 weight.
// The per-step scalars come from the host (fp64 there, rounded to fp32):
//   decay = 1 - lr*wd for decoupled decay (else 1); l2 = wd for coupled L2 (else 0).
template <int OPT>
__device__ __forceinline__ float rule(float g, float w, float& m, float& v, const OptScalars& s) {
  g = __builtin_fmaf(s.l2, w, g);
  const float wd = w * s.decay;
  if constexpr (OPT == FORGE_OPT_ADAMW) {
    // c1 = lr / (1 - beta1^t), c2 = 1 / (1 - beta2^t)
    m = __builtin_fmaf(s.b1, m, s.omb1 * g);
    v = __builtin_fmaf(s.b2, v, s.omb2 * (g * g));
    const float den = __builtin_amdgcn_sqrtf(v * s.c2) + s.eps;
    return __builtin_fmaf(-s.c1, m * __builtin_amdgcn_rcpf(den), wd);
  } else if constexpr (OPT == FORGE_OPT_NADAM) {
    // c1 = lr (1 - mu_t) / (1 - prod_t), c2 = 1 / (1 - beta2^t), c3 = lr mu_{t+1} / (1 - prod_{t+1})
    m = __builtin_fmaf(s.b1, m, s.omb1 * g);
    v = __builtin_fmaf(s.b2, v, s.omb2 * (g * g));
    const float den = __builtin_amdgcn_sqrtf(v * s.c2) + s.eps;
    const float num = __builtin_fmaf(s.c1, g, s.c3 * m);
    return wd - num * __builtin_amdgcn_rcpf(den);
  } else if constexpr (OPT == FORGE_OPT_RADAM) {
    // rectified: c1 = lr r_t sqrt(1 - beta2^t) / (1 - beta1^t); otherwise c1 = lr / (1 - beta1^t)
    m = __builtin_fmaf(s.b1, m, s.omb1 * g);
    v = __builtin_fmaf(s.b2, v, s.omb2 * (g * g));
    if (s.rect) {
      const float den = __builtin_amdgcn_sqrtf(v) + s.eps;
      return __builtin_fmaf(-s.c1, m * __builtin_amdgcn_rcpf(den), wd);
    }
    return __builtin_fmaf(-s.c1, m, wd);
  } else if constexpr (OPT == FORGE_OPT_LION) {
    const float c = __builtin_fmaf(s.b1, m, s.omb1 * g);
    const float sg = c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
    m = __builtin_fmaf(s.b2, m, s.omb2 * g);
    return __builtin_fmaf(-s.lr, sg, wd);
  } else if constexpr (OPT == FORGE_OPT_RMSPROP) {
    // b2 = alpha, omb2 = 1 - alpha
    v = __builtin_fmaf(s.b2, v, s.omb2 * (g * g));
    const float den = __builtin_amdgcn_sqrtf(v) + s.eps;
    return __builtin_fmaf(-s.lr, g * __builtin_amdgcn_rcpf(den), wd);
  } else if constexpr (OPT == FORGE_OPT_ADAGRAD) {
    v = __builtin_fmaf(g, g, v);
    const float den = __builtin_amdgcn_sqrtf(v) + s.eps;
    return __builtin_fmaf(-s.lr, g * __builtin_amdgcn_rcpf(den), wd);
  } else if constexpr (OPT == FORGE_OPT_SGD) {
    return __builtin_fmaf(-s.lr, g, wd);
  } else {  // SGD with momentum: c1 = momentum
    m = __builtin_fmaf(s.c1, m, g);
    return __builtin_fmaf(-s.lr, m, wd);
  }
}

template <int OPT>
struct RuleStates {
  static constexpr bool m = OPT == FORGE_OPT_ADAMW || OPT == FORGE_OPT_NADAM || OPT == FORGE_OPT_RADAM ||
                            OPT == FORGE_OPT_LION || OPT == FORGE_OPT_SGD_MOMENTUM;
  static constexpr bool v = OPT == FORGE_OPT_ADAMW || OPT == FORGE_OPT_NADAM || OPT == FORGE_OPT_RADAM ||
                            OPT == FORGE_OPT_RMSPROP || OPT == FORGE_OPT_ADAGRAD;
};

// ------------------------------------------------------------------ compile-time loops
// f(std::integral_constant<int, i>) for i = 0 .. N-1.  Register arrays indexed by a loop
// counter stay in registers only if the loop is unrolled; the compiler declines to unroll the
// large epilogue loops (the dynamic 8-bit map makes their bodies long) and would then move such
// arrays to scratch memory, so these loops take their index as a constant.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------------ vector memory helpers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 x) { *reinterpret_cast<u32x4*>(p) = x; }

// ------------------------------------------------------------------ int8 block-64 requantisation
// Two 8-bit maps of a block's values x / s (s = the block absmax), selected per call:
//  * linear: code = nearest-even of x * levels / s, levels 127 (signed, codes -127..127) or
//    255 (unsigned, 0..255);
//  * dynamic (the dynamic tree code of common 8-bit optimizers): a sign bit (signed maps only),
//    then in the B = 7 (signed) or 8 (unsigned) magnitude bits p a run of E zero bits, an
//    indicator bit and F = B - 1 - E fraction bits f; magnitude 10^-E (0.1 + 0.9 (f + 1) / 2^F),
//    i.e. the decade (10^-(E+1), 10^-E] in 2^F equal steps, p = 0 meaning 0.  Encoding takes
//    the nearest magnitude.
// Both: an unsigned (second-moment) value above zero never stores code 0 (otherwise the next
// step's denominator would lose that element's history while its first moment keeps it); a
// block of zeros stores zero codes with scale 0; a block holding a NaN or an infinity stores
// zero codes and a NaN scale, so it dequantises to NaN and stays visible.

// 10^-e for e = 0..7 (fp32)
__device__ __forceinline__ float pow10_neg(int e) {
  float r = 1.0f;
  r = e == 1 ? 1e-1f : r;
  r = e == 2 ? 1e-2f : r;
  r = e == 3 ? 1e-3f : r;
  r = e == 4 ? 1e-4f : r;
  r = e == 5 ? 1e-5f : r;
  r = e == 6 ? 1e-6f : r;
  r = e == 7 ? 1e-7f : r;
  return r;
}
__device__ __forceinline__ float pow10_pos(int e) {
  float r = 1.0f;
  r = e == 1 ? 1e1f : r;
  r = e == 2 ? 1e2f : r;
  r = e == 3 ? 1e3f : r;
  r = e == 4 ? 1e4f : r;
  r = e == 5 ? 1e5f : r;
  r = e == 6 ? 1e6f : r;
  r = e == 7 ? 1e7f : r;
  return r;
}

// Value of dynamic code c relative to the block absmax.
template <bool SIGNED>
__device__ __forceinline__ float dyn_decode(uint32_t c) {
  constexpr int B = SIGNED ? 7 : 8;
  const uint32_t p = c & (SIGNED ? 0x7Fu : 0xFFu);
  const int L = 32 - __builtin_clz(p | 1u);        // bit length of p (1 for p = 0, unused then)
  const int F = L - 1, E = B - L;
  const uint32_t f = p & ((1u << F) - 1u);
  const float mag = p ? pow10_neg(E) * __builtin_fmaf(0.9f * (float)(f + 1u), __builtin_ldexpf(1.0f, -F), 0.1f) : 0.0f;
  return (SIGNED && (c & 0x80u)) ? -mag : mag;
}

// Dynamic code of x given inv = 1 / s: the magnitude pattern p of the nearest magnitude.
template <bool SIGNED>
__device__ __forceinline__ uint32_t dyn_encode(float x, float inv) {
  constexpr int B = SIGNED ? 7 : 8, EMAX = B - 1;
  const float y = fminf(fabsf(x) * inv, 1.0f);
  int E = 0;  // the decade (10^-(E+1), 10^-E] holding y; EMAX for y <= 10^-EMAX
#pragma unroll
  for (int k = 1; k <= EMAX; ++k) E += y <= pow10_neg(k) ? 1 : 0;
  uint32_t p;
  if (E == EMAX) {
    // the only magnitudes left are 10^-EMAX and 0
    p = (y >= 0.5f * pow10_neg(EMAX)) ? 1u : 0u;
    if (!SIGNED && y > 0.0f) p = 1u;
  } else {
    // continuous step index in the decade; -1 is the top of the decade below (10^-(E+1))
    const int F = B - 1 - E;
    const float u = (__builtin_fmaf(y, pow10_pos(E), -0.1f)) * (__builtin_ldexpf(1.0f, F) / 0.9f) - 1.0f;
    const float f = fminf(fmaxf(__builtin_rintf(u), -1.0f), (float)((1 << F) - 1));
    p = (uint32_t)((int)(1 << F) + (int)f);
  }
  return (SIGNED && x < 0.0f && p) ? (p | 0x80u) : p;
}

// The new values x[0..C) of this lane, part of a 64-element block spread over LANES lanes
// (lane ^ 1, 2, ... < LANES; all of them active).  Returns the block scale and the codes.
template <bool SIGNED, bool DYN, int C, int LANES>
__device__ __forceinline__ float quant_block64(const float (&x)[C], uint32_t (&code)[C]) {
  float amax = 0.0f;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const float a = fabsf(x[j]);
    bad |= !(a <= 3.40282347e38f);
    amax = fmaxf(amax, a);
  }
#pragma unroll
  for (int o = 1; o < LANES; o <<= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    bad |= __shfl_xor(bad, o);
  }
  const bool use = !bad && amax > 0.0f;
  if constexpr (DYN) {
    const float inv = use ? 1.0f / amax : 0.0f;
#pragma unroll
    for (int j = 0; j < C; ++j) code[j] = use ? dyn_encode<SIGNED>(x[j], inv) : 0u;
  } else {
    const float inv = use ? (SIGNED ? 127.0f : 255.0f) / amax : 0.0f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float xj = bad ? 0.0f : x[j];
      float q = __builtin_rintf(xj * inv);
      if constexpr (SIGNED) {
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        code[j] = (uint32_t)(int32_t)q & 0xFFu;
      } else {
        q = fminf(fmaxf(q, (xj > 0.0f && inv > 0.0f) ? 1.0f : 0.0f), 255.0f);
        code[j] = (uint32_t)q;
      }
    }
  }
  return bad ? __builtin_nanf("") : amax;
}

// Dequantised value of an 8-bit code of either map.
template <bool SIGNED, bool DYN>
__device__ __forceinline__ float dequant8(uint32_t c, float scale) {
  if constexpr (DYN) return dyn_decode<SIGNED>(c) * scale;
  const float q = SIGNED ? (float)(int8_t)(c & 0xFFu) : (float)(c & 0xFFu);
  return q * (scale * (SIGNED ? (1.0f / 127.0f) : (1.0f / 255.0f)));
}

// ------------------------------------------------------------------ one 16-element segment
// The stored state of 16 consecutive elements, as loaded from memory (raw words).
struct SegIn {
  u32x4 w[4];   // bf16: w[0..1] used; fp32: w[0..3]
  u32x4 m[4];   // fp32: m[0..3]; int8: m[0]
  u32x4 v[4];
  float ms, vs; // int8 block scales
};

template <int OPT, int WT, int ST>
__device__ __forceinline__ void seg_load(SegIn& x, uint32_t i0, const EpiArgs& e) {
  constexpr bool HM = RuleStates<OPT>::m, HV = RuleStates<OPT>::v;
  if constexpr (WT == FORGE_W_BF16) {
    const uint16_t* wp = static_cast<const uint16_t*>(e.W) + i0;
    x.w[0] = ld16(wp);
    x.w[1] = ld16(wp + 8);
  } else {
    const float* wp = static_cast<const float*>(e.W) + i0;
#pragma unroll
    for (int q = 0; q < 4; ++q) x.w[q] = ld16(wp + 4 * q);
  }
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
      const float* mp = static_cast<const float*>(e.m) + i0;
#pragma unroll
      for (int q = 0; q < 4; ++q) x.m[q] = ld16(mp + 4 * q);
    } else {
      x.m[0] = ld16(static_cast<const int8_t*>(e.m) + i0);
      x.ms = e.m_scale[i0 >> 6];
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
      const float* vp = static_cast<const float*>(e.v) + i0;
#pragma unroll
      for (int q = 0; q < 4; ++q) x.v[q] = ld16(vp + 4 * q);
    } else {
      x.v[0] = ld16(static_cast<const uint8_t*>(e.v) + i0);
      x.vs = e.v_scale[i0 >> 6];
    }
  }
}

// Applies rule OPT to 16 consecutive elements of one row of W, starting at flat index i0
// (a multiple of 16).  The weight, moments and scales are read and written here.  For int8
// moments the 64-element block spans the 4 consecutive lanes lane^1, lane^2 (all four must
// be active); the lane holding the block's first segment writes the block scale.
template <int OPT, int WT, int ST>
__device__ __forceinline__ void seg_apply(const float (&g)[16], uint32_t i0, const SegIn& x, const EpiArgs& e) {
  constexpr bool HM = RuleStates<OPT>::m, HV = RuleStates<OPT>::v;
  float w[16], m[16], v[16];
  if constexpr (WT == FORGE_W_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[2 * q] = __uint_as_float(x.w[0][q] << 16);
      w[2 * q + 1] = __uint_as_float(x.w[0][q] & 0xFFFF0000u);
      w[8 + 2 * q] = __uint_as_float(x.w[1][q] << 16);
      w[8 + 2 * q + 1] = __uint_as_float(x.w[1][q] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) w[4 * q + c] = __uint_as_float(x.w[q][c]);
  }
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) m[4 * q + c] = __uint_as_float(x.m[q][c]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) m[4 * q + c] = dequant8<true, ST == FORGE_S_Q8D>(x.m[0][q] >> (8 * c), x.ms);
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * q + c] = __uint_as_float(x.v[q][c]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * q + c] = dequant8<false, ST == FORGE_S_Q8D>(x.v[0][q] >> (8 * c), x.vs);
    }
  }

  // --- the rule, element by element
  float wn[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float mj = HM ? m[j] : 0.0f, vj = HV ? v[j] : 0.0f;
    wn[j] = rule<OPT>(g[j], w[j], mj, vj, e.s);
    m[j] = mj;
    v[j] = vj;
  }

  if (e.w_pre) {
    float* pp = e.w_pre + i0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 a;
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(wn[4 * q + c]);
      st16(pp + 4 * q, a);
    }
  }

  // --- weight write-back
  if constexpr (WT == FORGE_W_BF16) {
    uint32_t r[16];
    if (e.sr) {
      const U64x4 o = philox4x64_10((uint64_t)(i0 >> 4), e.step, 0ull, 0ull, e.seed, 0ull);
#pragma unroll
      for (int j = 0; j < 16; ++j) r[j] = f32_to_bf16_sr(wn[j], sr_field(o, j));
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) r[j] = f32_to_bf16_rne(wn[j]);
    }
    u32x4 a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = r[2 * q] | (r[2 * q + 1] << 16);
      b[q] = r[8 + 2 * q] | (r[8 + 2 * q + 1] << 16);
    }
    uint16_t* wp = static_cast<uint16_t*>(e.W) + i0;
    st16(wp, a);
    st16(wp + 8, b);
  } else {
    float* wp = static_cast<float*>(e.W) + i0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 a;
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(wn[4 * q + c]);
      st16(wp + 4 * q, a);
    }
  }

  // --- moment write-back
  const bool leader = ((i0 >> 4) & 3u) == 0u;
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
      float* mp = static_cast<float*>(e.m) + i0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 a;
#pragma unroll
        for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(m[4 * q + c]);
        st16(mp + 4 * q, a);
      }
    } else {
      uint32_t code[16];
      const float scale = quant_block64<true, ST == FORGE_S_Q8D, 16, 4>(m, code);
      u32x4 a;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a[q] = code[4 * q] | (code[4 * q + 1] << 8) | (code[4 * q + 2] << 16) | (code[4 * q + 3] << 24);
      st16(static_cast<int8_t*>(e.m) + i0, a);
      if (leader) e.m_scale[i0 >> 6] = scale;
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
      float* vp = static_cast<float*>(e.v) + i0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 a;
#pragma unroll
        for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(v[4 * q + c]);
        st16(vp + 4 * q, a);
      }
    } else {
      uint32_t code[16];
      const float scale = quant_block64<false, ST == FORGE_S_Q8D, 16, 4>(v, code);
      u32x4 a;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        a[q] = code[4 * q] | (code[4 * q + 1] << 8) | (code[4 * q + 2] << 16) | (code[4 * q + 3] << 24);
      st16(static_cast<uint8_t*>(e.v) + i0, a);
      if (leader) e.v_scale[i0 >> 6] = scale;
    }
  }
}

// ------------------------------------------------------------------ one 4-element unit
// Lane-contiguous layout of the epilogue: consecutive lanes hold consecutive 4-element units
// of a row, so every load and store of a wave covers contiguous memory (streaming reads and
// writes of the same bytes run ~18 % faster this way than with 64-byte-strided lanes).  The 16
// elements of one stochastic-rounding counter are then the units of the 4 lanes of a quad, and
// a 64-element int8 block the units of 16 consecutive lanes.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 x) { *reinterpret_cast<u32x2*>(p) = x; }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void st4(void* p, uint32_t x) { *reinterpret_cast<uint32_t*>(p) = x; }

struct UnitIn {
  u32x4 w;       // bf16: w.x, w.y hold the 4 weights; fp32: all four
  u32x4 m, v;    // fp32 moments; int8: .x holds the 4 codes
  float ms, vs;  // int8 block scales
};

// Loads the stored state of the unit at flat index i0 (a multiple of 4).
template <int OPT, int WT, int ST>
__device__ __forceinline__ void unit_load(UnitIn& x, uint32_t i0, const EpiArgs& e) {
  constexpr bool HM = RuleStates<OPT>::m, HV = RuleStates<OPT>::v;
  if constexpr (WT == FORGE_W_BF16) {
    const u32x2 a = ld8(static_cast<const uint16_t*>(e.W) + i0);
    x.w.x = a.x;
    x.w.y = a.y;
  } else {
    x.w = ld16(static_cast<const float*>(e.W) + i0);
  }
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
      x.m = ld16(static_cast<const float*>(e.m) + i0);
    } else {
      x.m.x = ld4(static_cast<const int8_t*>(e.m) + i0);
      x.ms = e.m_scale[i0 >> 6];
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
      x.v = ld16(static_cast<const float*>(e.v) + i0);
    } else {
      x.v.x = ld4(static_cast<const uint8_t*>(e.v) + i0);
      x.vs = e.v_scale[i0 >> 6];
    }
  }
}

__device__ __forceinline__ uint64_t pick4(const U64x4& o, int j) {
  const uint64_t a = j == 1 ? o.w[1] : o.w[0];
  const uint64_t b = j == 3 ? o.w[3] : o.w[2];
  return j >= 2 ? b : a;
}

// Stochastic-rounding words of 4 rounds of units.  In round r this lane's unit starts at flat
// index i[r]; the quad's 4 lanes hold the 16 elements of counter i[r] >> 4 (lane u the unit u,
// which takes word u of the Philox block).  Lane u computes the block of round u, then the quad
// exchanges words so that out[r] is word u of round r's block.  All 4 lanes of every quad must
// be active.
__device__ __forceinline__ void sr_words4(const uint32_t (&i)[4], const EpiArgs& e, uint64_t (&out)[4]) {
  const int lane = (int)(threadIdx.x & 63), u = lane & 3, qb = lane & ~3;
  const uint32_t mine = u == 0 ? i[0] : u == 1 ? i[1] : u == 2 ? i[2] : i[3];
  const U64x4 o = philox4x64_10((uint64_t)(mine >> 4), e.step, 0ull, 0ull, e.seed, 0ull);
  // step k: lane s offers word (s - k) mod 4 of its block; lane u reads lane (u + k) mod 4 and
  // so receives word u of round (u + k) mod 4
  auto step = [&](int k) {
    const uint64_t offer = pick4(o, (u - k) & 3);
    const int src = qb + ((u + k) & 3);
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)offer, src);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(offer >> 32), src);
    return (uint64_t)lo | ((uint64_t)hi << 32);
  };
  const uint64_t g0 = step(0), g1 = step(1), g2 = step(2), g3 = step(3);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = (r - u) & 3;  // the step that delivered round r
    out[r] = k == 0 ? g0 : k == 1 ? g1 : k == 2 ? g2 : g3;
  }
}

// Applies rule OPT to the 4 elements of the unit at flat index i0 (a multiple of 4) and writes
// the weight and moments back.  srw: this unit's stochastic-rounding word (field c of it rounds
// element i0 + c).  For int8 moments the 16 lanes lane ^ 1, 2, 4, 8 hold the 64-element block
// and must all be active; the lane of its first unit writes the block scale.
template <int OPT, int WT, int ST>
__device__ __forceinline__ void unit_apply(const float (&g)[4], uint32_t i0, const UnitIn& x, uint64_t srw,
                                           const EpiArgs& e) {
  constexpr bool HM = RuleStates<OPT>::m, HV = RuleStates<OPT>::v;
  float w[4], m[4], v[4];
  if constexpr (WT == FORGE_W_BF16) {
    w[0] = __uint_as_float(x.w.x << 16);
    w[1] = __uint_as_float(x.w.x & 0xFFFF0000u);
    w[2] = __uint_as_float(x.w.y << 16);
    w[3] = __uint_as_float(x.w.y & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = __uint_as_float(x.w[c]);
  }
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
#pragma unroll
      for (int c = 0; c < 4; ++c) m[c] = __uint_as_float(x.m[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) m[c] = dequant8<true, ST == FORGE_S_Q8D>(x.m.x >> (8 * c), x.ms);
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = __uint_as_float(x.v[c]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = dequant8<false, ST == FORGE_S_Q8D>(x.v.x >> (8 * c), x.vs);
    }
  }

  float wn[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float mc = HM ? m[c] : 0.0f, vc = HV ? v[c] : 0.0f;
    wn[c] = rule<OPT>(g[c], w[c], mc, vc, e.s);
    m[c] = mc;
    v[c] = vc;
  }

  if (e.w_pre) {
    u32x4 a;
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(wn[c]);
    st16(e.w_pre + i0, a);
  }

  if constexpr (WT == FORGE_W_BF16) {
    uint32_t r[4];
    if (e.sr) {
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = f32_to_bf16_sr(wn[c], (uint32_t)(srw >> (16 * c)) & 0xFFFFu);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = f32_to_bf16_rne(wn[c]);
    }
    st8(static_cast<uint16_t*>(e.W) + i0, u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)});
  } else {
    u32x4 a;
#pragma unroll
    for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(wn[c]);
    st16(static_cast<float*>(e.W) + i0, a);
  }

  const bool leader = ((i0 >> 2) & 15u) == 0u;
  if constexpr (HM) {
    if constexpr (ST == FORGE_S_F32) {
      u32x4 a;
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(m[c]);
      st16(static_cast<float*>(e.m) + i0, a);
    } else {
      uint32_t code[4];
      const float scale = quant_block64<true, ST == FORGE_S_Q8D, 4, 16>(m, code);
      st4(static_cast<int8_t*>(e.m) + i0, code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24));
      if (leader) e.m_scale[i0 >> 6] = scale;
    }
  }
  if constexpr (HV) {
    if constexpr (ST == FORGE_S_F32) {
      u32x4 a;
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] = __float_as_uint(v[c]);
      st16(static_cast<float*>(e.v) + i0, a);
    } else {
      uint32_t code[4];
      const float scale = quant_block64<false, ST == FORGE_S_Q8D, 4, 16>(v, code);
      st4(static_cast<uint8_t*>(e.v) + i0, code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24));
      if (leader) e.v_scale[i0 >> 6] = scale;
    }
  }
}

// Applies rule OPT to 16 consecutive elements of one row of W, starting at flat index i0
// (a multiple of 16): loads the stored state, updates it, writes it back.  For int8 moments
// the 64-element block spans the 4 consecutive lanes lane^1, lane^2 (all four must be active).
template <int OPT, int WT, int ST>
__device__ __forceinline__ void step_segment16(const float (&g)[16], uint32_t i0, const EpiArgs& e) {
  SegIn x;
  seg_load<OPT, WT, ST>(x, i0, e);
  seg_apply<OPT, WT, ST>(g, i0, x, e);
}

}  // namespace forge
