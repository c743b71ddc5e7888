// fp8_codec.h -- device-side FP8 codec and step arithmetic for gfx950 (CDNA4).
//
// Formats: OCP E4M3FN and E5M2, the two FP8 formats whose bit splits the
// daoxuan.cc explainer of arXiv 2409.12517 tabulates (section on why Adam keeps
// m in E4M3 and v in E5M2, "The two FP8 formats") and the zyxy.net FP8
// article lists ("FP8 formats").  gfx950's packed converts implement exactly
// these (OCP) encodings with round-to-nearest-even; saturation is done by
// clamping to +-FMAX with v_med3_f32 first, so the converts never overflow.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8adam {

// FMAX = 0.875 * 2^kMaxExp for both formats: 448 = 0.875 * 2^9, 57344 = 0.875 * 2^16.
// kMantBits: mantissa field width; kMaxCode: the code of +FMAX.
template <int FMT> struct Format;
template <> struct Format<0> {  // E4M3
  static constexpr float kMax = 448.0f;
  static constexpr int kMaxExp = 9;
  static constexpr int kMantBits = 3;
  static constexpr uint32_t kMaxCode = 0x7Eu;
};
template <> struct Format<1> {  // E5M2
  static constexpr float kMax = 57344.0f;
  static constexpr int kMaxExp = 16;
  static constexpr int kMantBits = 2;
  static constexpr uint32_t kMaxCode = 0x7Bu;
};

// Re-express four codes quantized with the power-of-two scale 2^a in the scale
// 2^b (d = b - a, nonzero) by moving each exponent field down by d.  Where the
// code lies strictly between the smallest normal and FMAX, before and after the
// move, the unrounded value was a normal FP8 number at both scales (only the
// smallest-normal code can come from a subnormal value rounded up, and a code
// above it after the move leaves the value normal even if it was rounded up
// from the binade below), and multiplying by a power of two keeps the
// significand: rounding to nearest even, or stochastic rounding with the same
// random bits, then keeps the same mantissa bits in the other binade.  With
// zero_ok (the values shrink, d > 0, under round-to-nearest) a zero code stays
// itself: the value was at most half the smallest subnormal and only gets
// smaller.  Returns false if any of the four needs the value itself: a zero
// (unless zero_ok), subnormal or smallest-normal code, the FMAX code (which may
// hold a saturated value), a NaN/Inf code, or a result outside that range.
template <int FMT>
__device__ __forceinline__ bool shift_codes4(uint32_t w, int d, bool zero_ok, uint32_t& out) {
  constexpr int kMinNormal = 1 << Format<FMT>::kMantBits;
  constexpr int kTop = (int)Format<FMT>::kMaxCode;
  const int step = d * kMinNormal;  // d in exponent units, as a code difference
  bool ok = true;
  uint32_t r = 0u;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t b = (w >> (8 * j)) & 0xFFu;
    const int mag = (int)(b & 0x7Fu);
    const int nm = mag - step;
    const bool keep_zero = zero_ok && mag == 0;
    const bool normal = mag > kMinNormal && mag < kTop && nm > kMinNormal && nm < kTop;
    ok = ok && (keep_zero || normal);
    r |= ((b & 0x80u) | (keep_zero ? 0u : ((uint32_t)nm & 0x7Fu))) << (8 * j);
  }
  out = r;
  return ok;
}

// Four codes packed little-endian in a dword -> four floats (exact).
template <int FMT>
__device__ __forceinline__ void decode4(uint32_t w, float (&out)[4]) {
  if constexpr (FMT == 0) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
  } else {
    auto lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
  }
}

template <int FMT>
__device__ __forceinline__ float decode1(uint32_t code) {
  if constexpr (FMT == 0) return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
  else return __builtin_amdgcn_cvt_pk_f32_bf8((int)code, false)[0];
}

// Four floats -> four codes (RNE, saturating at +-FMAX), packed little-endian.
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  constexpr float M = Format<FMT>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

template <int FMT>
__device__ __forceinline__ uint32_t encode1(float a) {
  return encode4<FMT>(a, 0.0f, 0.0f, 0.0f) & 0xFFu;
}

// Stochastic rounding (the zyxy.net article's strategies section: stochastic
// rounding against the error that accumulates over many updates).  Let lo and
// lo + s be the FP8 neighbours of |q| (s = the FP8 spacing at |q|, fixed below
// the smallest normal) and f = (|q| - lo) / s; q rounds up iff
// floor(f * 2^16) + r16 >= 2^16.  gfx950's stochastic-rounding converts
// (v_cvt_sr_fp8_f32 / v_cvt_sr_bf8_f32) add their random operand to the bits
// that are rounded away, aligned at the top of those bits, and carry; with the
// 16 random bits in the operand's top half and zeros below, that is exactly the
// rule above, in the normal and the subnormal FP8 range alike (checked against
// an independent encoder for every fp32 pattern in the FP8 range and for all
// 2^16 values of r16 on sampled inputs).  Inputs are clamped to +-FMAX first,
// so the converts saturate instead of overflowing; NaN inputs are outside the
// contract.  r16[j] holds 16 random bits in its low half.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_sr(float a, float b, float c, float d, const uint32_t (&r16)[4]) {
  constexpr float M = Format<FMT>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (FMT == 0) {
    w = __builtin_amdgcn_cvt_sr_fp8_f32(a, (int)(r16[0] << 16), 0, 0);
    w = __builtin_amdgcn_cvt_sr_fp8_f32(b, (int)(r16[1] << 16), w, 1);
    w = __builtin_amdgcn_cvt_sr_fp8_f32(c, (int)(r16[2] << 16), w, 2);
    w = __builtin_amdgcn_cvt_sr_fp8_f32(d, (int)(r16[3] << 16), w, 3);
  } else {
    w = __builtin_amdgcn_cvt_sr_bf8_f32(a, (int)(r16[0] << 16), 0, 0);
    w = __builtin_amdgcn_cvt_sr_bf8_f32(b, (int)(r16[1] << 16), w, 1);
    w = __builtin_amdgcn_cvt_sr_bf8_f32(c, (int)(r16[2] << 16), w, 2);
    w = __builtin_amdgcn_cvt_sr_bf8_f32(d, (int)(r16[3] << 16), w, 3);
  }
  return (uint32_t)w;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32x32->64-bit multiplies; the key
// is bumped by the two Weyl constants between rounds.  Each round's two
// three-way XORs are single gfx950 v_bitop3_b32 instructions (truth table 0x96),
// which the compiler otherwise splits into two XORs each.  The key (uniform,
// in scalar registers) is bumped in place behind an empty asm statement each
// round: left to itself the compiler computed all twenty round keys up front
// and, short of scalar registers at eight waves per SIMD, spilled them to
// vector lanes and read them back in the rounds.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
    asm volatile("" : "+s"(k0), "+s"(k1));  // emits nothing; keeps the schedule sequential
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// bf16 <-> fp32.  Widening is exact (shift); narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN, sign kept
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Scale from the amax of a block (fp32 bit pattern, sign bit clear).
// POW2 (mode 0): smallest power of two s with amax/s <= FMAX; with
// amax = f * 2^e, f in [0.5, 1): k = e - kMaxExp + [f > 0.875], clamped to
// [-126, 126]; f > 0.875 <=> the fp32 mantissa field exceeds 0x600000.
// AMAX (mode 1): s = amax/FMAX, inv = FMAX/amax, correctly rounded; s below
// 2^-126 is raised to it.  amax = 0 or non-finite gives s = inv = 1.
// The dynamic-range rule follows the zyxy.net article's "Strategies" section
// (track the max-abs value, adjust the exponent offset).
template <int FMT, int SMODE>
__device__ __forceinline__ void choose_scale(uint32_t amax_bits, float& s, float& inv) {
  const uint32_t ef = amax_bits >> 23;
  if (amax_bits == 0u || ef >= 255u) {
    s = 1.0f;
    inv = 1.0f;
    return;
  }
  if constexpr (SMODE == 0) {
    int k = (ef == 0u) ? -126
                       : (int)ef - 126 - Format<FMT>::kMaxExp + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    k = k < -126 ? -126 : (k > 126 ? 126 : k);
    s = __uint_as_float((uint32_t)(k + 127) << 23);
    inv = __uint_as_float((uint32_t)(127 - k) << 23);
  } else {
    const float a = __uint_as_float(amax_bits);
    const float sc = __fdiv_rn(a, Format<FMT>::kMax);
    if (sc < 0x1p-126f) {
      s = 0x1p-126f;
      inv = 0x1p126f;
    } else {
      s = sc;
      inv = __fdiv_rn(Format<FMT>::kMax, a);
    }
  }
}

// Per-step constants, computed on the host from the hyperparameters.
struct StepConsts {
  float b1, b2;        // beta1, beta2
  float omb1, omb2;    // 1 - beta (fp32)
  float decay;         // 1 - lr * weight_decay (1 with coupled L2)
  float l2;            // coupled L2: weight_decay, added to the gradient as l2 * p
  float step_size;     // lr / (1 - beta1^t)
  float inv_bc2;       // 1 / (1 - beta2^t)
  float eps;
  float grow_m, grow_v; // speculative schedule: predicted amax growth from step t-1 to t
  float gfac;          // factor applied to every bf16 gradient first (1; loss-scale unscaling and clipping)
  uint32_t seed_lo, seed_hi;  // stochastic rounding: the generator's key
  uint32_t rng_t;      // stochastic rounding: the step t in the generator's counter
  float margin_scale;  // delayed scaling: 2^margin
  int hist_len;        // delayed scaling: H (0: no history)
  int hist_slot;       // delayed scaling: (t-1) mod H, the slot this step's amax goes to
};

// Moment update (daoxuan.cc explainer, "Adam's update makes the needs
// asymmetric": m averages g, v averages g^2).  Evaluated exactly as
// fma(b1, m, (1-b1)*g) and fma(b2, v, (1-b2)*(g*g)) so the FP8 codes that
// follow are bit-exact functions of the inputs; contraction is off here.
__device__ __forceinline__ void moment_update(const StepConsts& c, float g, float m, float v,
                                              float& m1, float& v1) {
#pragma clang fp contract(off)
  const float gm = c.omb1 * g;
  const float gg = g * g;
  const float gv = c.omb2 * gg;
  m1 = __builtin_fmaf(c.b1, m, gm);
  v1 = __builtin_fmaf(c.b2, v, gv);
}

// Gradient the moments see: g, or with coupled L2 g + l2 * p (one fp32
// rounding, the parameter before the step).  The L2-regularised loss is the
// objective of Theorem 1's set-up in the daoxuan.cc explainer (section on why
// the two SwiGLU weight vectors align).
template <bool L2>
__device__ __forceinline__ float grad_eff(const StepConsts& c, float g, float p) {
  if constexpr (L2) return __builtin_fmaf(c.l2, p, g);
  else return g;
}

// The gradient as the moments take it: times the step's gradient factor (exact
// for 1), then the coupled-L2 term if any.
template <bool L2>
__device__ __forceinline__ float grad_in(const StepConsts& c, float g, float p) {
  return grad_eff<L2>(c, g * c.gfac, p);
}

// AdamW parameter update from the fresh moments: m in the numerator times the
// bias-corrected step size, eps added after the square root of v-hat
// (daoxuan.cc explainer, numerical example), decoupled decay (AdamW in the
// zyxy.net code example).  Hardware sqrt / reciprocal: about 1 ulp each.
__device__ __forceinline__ float param_update(const StepConsts& c, float p, float m1, float v1) {
  const float den = __builtin_amdgcn_sqrtf(v1 * c.inv_bc2) + c.eps;
  const float upd = (c.step_size * m1) * __builtin_amdgcn_rcpf(den);
  return __builtin_fmaf(p, c.decay, -upd);
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

}  // namespace fp8adam
