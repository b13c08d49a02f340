// Device helpers shared by the AWQ kernels (gfx950 / CDNA4, wave64).
//
// The group quantizer here is the only one on the GPU: the stand-alone quantize+pack
// kernel and the grid-search kernel both call it, so the codes the search scores are
// the codes the pack kernel writes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "awq.h"

namespace awq {

constexpr int kGroup = 128;   // input channels per quantization group
constexpr int kQMax = 15;     // 4-bit unsigned codes 0..15 with a zero point (8-bit: 0..255)
constexpr int kWave = 64;

// Packed word layout: word w covers input channels 8w..8w+7; channel i sits in nibble
// kNibbleOf[i] (bits 4n..4n+3). Channels 0, 2, 4, 6 fill the low nibbles of the four bytes
// and 1, 3, 5, 7 the high ones, so (word >> 4p) & 0x000F000F holds the adjacent pair
// (2p, 2p+1) in its two 16-bit halves.
__device__ constexpr int kNibbleOf[8] = {0, 4, 1, 5, 2, 6, 3, 7};

__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h_bits(float f) {  // v_cvt_f16_f32, round-to-nearest-even
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// ------------------------------------------------------------------ DPP reductions
// Reductions inside one 16-lane DPP row: quad_perm butterflies, then row rotations.
// Every lane of the row ends up with the result.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// min / max of a value and the value of the lane a DPP control selects, as one
// DPP-modified instruction each (through the compiler, a DPP move plus a canonicalizing
// max plus the min / max). s_nop 1 covers the two wait states a VALU write needs before a
// DPP read of the same register.
#define AWQ_DPP_MINMAX(NAME, CTRL)                                                        \
  __device__ __forceinline__ void NAME(float& mn, float& mx) {                            \
    float a, b;                                                                           \
    asm("s_nop 1\n\tv_min_f32_dpp %0, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"     \
        "v_max_f32_dpp %1, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf"                     \
        : "=&v"(a), "=&v"(b)                                                              \
        : "v"(mn), "v"(mx));                                                              \
    mn = a;                                                                               \
    mx = b;                                                                               \
  }
AWQ_DPP_MINMAX(minmax_quad_xor1, "quad_perm:[1,0,3,2]")
AWQ_DPP_MINMAX(minmax_quad_xor2, "quad_perm:[2,3,0,1]")
AWQ_DPP_MINMAX(minmax_row_ror4, "row_ror:4")
AWQ_DPP_MINMAX(minmax_row_ror8, "row_ror:8")
AWQ_DPP_MINMAX(minmax_row_half_mirror, "row_half_mirror")
#undef AWQ_DPP_MINMAX

// max only (the reductions of a nonnegative largest |D|): one DPP-modified instruction
#define AWQ_DPP_MAX(NAME, CTRL)                                                           \
  __device__ __forceinline__ void NAME(float& mx) {                                       \
    float b;                                                                              \
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf"         \
        : "=&v"(b)                                                                        \
        : "v"(mx));                                                                       \
    mx = b;                                                                               \
  }
AWQ_DPP_MAX(max_quad_xor1, "quad_perm:[1,0,3,2]")
AWQ_DPP_MAX(max_quad_xor2, "quad_perm:[2,3,0,1]")
AWQ_DPP_MAX(max_row_ror4, "row_ror:4")
AWQ_DPP_MAX(max_row_ror8, "row_ror:8")
AWQ_DPP_MAX(max_row_half_mirror, "row_half_mirror")
#undef AWQ_DPP_MAX

// Min / max over each 16-lane DPP row (128-channel groups): quad butterflies, then row
// rotations; every lane of the row ends up with the result.
__device__ __forceinline__ void row16_minmax(float& mn, float& mx) {
  minmax_quad_xor1(mn, mx);
  minmax_quad_xor2(mn, mx);
  minmax_row_ror4(mn, mx);
  minmax_row_ror8(mn, mx);
}

// Min / max over the 8-lane halves of each DPP row (64-channel groups): quad butterflies,
// then row_half_mirror, which pairs lane i of a half with lane 7 - i (the other quad).
__device__ __forceinline__ void row8_minmax(float& mn, float& mx) {
  minmax_quad_xor1(mn, mx);
  minmax_quad_xor2(mn, mx);
  minmax_row_half_mirror(mn, mx);
}

// Min / max over each quad of lanes (32-channel groups): the two quad_perm butterflies.
__device__ __forceinline__ void quad_minmax(float& mn, float& mx) {
  minmax_quad_xor1(mn, mx);
  minmax_quad_xor2(mn, mx);
}

// Group min / max when each lane holds 8 consecutive channels: a group of g channels is
// g / 8 adjacent lanes (16 for g = 128, 8 for g = 64, 4 for g = 32).
__device__ __forceinline__ void group_minmax(float& mn, float& mx, int group) {
  if (group == 128) row16_minmax(mn, mx);
  else if (group == 64) row8_minmax(mn, mx);
  else quad_minmax(mn, mx);
}

// Max over each 16-lane row / each group of g / 8 adjacent lanes, as group_minmax.
__device__ __forceinline__ void row16_max(float& mx) {
  max_quad_xor1(mx);
  max_quad_xor2(mx);
  max_row_ror4(mx);
  max_row_ror8(mx);
}
__device__ __forceinline__ void group_max(float& mx, int group) {
  max_quad_xor1(mx);
  max_quad_xor2(mx);
  if (group == 128) {
    max_row_ror4(mx);
    max_row_ror8(mx);
  } else if (group == 64) {
    max_row_half_mirror(mx);
  }
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return v;
}

// Sum over the whole wave; the result is valid in every lane. Fixed order, so the
// result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// ------------------------------------------------------------------ group quantizer
// Per group of g values w' (= w * s, an exact fp32 product), in fp32 with
// round-to-nearest-even and no contraction:
//   sc = max((mx - mn) / 15, 2^-14), clamped at 65504; sc_h = fp16(sc);
//   z = clamp(rint(-mn / sc_h), 0, 15);  q = clamp(rint(w' / sc_h) + z, 0, 15).
struct GroupQ {
  float qmax;    // largest code: 15 (4-bit) or 255 (8-bit)
  float scf;     // the stored scale as fp32
  float rcp;     // hardware reciprocal of scf (within 1 ulp), only to guess quotients
  float z;       // zero point, 0..15
  uint16_t sch;  // fp16 bits of the stored scale
  bool clamped;  // sc exceeded 65504
};

// rint(w_i / scf) for NV values, equal to rint of the correctly rounded quotient. The
// product w * rcp is within 1.5 * 2^-23 (relative) of the real quotient; unless it sits
// within |q| * 2^-21 of a half-integer, it lies on the same side of that half-integer as
// the correctly rounded quotient and rint gives the same integer. Close calls are rare
// (about 2^-17 per value): the wave takes the correctly rounded division for them in a
// branch it skips unless one of its lanes has one, so the common path has no division.
template <int NV>
__device__ __forceinline__ void rint_quotients(const float (&w)[NV], float scf, float rcp,
                                               float (&q)[NV]) {
#pragma clang fp contract(off)
  bool close[NV];
  bool any = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float qa = w[i] * rcp;
    const float fl = __builtin_floorf(qa);
    const float d = __builtin_fabsf((qa - fl) - 0.5f);
    close[i] = !(d > __builtin_fabsf(qa) * 0x1p-21f + 0x1p-60f);
    any |= close[i];
    q[i] = qa;
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
    asm volatile("");  // keeps the division in this branch (not speculated into the common path)
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (close[i]) q[i] = w[i] / scf;  // correctly rounded division
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) q[i] = __builtin_rintf(q[i]);
}

// x / d correctly rounded, for the divisors of the group scales (d = 3, 7, 15, 127, 255),
// given y = RN(1 / d): q0 = RN(x y), the residual r = x - q0 d exactly (one fma), then
// RN(q0 + r y) (one fma), Markstein's correction. For these five divisors it equals the
// IEEE quotient for every fp32 significand (checked exhaustively: the test of the
// division method); scaling by a power of two commutes with it while r stays normal, and
// below that the quotient is far under the 2^-14 floor the scales take. Non-finite x: x y
// (Inf or NaN, as the division gives). Three instructions and a select instead of the
// division's ten.
__device__ __forceinline__ float div_small(float x, float d, float y) {
#pragma clang fp contract(off)
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, d, x);
  const float q1 = __builtin_fmaf(r, y, q0);
  return __builtin_isfinite(x) ? q1 : q0;
}

// The divisor of the group scale and its correctly rounded reciprocal: qmax for asymmetric
// codes, h - 1 = (qmax - 1) / 2 for symmetric ones. Uniform: computed once per kernel.
struct ScaleDiv {
  float d, y;
};
__device__ __forceinline__ ScaleDiv scale_divisor(float qmax, bool sym) {
  const float d = sym ? 0.5f * (qmax + 1.0f) - 1.0f : qmax;  // exact
  return ScaleDiv{d, 1.0f / d};                               // correctly rounded
}

// Asymmetric group parameters for codes 0..qmax (qmax = 2^w_bit - 1); sd = scale_divisor(qmax, false).
__device__ __forceinline__ GroupQ group_params(float mn, float mx, float qmax, ScaleDiv sd) {
#pragma clang fp contract(off)
  GroupQ g;
  g.qmax = qmax;
  float sc = div_small(mx - mn, sd.d, sd.y);  // the correctly rounded (mx - mn) / qmax
  sc = fmaxf(sc, 0x1p-14f);
  g.clamped = sc > 65504.0f;
  sc = fminf(sc, 65504.0f);
  g.sch = f2h_bits(sc);
  g.scf = h2f(g.sch);
  g.rcp = __builtin_amdgcn_rcpf(g.scf);
  const float nmn[1] = {-mn};
  float zq[1];
  rint_quotients(nmn, g.scf, g.rcp, zq);
  g.z = __builtin_amdgcn_fmed3f(zq[0], 0.0f, qmax);  // clamp to [0, qmax]
  return g;
}

// Symmetric variant (zero point off): sc = max(|mx|, |mn|) / (h - 1) with the same floor
// and clamp, and the fixed zero h = 2^(w_bit - 1) (8 or 128), so q - h = clamp(rint(w /
// sc_h), -h, h - 1) is the signed code and the stored format (and its dequantization
// (q - z) sc) is unchanged.
// sd = scale_divisor(qmax, true).
__device__ __forceinline__ GroupQ group_params_sym(float mn, float mx, float qmax, ScaleDiv sd) {
#pragma clang fp contract(off)
  GroupQ g;
  g.qmax = qmax;
  const float h = 0.5f * (qmax + 1.0f);  // exact
  float sc = div_small(fmaxf(__builtin_fabsf(mx), __builtin_fabsf(mn)), sd.d, sd.y);  // / (h - 1)
  sc = fmaxf(sc, 0x1p-14f);
  g.clamped = sc > 65504.0f;
  sc = fminf(sc, 65504.0f);
  g.sch = f2h_bits(sc);
  g.scf = h2f(g.sch);
  g.z = h;
  g.rcp = __builtin_amdgcn_rcpf(g.scf);
  return g;
}

// Codes q = clamp(rint(w / sc_h) + z, 0, qmax) of NV values w of one group, each the
// exact fp32 product of two fp16 numbers (at most 22 significant bits).
// q0 = rint(w * rcp) is taken when the residual e = w - q0 sc_h, formed by one fma, has
// |e| < sc_h / 2. For |q0| < 2^12, q0 sc_h is exact (at most 23 bits) and so is e: when
// q0 is within 1 of the quotient, |e| < 1.5 sc_h, and e is a multiple of the finer of
// ulp(w) and ulp(sc_h), at least 2^-23 |e| when q0 != 0 (then |w| >= sc_h / 2), so e fits
// 24 bits; q0 = 0 gives e = w. The test is therefore exact, and q0 is then the rint of
// the real quotient. For larger
// |q0| the guess is still within 1 of it and q0 + z lies far outside [0, qmax], so the
// clamp gives the same code either way. Everything else (|e| >= sc_h / 2: a wrong guess
// or an exact tie; NaN; Inf) takes the correctly rounded division in a branch the wave
// enters only when one of its lanes needs it.
template <int NV>
__device__ __forceinline__ void quant_codes(const float (&w)[NV], const GroupQ& g, float (&q)[NV]) {
#pragma clang fp contract(off)
  const float half_sc = 0.5f * g.scf;  // exact
  bool close[NV];
  bool any = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    q[i] = __builtin_rintf(w[i] * g.rcp);
    const float e = __builtin_fmaf(-q[i], g.scf, w[i]);
    close[i] = !(__builtin_fabsf(e) < half_sc) && !(__builtin_fabsf(q[i]) >= 4096.0f);
    any |= close[i];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (close[i]) q[i] = __builtin_rintf(w[i] / g.scf);  // correctly rounded division
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i] + g.z, 0.0f, g.qmax);  // clamp
}

// The centered codes q - z of quant_codes, formed directly as clamp(rint(w / sc_h), -z,
// qmax - z): small integers, so the same values as clamping rint(w / sc_h) + z to [0, qmax]
// and subtracting z. For the searches, which only need (q - z) sc_h. The guess is kept on
// the same exact-residual test; here a large guess (|q0| >= 2^12, only in groups whose scale
// is floored) whose residual fails it also takes the division, which changes no result.
template <int NV>
__device__ __forceinline__ void quant_centered(const float (&w)[NV], const GroupQ& g,
                                               float (&qz)[NV]) {
#pragma clang fp contract(off)
  const float half_sc = 0.5f * g.scf;  // exact
  bool close[NV];
  bool any = false;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    qz[i] = __builtin_rintf(w[i] * g.rcp);
    const float e = __builtin_fmaf(-qz[i], g.scf, w[i]);
    close[i] = !(__builtin_fabsf(e) < half_sc);
    any |= close[i];
  }
  if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (close[i]) qz[i] = __builtin_rintf(w[i] / g.scf);  // correctly rounded division
  }
  const float lo = -g.z, hi = g.qmax - g.z;  // exact
  // the clamp as a median of three (one instruction, the same value for every input)
#pragma unroll
  for (int i = 0; i < NV; ++i) qz[i] = __builtin_amdgcn_fmed3f(qz[i], lo, hi);
}

// The packed word of 8 codes of channels 8w .. 8w + 7 (channel i in nibble kNibbleOf[i]):
// byte b holds one channel pair, (0, 2), (4, 6), (1, 3), (5, 7) for b = 0 .. 3, so each
// byte is qa + 16 qb (exact) written with one v_cvt_pk_u8_f32.
__device__ __forceinline__ uint32_t pack_codes8(const float (&q)[8]) {
  uint32_t word = 0;
  word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[2], 16.0f, q[0]), 0, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[6], 16.0f, q[4]), 1, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[3], 16.0f, q[1]), 2, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[7], 16.0f, q[5]), 3, word);
  return word;
}

// 3-bit codes of 8 consecutive channels 0..7 (values 0..7 as floats) as their shares of
// the two bit planes: lo = bits 0-1 of channel 2i + e at bits 2i + 16e, hi = bit 2 of
// channel 2i + e at bit i + 16e (i = 0..3, e = 0..1), both for a lane whose channels start
// a plane word; the caller shifts them to the lane's place in the word.
__device__ __forceinline__ void planes3(const float (&q)[8], uint32_t& lo, uint32_t& hi) {
  lo = 0;
  hi = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t c = (uint32_t)q[t];
    lo |= (c & 3u) << (2 * (t >> 1) + 16 * (t & 1));
    hi |= (c >> 2) << ((t >> 1) + 16 * (t & 1));
  }
}

// 3-bit channel pair -> fp16 bits (1024 + q_a, 1024 + q_b), exactly: the pair's 2-bit field f
// of the low-plane word (bits 2f and 16 + 2f) shifted to bits 0-1 and OR-ed under the
// exponent (v_and_or_b32), its high-plane bit p (bits p and 16 + p) shifted to bit 2 and
// inserted (v_bfi_b32); `magic` holds 0x64006400. Callers unroll, so f and p are constants.
__device__ __forceinline__ uint32_t widen3_pair(uint32_t lo, uint32_t hi, int f, int p,
                                                uint32_t magic) {
  const uint32_t ls = lo >> (2 * f);
  const uint32_t hs = p >= 2 ? (hi >> (p - 2)) : (hi << (2 - p));
  uint32_t lm, u;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(lm) : "v"(ls), "s"(0x00030003u), "v"(magic));
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(u) : "s"(0x00040004u), "v"(hs), "v"(lm));
  return u;
}

// One word of four 8-bit codes, byte i = code i.
__device__ __forceinline__ uint32_t pack_bytes4(float q0, float q1, float q2, float q3) {
  uint32_t word = 0;
  word = __builtin_amdgcn_cvt_pk_u8_f32(q0, 0, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(q1, 1, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(q2, 2, word);
  word = __builtin_amdgcn_cvt_pk_u8_f32(q3, 3, word);
  return word;
}

// ------------------------------------------------------------------ fp64 -> fp16
// Exact round-to-nearest-even conversion of a double to binary16 bits (one rounding;
// a detour through fp32 would round twice).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double d) {
  uint64_t b = __builtin_bit_cast(uint64_t, d);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull) return sign | (mag > 0x7FF0000000000000ull ? 0x7E00 : 0x7C00);
  int e = (int)(mag >> 52) - 1023;
  if (e > 15) return sign | 0x7C00;
  if (e < -40) return sign;  // far below half the smallest subnormal
  uint64_t m = (mag & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);
  uint64_t q = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) return sign | (uint16_t)(((uint32_t)(e + 15) << 10) + (uint32_t)(q - 1024));
  return sign | (uint16_t)q;
}

// Magnitude of an fp16 value in units of 2^-24 (every finite fp16 is an integer
// multiple of 2^-24 below 2^40 units); returns -1 for Inf/NaN.
__device__ __forceinline__ int64_t f16_abs_units(uint16_t h) {
  uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  if (e == 31) return -1;
  if (e == 0) return (int64_t)m;
  return (int64_t)(1024 + m) << (e - 1);
}

// Shrink ratio of the weight-clipping grid: r_i = (steps - i) / steps, the correctly
// rounded fp32 quotient of two exact integers.
__device__ __forceinline__ float clip_ratio(int i, int steps) {
  return (float)(steps - i) / (float)steps;
}

// SiLU(v) = v / (1 + e^-v) in fp32, the activation of the fused gate|up epilogue, with
// the hardware exponential and reciprocal (relative error about 1e-6 for |v| <= 20, far
// below the result's fp16 rounding); large negative v: e^-v = inf, rcp(inf) = 0, -0.
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// Copy of a loaded vector through VGPRs the optimizer cannot see through. Storing a
// loaded value straight to LDS can otherwise leave it in a stack slot (scratch memory),
// whose reload waits, like any vector memory access, for every load still in flight.
__device__ __forceinline__ uint4 vgpr_copy(uint4 v) {
  uint4 r;
  asm volatile("v_mov_b32 %0, %4\n\tv_mov_b32 %1, %5\n\tv_mov_b32 %2, %6\n\tv_mov_b32 %3, %7"
               : "=v"(r.x), "=v"(r.y), "=v"(r.z), "=v"(r.w)
               : "v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
  return r;
}

}  // namespace awq
