// Device codecs for the NVFP4 / MXFP8 expert layer on gfx950.
//
// Formats are the ones named on "Inkling 2 Small uses four-bit training ..."
// (ai-primer), section "Block scales and per-token activations": E2M1 elements
// with an E4M3 scale per 16 (NVFP4), E4M3 elements with an E8M0 scale per 32
// (MXFP8). Every routine is exact integer/float bit manipulation whose result
// is fixed by IEEE binary32 arithmetic (no fused multiply-add is relied on;
// the library is compiled with -ffp-contract=off), so results are identical
// on any conforming implementation of the same rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4moe {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float u2f(uint32_t x) { return __uint_as_float(x); }

// bfloat16 bit pattern -> float32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return u2f(h << 16); }

// float32 -> bfloat16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = f2u(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> two bf16 in one word (a in the low half), rounded to nearest
// even by gfx950's packed conversion (one instruction; the same result as
// f32_to_bf16_rne for every non-NaN input).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ----------------------------------------------------------------- E2M1

// Eight floats -> eight E2M1 codes packed in a word (element j in bits
// 4j..4j+3), rounded to nearest with ties to the even code, saturating at 6,
// sign bit kept (so -0 and tiny negatives give code 8). This is
// v_cvt_scalef32_pk_fp4_f32 with a unit scale, checked against the
// threshold rule (a midpoint of neighbouring grid values goes to the one
// with the even code) on every midpoint, its float32 neighbours, a dense
// sweep of [0, 8) and saturating values, for both signs.
__device__ __forceinline__ uint32_t e2m1x8_rne(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// Stochastic rounding of y onto the E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}
// with a 16-bit draw u: with lo the grid value at or below |y| and D its
// fractional distance to the next one, round up iff u + floor(D * 2^16) >=
// 2^16. |y| >= 6 gives 6 (saturation, reached only through float32 rounding
// when block scales are rounded up). The sign bit of y is kept. Position
// arithmetic is exact: 2|y|, |y| - 2 and (|y| - 4) / 2 are exact in float32.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) {
  const float a = fabsf(y);
  uint32_t mag;
  if (a >= 6.0f) {
    mag = 7u;
  } else {
    float t;
    uint32_t base;
    if (a < 2.0f) { t = a * 2.0f; base = 0u; }                 // codes 0..3, step 0.5
    else if (a < 4.0f) { t = a - 2.0f; base = 4u; }            // codes 4..5, step 1
    else { t = (a - 4.0f) * 0.5f; base = 6u; }                 // code 6, step 2
    const float fl = floorf(t);
    const uint32_t d16 = (uint32_t)((t - fl) * 65536.0f);      // floor: exact product
    mag = base + (uint32_t)fl + ((u + d16) >> 16);
  }
  return mag | ((f2u(y) >> 28) & 8u);
}

// Eight values -> eight stochastically rounded E2M1 codes packed in a word
// (element j in bits 4j..4j+3), draws u[j].
__device__ __forceinline__ uint32_t e2m1x8_sr(const float* v, const uint32_t* u) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= e2m1_sr(v[j], u[j]) << (4 * j);
  return w;
}

// Two E2M1 codes (one byte: element 2i low nibble) -> float32 values
// (v_cvt_scalef32_pk_f32_fp4 with a unit scale decodes exactly).
__device__ __forceinline__ void e2m1x2_to_f32(uint32_t word, int byte, float& lo, float& hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  f32x2_t v;
  switch (byte) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
  }
  lo = v.x;
  hi = v.y;
}

// ----------------------------------------------------------------- E4M3

// Value of a non-negative E4M3FN code (0..0x7E) as float32 (exact).
__device__ __forceinline__ float e4m3_pos_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0.001953125f;            // m * 2^-9, exact
  const float nrm = u2f(((e + 120u) << 23) | (m << 20));
  return e ? nrm : sub;
}

// Round a non-negative float32 to E4M3FN, nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat_pos(float t) {
  if (t >= 448.0f) return 0x7Eu;
  if (t < 0.015625f)                                     // below 2^-6: step 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);      // 0..8, exact product
  uint32_t b = f2u(t);
  b += 0x7FFFFu + ((b >> 20) & 1u);                     // round mantissa to 3 bits
  return (b >> 20) - (120u << 3);                       // rebias exponent 127 -> 7
}

// Smallest E4M3FN value >= t for t >= 0 (448 for larger t) -> code.
__device__ __forceinline__ uint32_t e4m3_ceil_pos(float t) {
  uint32_t c = e4m3_rne_sat_pos(t);
  if (c < 0x7Eu && e4m3_pos_to_f32(c) < t) ++c;
  return c;
}

// Four values with |y| <= 448 -> E4M3FN bytes (first value in the low byte),
// round to nearest even (ties to the even code), sign kept: v_cvt_pk_fp8_f32
// (checked against a brute-force nearest-even search on subnormal ties and a
// dense sweep of [-448, 448]).
__device__ __forceinline__ uint32_t e4m3x4_rne(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Stochastic rounding of four values |y| <= 448 to E4M3FN bytes (first value
// in the low byte) with 16-bit draws u0..u3. With lo the grid value at or
// below |y| and D = (|y| - lo) / gap, a value rounds up iff
// u + floor(D * 2^16) >= 2^16; sign kept. v_cvt_sr_fp8_f32 implements exactly
// this rule when the draw occupies the high 16 bits of its random operand
// (checked against the rule on 2.6e5 values spanning the normal and subnormal
// E4M3 ranges, grid values and both signs).
__device__ __forceinline__ uint32_t e4m3x4_sr(float y0, float y1, float y2, float y3, uint32_t u0,
                                              uint32_t u1, uint32_t u2, uint32_t u3) {
  int w = __builtin_amdgcn_cvt_sr_fp8_f32(y0, u0 << 16, 0, 0);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(y1, u1 << 16, w, 1);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(y2, u2 << 16, w, 2);
  w = __builtin_amdgcn_cvt_sr_fp8_f32(y3, u3 << 16, w, 3);
  return (uint32_t)w;
}

// The same two conversions with the division by the block scale folded into
// the instruction: `scale` is a float32 whose exponent field is the block's
// E8M0 code c (mantissa zero), and the result equals converting x * 2^(127-c)
// after an exact float32 multiply. Checked on gfx950 for every code from 0
// (2^-127) to 247 (2^120), with x in the normal, subnormal and below-half-step
// ranges of the scaled value, at grid points, at 0 and 448, both signs, and
// with x itself a float32 subnormal.
// Each random operand holds its 16-bit draw in the high half and zeros below,
// as for e4m3x4_sr.
__device__ __forceinline__ uint32_t e4m3x4_sr_scaled(float x0, float x1, float x2, float x3,
                                                     uint32_t r0, uint32_t r1, uint32_t r2,
                                                     uint32_t r3, float scale) {
  int w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, x0, r0, scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, x1, r1, scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, x2, r2, scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(w, x3, r3, scale, 3);
  return (uint32_t)w;
}
__device__ __forceinline__ uint32_t e4m3x4_rne_scaled(float x0, float x1, float x2, float x3,
                                                      float scale) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  s16x2_t w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x0, x1, scale, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x2, x3, scale, true);
  return (uint32_t)(uint16_t)w[0] | ((uint32_t)(uint16_t)w[1] << 16);
}

// ----------------------------------------------------------------- E8M0

// Smallest e with amax <= 448 * 2^e, clamped to [-127, 127]; 0 gives -127.
__device__ __forceinline__ int e8m0_ceil(float amax) {
  const uint32_t b = f2u(amax);
  if (b < 0x00800000u) return -127;                     // zero or subnormal
  const int E = (int)(b >> 23) - 127;
  const int e = ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;   // m <= 1.75
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// The same exponent as an E8M0 code c = e + 127, from the bits of a
// non-negative float32 amax: adding 0x1FFFFF carries into the exponent field
// exactly when the mantissa exceeds 0.75 (amax > 1.75 * 2^E), so the field
// becomes E + 127 + [m > 0.75] and c = field - 8 (E + 119 is 448 = 1.75 * 2^8
// away). Zero and subnormal amax give a field of 0 or 1, clamped to c = 0.
// Finite amax gives c <= 247.
__device__ __forceinline__ uint32_t e8m0_code_bits(uint32_t amax_bits) {
  const uint32_t t = (amax_bits + 0x1FFFFFu) >> 23;
  return (t > 8u ? t : 8u) - 8u;
}

// 2^-e as float32 for e in [-127, 120] (always a normal number).
__device__ __forceinline__ float exp2_neg(int e) { return u2f((uint32_t)(127 - e) << 23); }

// ----------------------------------------------------------------- Philox

struct Philox4 {
  uint32_t w0, w1, w2, w3;
};

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, SC'11): each round
// multiplies words 0 and 2 by the two round constants into 64-bit products and
// mixes their halves with words 1 and 3 and the key; the key is bumped by the
// two Weyl constants between rounds.
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    // three-way XORs in one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{c0, c1, c2, c3};
}

// The eight 16-bit draws for output indices 8q .. 8q+7 (index 8q+i is half
// i&1 of word i>>1, low half first), keyed by (seed, tag).
struct Draws8 {
  uint32_t w[4];
  __device__ __forceinline__ uint32_t get(int i) const {
    return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
  }
};

__device__ __forceinline__ Draws8 draws8(uint64_t q, uint64_t seed, uint32_t tag) {
  const Philox4 p = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), tag, 0u,
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
  return Draws8{{p.w0, p.w1, p.w2, p.w3}};
}

// ----------------------------------------------------------------- misc

// Maximum over the four lanes of a quad (lanes 4q .. 4q+3, all active), on
// the bits of non-negative floats (their order is the integer order); two
// DPP quad permutations, no LDS traffic.
__device__ __forceinline__ uint32_t quad_max_bits(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true));  // lane ^ 1
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));  // lane ^ 2
  return m;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace nvfp4moe
