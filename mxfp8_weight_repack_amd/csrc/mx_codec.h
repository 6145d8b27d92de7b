// mx_codec.h -- bit-exact MXFP8 encoding helpers for the HIP kernels.
//
// [OCP-MX] (the MXFP format cited by SS-HSDP §1/§2.3): an MX block shares one
// E8M0 scale 2^e; each element is stored as an E4M3 code of x * 2^-e.  E4M3 is
// the OCP "FN" variant: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest
// finite 448 (S.1111.110), NaN S.1111.111, no infinities.
//
// Scale rule: e = the least integer with amax <= 448 * 2^e, clamped to
// [-127, 127]; an all-zero block gets e = -127 and a block holding NaN/Inf
// gets the E8M0 NaN byte 0xFF.  With amax = (1 + f) * 2^E (f the 23-bit
// fraction), 448 = 1.75 * 2^8, so e = E - 8 when f <= 0.75 and E - 7 otherwise.
//
// Everything is integer logic on the float32 bit pattern: no float rounding,
// no dependence on the denormal mode, exact for every finite input.  The
// header compiles for the host as well, so the encoder can be checked on the
// CPU against a library conversion before it runs on a GPU.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MX_HD __host__ __device__ __forceinline__
#else
#define MX_HD static inline
#endif

// Scale byte (e + 127) of a block from the largest |x| bit pattern
// (max over (bits & 0x7fffffff) as unsigned, which also orders NaN above Inf).
MX_HD uint32_t mx_scale_byte(uint32_t amax_bits) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;       // NaN or Inf in the block
  const uint32_t ex = amax_bits >> 23;
  if (ex == 0u) return 0u;                          // zero or subnormal amax: e = -127
  int e = (int)ex - 135 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  if (e < -127) e = -127;
  return (uint32_t)(e + 127);
}

// Round-to-nearest-even right shift of a significand m < 2^24 by sh bits
// (sh <= 0 shifts left, at most by 3 here).  Written with selects only, so a
// wavefront runs it without divergent branches.
MX_HD uint32_t mx_rne_shr(uint32_t m, int sh) {
  const int s = sh < 0 ? 0 : (sh > 31 ? 31 : sh);
  const uint32_t q = m >> s;
  const uint32_t rem = m & ((1u << s) - 1u);
  const uint32_t half = s > 0 ? 1u << (s - 1) : 0u;
  const uint32_t up = (rem > half || (rem == half && half != 0u && (q & 1u))) ? 1u : 0u;
  const uint32_t left = m << (sh < 0 ? -sh : 0);
  return sh <= 0 ? left : q + up;
}

MX_HD int mx_clz32(uint32_t v) {                     // v != 0
#if defined(__HIPCC__) || defined(__GNUC__)
  return __builtin_clz(v);
#else
  int n = 0;
  while (!(v & 0x80000000u)) { v <<= 1; ++n; }
  return n;
#endif
}

// E4M3FN code of x * 2^-e for a finite float32 x (bits) whose block has scale
// exponent e (so |x * 2^-e| <= 448).  Ties to the even mantissa, sign kept.
// Branch-free: the normal and the subnormal encodings are both formed and one
// is selected.
MX_HD uint32_t mx_e4m3_code(uint32_t xb, int e) {
  const uint32_t sign = (xb >> 24) & 0x80u;
  const uint32_t ex = (xb >> 23) & 0xFFu;
  const uint32_t mx = xb & 0x7FFFFFu;
  const uint32_t m = ex == 0u ? mx : (mx | 0x800000u);           // |x| = m * 2^k
  const int k = (ex == 0u ? -149 : (int)ex - 150) - e;            // |y| = m * 2^k
  const int nb = 32 - mx_clz32(m | 1u);                           // m in [2^(nb-1), 2^nb)
  const int ey = nb - 1 + k;                                      // floor(log2 |y|)
  // normal: 1 + 3 fraction bits; a rounding carry (q = 16) moves into the exponent
  const uint32_t qn = mx_rne_shr(m, nb - 4);
  const uint32_t cn = (uint32_t)(ey + 7) * 8u + (qn - 8u);
  // subnormal: units of 2^-9 (q = 8 is the smallest normal, code 0x08)
  const uint32_t cs = mx_rne_shr(m, -(k + 9));
  const uint32_t code = ey >= -6 ? cn : cs;
  return sign | (m == 0u ? 0u : code);
}

// bfloat16 bits of a float32, round to nearest even (NaN kept quiet).
MX_HD uint32_t mx_bf16_bits(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
