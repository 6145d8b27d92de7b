// mx_device.h -- device-side MXFP8 pieces of the G kernels (1 x 32 blocks,
// with or without AdamW fused in front).
//
// A lane owns 4 consecutive elements of a row and 8 consecutive lanes (aligned
// to 8) one 32-element block along K.  The block amax is an integer max of the
// |x| bit patterns (which also ranks NaN above Inf) over those 8 lanes; the
// scale byte comes from mx_scale_byte (mx_codec.h); the codes are the hardware
// E4M3FN conversion (round to nearest even) of x * 2^-e, which is exact down to
// 2^-126 -- anything smaller encodes as a signed zero either way.  The
// conversion matches the integer encoder mx_e4m3_code for every finite
// |y| <= 448 (checked exhaustively on the device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_codec.h"

namespace sshdp {

// Block amax bits over 8 aligned lanes.  Every lane of the wave must call it.
__device__ __forceinline__ uint32_t mx_amax8(const float4 &v) {
  uint32_t a = max(max(__float_as_uint(v.x) & 0x7FFFFFFFu, __float_as_uint(v.y) & 0x7FFFFFFFu),
                   max(__float_as_uint(v.z) & 0x7FFFFFFFu, __float_as_uint(v.w) & 0x7FFFFFFFu));
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  a = max(a, (uint32_t)__shfl_xor((int)a, 4));
  return a;
}

// The four E4M3FN codes of v under scale byte sb, packed little-endian.
__device__ __forceinline__ uint32_t mx_encode4(const float4 &v, uint32_t sb) {
  if (sb == 0xFFu) return 0x7F7F7F7Fu;               // a block holding NaN/Inf
  const int ex = 127 - (int)sb;
  int pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v.x, ex), ldexpf(v.y, ex), 0, false);
  pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v.z, ex), ldexpf(v.w, ex), pk, true);
  return (uint32_t)pk;
}

// TILE32X4 scale index of block (n, kb) of a region at element offset `abs`
// with KB = cols/32 blocks per row.
__device__ __forceinline__ int64_t mx_tile32x4_index(int64_t abs, int64_t KB, int64_t n, int64_t kb) {
  return (abs >> 5) + ((n >> 5) * (KB >> 2) + (kb >> 2)) * 128 + (n & 31) * 4 + (kb & 3);
}

}  // namespace sshdp
