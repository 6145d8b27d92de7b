// lds_swizzle.h -- 16-byte chunk swizzle of the contraction's LDS operand rows.
//
// A stage holds rows of BK bf16 (128 bytes for BK = 64, 64 bytes for BK = 32);
// logical chunk c of row r sits at physical chunk c ^ lds_swz<BK>(r).  A
// fragment read has lanes 0..31 on 32 consecutive rows at one logical chunk
// (lanes 32..63 on the next chunk); with the swizzle every aligned group of 8
// and of 16 such lanes hits distinct 16-byte bank groups.  The pattern repeats
// every 32 (BK = 64) or 16 (BK = 32) rows, so each buffer load -- which fills 8
// or 16 whole rows -- needs a single per-lane pattern.  Host-compilable so the
// properties can be checked on the CPU.
#pragma once

#if defined(__HIPCC__)
#define LDS_HD __host__ __device__ __forceinline__
#else
#define LDS_HD static inline
#endif

template <int BK>
LDS_HD int lds_swz(int r) {
  if (BK == 64) return ((r & 31) ^ ((r & 31) >> 3)) & 7;
  return (((r & 15) >> 1) ^ ((r & 15) >> 3)) & 3;
}
