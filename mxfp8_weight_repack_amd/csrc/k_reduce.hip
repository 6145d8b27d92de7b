// k_reduce.hip -- the reduce-scatter tail: FP32 reduction of the slices that
// arrive for one output partition, BF16 partials with stochastic rounding, and
// the final reduction straight into the persistent FP32 accumulation buffer.
//
// [SS-HSDP §4.3 "Reduce-Scatter", Figure 5(e)]: a local reducer sums the
// intra-node contributions in FP32; for BF16 gradients the partial is stored
// as BF16 with stochastic rounding; the final FP32 reduction accumulates into
// G'z2 itself, so there is no result buffer and no separate addition pass.
// On one GPU the slices are device buffers (what peer copies would deliver).
//
// Summation: inputs left to right, each addition rounded to FP32.  SR: the
// fp32 bit pattern plus a 16-bit random, truncated to the upper half (NaN kept
// quiet): away from zero with probability (discarded bits) / 2^16.  Randoms:
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011) with key (seed, 0) and counter (g/16 + 1, ctr, 0, 0)
// for element g of the whole tensor; word (g/4) % 4, bits 16*(g%4).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace sshdp {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct Philox4x64 {
  uint64_t x[4];
};

// Philox4x64-10 block: ten rounds of two 64x64 -> 128-bit products with the
// published multipliers, the key bumped by the published Weyl constants.
__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t a = c0, b = c1, c = 0, d = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, a), lo0 = M0 * a;
    const uint64_t hi1 = __umul64hi(M1, c), lo1 = M1 * c;
    const uint64_t na = hi1 ^ b ^ k0, nb = lo1, nc = hi0 ^ d ^ k1, nd = lo0;
    a = na; b = nb; c = nc; d = nd;
    k0 += W0;
    k1 += W1;
  }
  return {{a, b, c, d}};
}

struct RsArgs {
  const void *in[kRsMaxInputs];
  int n_in;
  int first;                 // accumulate: the first microbatch initialises g
  int64_t n;                 // elements (multiple of 16)
  uint64_t seed, ctr;
  int64_t g0;                // index of element 0 in the whole tensor (multiple of 16)
};

// The 16 consecutive elements at e of every input, summed left to right in
// fp32 (init: acc starts from input 0, else from acc).  All inputs' loads are
// issued before the first addition.
template <bool BF16>
__device__ __forceinline__ void sum_inputs(const RsArgs &a, int64_t e, float (&acc)[16], bool init) {
  constexpr int W = BF16 ? 2 : 4;                    // 16-byte words per input
  u32x4_t raw[kRsMaxInputs][W];
#pragma unroll
  for (int k = 0; k < kRsMaxInputs; ++k) {
    if (k < a.n_in) {
      const u32x4_t *q = BF16 ? reinterpret_cast<const u32x4_t *>(static_cast<const uint16_t *>(a.in[k]) + e)
                              : reinterpret_cast<const u32x4_t *>(static_cast<const float *>(a.in[k]) + e);
#pragma unroll
      for (int h = 0; h < W; ++h) raw[k][h] = __builtin_nontemporal_load(q + h);
    }
  }
#pragma unroll
  for (int k = 0; k < kRsMaxInputs; ++k) {
    if (k < a.n_in) {
      float v[16];
#pragma unroll
      for (int h = 0; h < W; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (BF16) {
            v[8 * h + 2 * j] = __uint_as_float(raw[k][h][j] << 16);
            v[8 * h + 2 * j + 1] = __uint_as_float(raw[k][h][j] & 0xFFFF0000u);
          } else {
            v[4 * h + j] = __uint_as_float(raw[k][h][j]);
          }
        }
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = (init && k == 0) ? v[j] : acc[j] + v[j];
    }
  }
}

template <bool IN_BF16, bool OUT_SR>
__global__ __launch_bounds__(256) void k_rs_reduce(RsArgs a, void *out) {
  const int64_t groups = a.n / 16;
  for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = gi * 16;
    float acc[16];
    sum_inputs<IN_BF16>(a, e, acc, true);
    if (!OUT_SR) {
      f32x4_t *o = reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + e);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4_t w = {acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
        __builtin_nontemporal_store(w, o + h);
      }
    } else {
      const Philox4x64 r = philox4x64_10((uint64_t)((a.g0 + e) / 16) + 1, a.ctr, a.seed, 0);
      uint32_t h16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t u = __float_as_uint(acc[j]);
        const uint32_t rnd = (uint32_t)(r.x[j / 4] >> (16 * (j % 4))) & 0xFFFFu;
        h16[j] = (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : ((u + rnd) >> 16);
      }
      u32x4_t *o = reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(out) + e);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t w = {h16[8 * h] | (h16[8 * h + 1] << 16), h16[8 * h + 2] | (h16[8 * h + 3] << 16),
                           h16[8 * h + 4] | (h16[8 * h + 5] << 16), h16[8 * h + 6] | (h16[8 * h + 7] << 16)};
        __builtin_nontemporal_store(w, o + h);
      }
    }
  }
}

template <bool IN_BF16>
__global__ __launch_bounds__(256) void k_rs_accumulate(RsArgs a, float *g) {
  const int64_t groups = a.n / 16;
  for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = gi * 16;
    float acc[16];
    if (!a.first) {
      const f32x4_t *q = reinterpret_cast<const f32x4_t *>(g + e);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4_t w = q[h];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * h + j] = w[j];
      }
    }
    sum_inputs<IN_BF16>(a, e, acc, a.first != 0);
    f32x4_t *o = reinterpret_cast<f32x4_t *>(g + e);
#pragma unroll
    for (int h = 0; h < 4; ++h) o[h] = f32x4_t{acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
  }
}

RsArgs rs_args(const void *const *inputs, int n_in, int64_t n, uint64_t seed, uint64_t ctr, int64_t g0, int first) {
  RsArgs a{};
  for (int k = 0; k < n_in; ++k) a.in[k] = inputs[k];
  a.n_in = n_in;
  a.first = first;
  a.n = n;
  a.seed = seed;
  a.ctr = ctr;
  a.g0 = g0;
  return a;
}

unsigned rs_grid(int64_t n) {
  const int64_t groups = n / 16, blocks = (groups + 255) / 256;
  return (unsigned)std::min<int64_t>(std::max<int64_t>(blocks, 1), 1 << 20);
}

}  // namespace

hipError_t launch_rs_reduce(const void *const *inputs, int n_in, int in_bf16, void *out, int out_sr, int64_t n,
                            uint64_t seed, uint64_t ctr, int64_t g0, hipStream_t s) {
  const RsArgs a = rs_args(inputs, n_in, n, seed, ctr, g0, 1);
  const dim3 grid(rs_grid(n)), block(256);
  if (in_bf16 && out_sr) hipLaunchKernelGGL((k_rs_reduce<true, true>), grid, block, 0, s, a, out);
  else if (in_bf16) hipLaunchKernelGGL((k_rs_reduce<true, false>), grid, block, 0, s, a, out);
  else if (out_sr) hipLaunchKernelGGL((k_rs_reduce<false, true>), grid, block, 0, s, a, out);
  else hipLaunchKernelGGL((k_rs_reduce<false, false>), grid, block, 0, s, a, out);
  return hipGetLastError();
}

hipError_t launch_rs_accumulate(const void *const *inputs, int n_in, int in_bf16, float *g, int64_t n, int first,
                                hipStream_t s) {
  const RsArgs a = rs_args(inputs, n_in, n, 0, 0, 0, first);
  const dim3 grid(rs_grid(n)), block(256);
  if (in_bf16) hipLaunchKernelGGL((k_rs_accumulate<true>), grid, block, 0, s, a, g);
  else hipLaunchKernelGGL((k_rs_accumulate<false>), grid, block, 0, s, a, g);
  return hipGetLastError();
}

}  // namespace sshdp
