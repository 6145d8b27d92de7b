// k_ns.hip -- Newton-Schulz (f1) on gfx950 bf16 matrix cores, with f2 fused
// into the last product.
//
// [SS-HSDP §3.1 EG1]: f1 applies Newton-Schulz to the BF16 intermediate u and
// produces the FP32 update direction; f2 updates the main weight from it.
// [SS-HSDP §4.1]: f1 groups matrices of matching shape and layout into batched
// GEMMs.  The quintic iteration (five steps, a = 3.4445, b = -4.7750,
// c = 2.0315, on the Frobenius-normalised u) is the tiny attention block's
// stated setting:
//     A = X X^T;  B = b A + c A A;  X <- a X + B X.
//
// Every product here is one batched "NT" contraction O = alpha P Q^T + beta D
// with both operands K-contiguous, which is the layout the MFMA operands want:
//   Gram    A = X X^T            P = Q = X   (r x c)
//   poly    B = c A A + b A      P = Q = A   (A symmetric, so A A^T = A A)
//   update  X' = a X + B X       P = B, Q = X^T (c x r), D = X; the epilogue
//           writes X' and X'^T, the operands of the next step, so no
//           separate transpose pass exists.
// The normalisation is folded into the first step's scalars: with s =
// 1/(||u|| + eps), A0 = s^2 u u^T and X1 = s (B0 u) + a s u, so u is never
// rescaled in memory.  A tall unit is iterated on its transpose (same map:
// X (X^T X) = (X X^T) X); its own layout simply plays the role of X^T.
//
// Kernel: a TILE x TILE macro tile per workgroup of 4 waves (2 x 2), each wave
// (TILE/2)^2 as (TILE/64)^2 blocks of v_mfma_f32_32x32x16_bf16; K in steps of
// 64 through double-buffered LDS (rows padded by 16 bytes: conflict-free
// 16-byte fragment reads); fp32 accumulation; epilogue in fp32.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "mx_codec.h"

namespace sshdp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const uint16_t *P, *Q, *D;
  uint16_t *O, *OT;
  int64_t sP, sQ, sD, sO, sOT;     // batch strides (elements)
  int M, N, K;                     // P: M x K, Q: N x K, D/O: M x N, OT: N x M
  float alpha, beta;
  const float *uscale;             // per-unit 1/(||u|| + eps)
  int alpha_pow, beta_pow;         // alpha *= s^alpha_pow, beta *= s^beta_pow
  int unit_base;                   // batch b <-> unit unit_base + b
  const MuonUnit *units;           // FINAL: the units' views into w
  float *w;
  float lr, decay;                 // FINAL: w <- w*decay - lr*scale*x
};

__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f_to_bf16(float x) { return (uint16_t)mx_bf16_bits(__float_as_uint(x)); }

// One BK = 64 slice of the macro tile from LDS: 4 K-steps of 16, each
// MB A fragments and MB B fragments (16 bytes per lane) and MB*MB MFMAs.
template <int MB, int PITCH, int OPS>
__device__ __forceinline__ void mma_step(const uint16_t *__restrict__ s, int fa, int fb, f32x16_t (&acc)[MB][MB]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t af[MB], bfr[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) af[i] = *reinterpret_cast<const bf16x8_t *>(&s[fa + i * 32 * PITCH + kk * 16]);
#pragma unroll
    for (int j = 0; j < MB; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t *>(&s[OPS + fb + j * 32 * PITCH + kk * 16]);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

template <int TILE, bool FINAL>
__global__ __launch_bounds__(256, 1) void k_gemm_nt(GemmArgs a) {
  constexpr int BK = 64, PITCH = BK + 8;             // LDS row: 64 bf16 + 16 bytes of padding
  constexpr int WT = TILE / 2, MB = WT / 32;         // wave tile, 32x32 blocks per wave edge
  constexpr int LPT = TILE * BK / 8 / 256;           // 16-byte loads per thread per operand
  constexpr int OPS = TILE * PITCH;                  // one operand tile in LDS (elements)
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * OPS];   // [buf][A|B]

  const int b = blockIdx.y;
  const int tiles_n = a.N / TILE;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t K = a.K;

  // global -> LDS copy: thread t moves rows (t>>3) + 32 i, 16 bytes at column (t&7)*8
  const uint16_t *gA = a.P + b * a.sP + ((int64_t)tm * TILE + (t >> 3)) * K + (t & 7) * 8;
  const uint16_t *gB = a.Q + b * a.sQ + ((int64_t)tn * TILE + (t >> 3)) * K + (t & 7) * 8;
  const int sofs = (t >> 3) * PITCH + (t & 7) * 8;
  // fragment reads: lane holds row (lane&31) of a 32-row block, 8 K-values at (lane>>5)*8
  const int fa = (wm * WT + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const int fb = (wn * WT + (lane & 31)) * PITCH + (lane >> 5) * 8;

  f32x16_t acc[MB][MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 ra[LPT], rb[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    ra[i] = *reinterpret_cast<const uint4 *>(gA + (int64_t)i * 32 * K);
    rb[i] = *reinterpret_cast<const uint4 *>(gB + (int64_t)i * 32 * K);
  }
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    *reinterpret_cast<uint4 *>(&smem[sofs + i * 32 * PITCH]) = ra[i];
    *reinterpret_cast<uint4 *>(&smem[OPS + sofs + i * 32 * PITCH]) = rb[i];
  }
  __syncthreads();

  const int nk = a.K / BK;
  int cur = 0;
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int64_t k0 = (int64_t)(kt + 1) * BK;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      ra[i] = *reinterpret_cast<const uint4 *>(gA + (int64_t)i * 32 * K + k0);
      rb[i] = *reinterpret_cast<const uint4 *>(gB + (int64_t)i * 32 * K + k0);
    }
    mma_step<MB, PITCH, OPS>(smem + cur, fa, fb, acc);
    const int nxt = 2 * OPS - cur;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      *reinterpret_cast<uint4 *>(&smem[nxt + sofs + i * 32 * PITCH]) = ra[i];
      *reinterpret_cast<uint4 *>(&smem[nxt + OPS + sofs + i * 32 * PITCH]) = rb[i];
    }
    __syncthreads();
    cur = nxt;
  }
  mma_step<MB, PITCH, OPS>(smem + cur, fa, fb, acc);

  // ---- epilogue: element (m, n) of a 32x32 block sits in lane n + 32*((m/4)%2),
  // register (m/8)*4 + m%4; each lane holds 4 consecutive rows of one column.
  float alpha = a.alpha, beta = a.beta;
  const int unit = a.unit_base + b;
  if (a.alpha_pow | a.beta_pow) {
    const float s = a.uscale[unit];
    if (a.alpha_pow == 1) alpha *= s;
    if (a.alpha_pow == 2) alpha *= s * s;
    if (a.beta_pow == 1) beta *= s;
  }
  const uint16_t *D = a.D ? a.D + b * a.sD : nullptr;
  uint16_t *O = a.O ? a.O + b * a.sO : nullptr;
  uint16_t *OT = a.OT ? a.OT + b * a.sOT : nullptr;
  MuonUnit u{};
  int r_unit = 0, c_unit = 0;
  if (FINAL) {
    u = a.units[unit];
    r_unit = u.tall ? u.cols : u.rows;
    c_unit = u.tall ? u.rows : u.cols;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int col = tn * TILE + wn * WT + j * 32 + (lane & 31);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int row0 = tm * TILE + wm * WT + i * 32 + g4 * 8 + (lane >> 5) * 4;
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = alpha * acc[i][j][g4 * 4 + q];
        if (D) {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = fmaf(beta, bf16_to_f(D[(int64_t)(row0 + q) * a.N + col]), x[q]);
        }
        if (!FINAL) {
          uint16_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            h[q] = f_to_bf16(x[q]);
            O[(int64_t)(row0 + q) * a.N + col] = h[q];
          }
          if (OT) {
            uint2 pk;
            pk.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            pk.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            *reinterpret_cast<uint2 *>(OT + (int64_t)col * a.M + row0) = pk;
          }
        } else if (col < c_unit) {
          const float ls = a.lr * u.upd_scale;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = row0 + q;
            if (row < r_unit) {
              const int64_t idx = u.tall ? u.abs + (int64_t)col * u.row_stride + row
                                         : u.abs + (int64_t)row * u.row_stride + col;
              a.w[idx] = fmaf(a.w[idx], a.decay, -ls * x[q]);
            }
          }
        }
      }
    }
  }
}

template <int TILE, bool FINAL>
hipError_t launch(const GemmArgs &a, int batch, hipStream_t s) {
  const dim3 grid((unsigned)((a.M / TILE) * (a.N / TILE)), (unsigned)batch);
  hipLaunchKernelGGL((k_gemm_nt<TILE, FINAL>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t dispatch(const GemmArgs &a, int batch, int tile, bool final_, hipStream_t s) {
  if (tile == 128) return final_ ? launch<128, true>(a, batch, s) : launch<128, false>(a, batch, s);
  if (tile == 256) return final_ ? launch<256, true>(a, batch, s) : launch<256, false>(a, batch, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ns_stage(const sshdp_plan &p, const Group &g, int stage, int iter, char *ws, float *w_main,
                           float lr, float wd, hipStream_t s) {
  uint16_t *X = reinterpret_cast<uint16_t *>(ws + g.off_x);
  uint16_t *XT[2] = {reinterpret_cast<uint16_t *>(ws + g.off_xt0), reinterpret_cast<uint16_t *>(ws + g.off_xt1)};
  uint16_t *A = reinterpret_cast<uint16_t *>(ws + g.off_a);
  uint16_t *B = reinterpret_cast<uint16_t *>(ws + g.off_b);
  const int64_t sx = (int64_t)g.r_pad * g.c_pad, sa = (int64_t)g.r_pad * g.r_pad;
  GemmArgs a{};
  a.uscale = reinterpret_cast<const float *>(ws + p.ws_uscale);
  a.unit_base = g.unit_base;
  a.units = p.d.munits;
  a.w = w_main;
  a.lr = lr;
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  if (stage == 0) {                       // A = alpha X X^T
    a.P = a.Q = X; a.sP = a.sQ = sx;
    a.O = A; a.sO = sa;
    a.M = a.N = g.r_pad; a.K = g.c_pad;
    a.alpha = 1.f; a.alpha_pow = iter == 0 ? 2 : 0;
  } else if (stage == 1) {                // B = c A A + b A
    a.P = a.Q = A; a.sP = a.sQ = sa;
    a.D = A; a.sD = sa;
    a.O = B; a.sO = sa;
    a.M = a.N = a.K = g.r_pad;
    a.alpha = p.opts.ns_c; a.beta = p.opts.ns_b;
  } else {                                // X' = alpha B X + beta X
    a.P = B; a.sP = sa;
    a.Q = XT[iter & 1]; a.sQ = sx;
    a.D = X; a.sD = sx;
    if (stage == 2) {
      a.O = X; a.sO = sx;
      a.OT = XT[(iter + 1) & 1]; a.sOT = sx;
    }
    a.M = g.r_pad; a.N = g.c_pad; a.K = g.r_pad;
    a.alpha = 1.f; a.beta = p.opts.ns_a;
    a.alpha_pow = a.beta_pow = iter == 0 ? 1 : 0;
  }
  return dispatch(a, g.n, g.tile, stage == 3, s);
}

hipError_t launch_gemm_raw(const void *P, const void *Q, const void *D, void *O, void *OT, int M, int N, int K,
                           int batch, float alpha, float beta, int tile, hipStream_t s) {
  GemmArgs a{};
  a.P = static_cast<const uint16_t *>(P);
  a.Q = static_cast<const uint16_t *>(Q);
  a.D = static_cast<const uint16_t *>(D);
  a.O = static_cast<uint16_t *>(O);
  a.OT = static_cast<uint16_t *>(OT);
  a.sP = (int64_t)M * K;
  a.sQ = (int64_t)N * K;
  a.sD = a.sO = a.sOT = (int64_t)M * N;
  a.M = M; a.N = N; a.K = K;
  a.alpha = alpha; a.beta = beta;
  return dispatch(a, batch, tile, false, s);
}

}  // namespace sshdp
