// k_elementwise.hip -- the HBM-streaming stages of the update phase on gfx950:
//   f0   Muon momentum + bf16 u (own layout and transposed) + ||u||^2 partials
//   norm per-unit 1 / (||u||_F + eps), deterministic reduction of the partials
//   AdamW for elementwise units
//   G    MXFP8 requantisation (1x32 blocks along K), optionally fused with AdamW
//
// [SS-HSDP §3.1 EG1]: f0 updates the momentum from the gradient and writes a
// BF16 intermediate u; G quantises the main weight to FP8 with UE8M0 scales and
// Tw relays the scales out for the GEMM.  [SS-HSDP §4.1]: the elementwise
// stages run as multi-tensor kernels over all units in one launch.  [OCP-MX]:
// one E8M0 scale per 32-element block, E4M3 elements.
//
// Memory access: every global access is a 16-byte vector per lane with
// consecutive lanes on consecutive addresses (8 lanes = one 128-byte MX block);
// block amax is an 8-lane butterfly over the lanes holding the block.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "internal.h"
#include "mx_codec.h"
#include "mx_device.h"

namespace sshdp {
namespace {

__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bfloat16 (a in the low half), v_cvt_pk_bf16_f32: round
// to nearest even, identical to mx_bf16_bits for every non-NaN float32
// (checked exhaustively on the device).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Streaming accesses that are not kept in the caches: every element of the
// AdamW/requant passes is read once and written once.  On the flat 5e8-element
// shard, nontemporal loads and stores of w, m, v (not only g and the codes)
// took the fused pass from 62% to 70% of HBM peak.
__device__ __forceinline__ float4 load_nt(const float *p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(float *p, const float4 &v) {
  __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t *>(p));
}

// ----------------------------------------------------------------------------- f0
// One 64x64 tile of a Muon unit's own (padded) layout per workgroup of 256.
// Elements outside the unit write u = 0 (the padding the GEMMs rely on).
__global__ __launch_bounds__(256) void k_f0(const MuonUnit *__restrict__ units, const F0Tile *__restrict__ tiles,
                                            const float *__restrict__ g, float *__restrict__ m, float mu,
                                            int nesterov, char *__restrict__ ws, float *__restrict__ partials) {
  constexpr int T = kF0Tile, PITCH = T + 8;          // bf16 elements; rows 16-byte aligned
  __shared__ uint16_t lds[T * PITCH];
  __shared__ float red[4];
  const F0Tile tl = tiles[blockIdx.x];
  const MuonUnit u = units[tl.unit];
  const int t = threadIdx.x;
  const int cq = t & 15, r0 = t >> 4;
  const int col = tl.tc * T + cq * 4;
  // either copy may be absent (-1): groups whose Gram reads X^T keep only u^T
  uint16_t *orig = u.ws_orig >= 0 ? reinterpret_cast<uint16_t *>(ws + u.ws_orig) : nullptr;
  uint16_t *trans = u.ws_trans >= 0 ? reinterpret_cast<uint16_t *>(ws + u.ws_trans) : nullptr;
  // all eight 16-byte loads first, so each lane has them in flight together
  float4 gvs[4], mvs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = tl.tr * T + r0 + 16 * i;
    if (row < u.rows && col < u.cols) {
      const int64_t e = u.abs + (int64_t)row * u.row_stride + col;
      gvs[i] = load_nt(g + e);
      mvs[i] = load_nt(m + e);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = r0 + 16 * i;
    const int row = tl.tr * T + lr;
    uint32_t b[4] = {0u, 0u, 0u, 0u};
    if (row < u.rows && col < u.cols) {
      const int64_t e = u.abs + (int64_t)row * u.row_stride + col;
      const float4 gv = gvs[i];
      float4 mv = mvs[i];
      mv.x = fmaf(mu, mv.x, gv.x);
      mv.y = fmaf(mu, mv.y, gv.y);
      mv.z = fmaf(mu, mv.z, gv.z);
      mv.w = fmaf(mu, mv.w, gv.w);
      store_nt(m + e, mv);
      float4 src = mv;
      if (nesterov) {
        src.x = fmaf(mu, mv.x, gv.x);
        src.y = fmaf(mu, mv.y, gv.y);
        src.z = fmaf(mu, mv.z, gv.z);
        src.w = fmaf(mu, mv.w, gv.w);
      }
      b[0] = mx_bf16_bits(fbits(src.x));
      b[1] = mx_bf16_bits(fbits(src.y));
      b[2] = mx_bf16_bits(fbits(src.z));
      b[3] = mx_bf16_bits(fbits(src.w));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float q = __uint_as_float(b[j] << 16);
        ss = fmaf(q, q, ss);
      }
    }
    uint2 packed;
    packed.x = b[0] | (b[1] << 16);
    packed.y = b[2] | (b[3] << 16);
    if (orig) *reinterpret_cast<uint2 *>(orig + (int64_t)row * u.Cp + col) = packed;
    if (trans) {
#pragma unroll
      for (int j = 0; j < 4; ++j) lds[(cq * 4 + j) * PITCH + lr] = (uint16_t)b[j];
    }
  }
  // sum of squares: wave butterfly, then the 4 waves in order (deterministic)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  if (t == 0) partials[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
  // transposed tile: row c of the transpose = column c of the tile
  if (!trans) return;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = (t >> 3) + 32 * pass, seg = t & 7;
    const uint4 v = *reinterpret_cast<const uint4 *>(&lds[c * PITCH + seg * 8]);
    *reinterpret_cast<uint4 *>(trans + (int64_t)(tl.tc * T + c) * u.Rp + tl.tr * T + seg * 8) = v;
  }
}

// ----------------------------------------------------------------------------- norm
// One workgroup per unit sums the unit's f0 partials in a fixed order: thread t
// keeps kNormUnroll running sums (partials t + kNormThreads*(kNormUnroll*j + k)),
// so each thread has that many loads in flight, then the sums, the wave
// butterfly and the waves are combined in order (bit-reproducible).
constexpr int kNormThreads = 1024, kNormUnroll = 8;
__global__ __launch_bounds__(kNormThreads) void k_norm(const MuonUnit *__restrict__ units,
                                                       const int32_t *__restrict__ ulist,
                                                       const float *__restrict__ partials,
                                                       float *__restrict__ uscale, float eps) {
  constexpr int NW = kNormThreads / 64;
  __shared__ float red[NW];
  const int32_t ui = ulist[blockIdx.x];
  const MuonUnit u = units[ui];
  const int t = threadIdx.x, n = u.tile_end - u.tile_begin;
  const float *pp = partials + u.tile_begin;
  float acc[kNormUnroll];
#pragma unroll
  for (int k = 0; k < kNormUnroll; ++k) acc[k] = 0.f;
  for (int base = 0; base < n; base += kNormThreads * kNormUnroll) {
#pragma unroll
    for (int k = 0; k < kNormUnroll; ++k) {
      const int i = base + k * kNormThreads + t;
      if (i < n) acc[k] += pp[i];
    }
  }
#pragma unroll
  for (int w = kNormUnroll / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int k = 0; k < w; ++k) acc[k] = acc[2 * k] + acc[2 * k + 1];
  float s = acc[0];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
#pragma unroll
    for (int w = NW / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int k = 0; k < w; ++k) red[k] = red[2 * k] + red[2 * k + 1];
    const float tot = red[0];
    // an all-zero unit gets scale 0: its Newton-Schulz products are skipped (direction exactly 0)
    uscale[ui] = tot > 0.f ? 1.0f / (sqrtf(tot) + eps) : 0.f;
  }
}

// ----------------------------------------------------------------------------- AdamW
// Constants in float64, from the float32 hyper-parameters the ABI receives.
struct AdamConst {
  double b1, b2, omb1, omb2;      // beta1, beta2, 1-beta1, 1-beta2
  double lrwd, lr, eps;           // lr*wd, lr, eps
  double rbc1, rbc2;              // 1/(1-b1^t), 1/(1-b2^t)
};

// 1/d: the hardware reciprocal refined by one Newton step (relative error far
// below the float32 rounding of the result).
__device__ __forceinline__ double rcp64(double d) {
  const double r = __builtin_amdgcn_rcp(d);
  return fma(r, fma(-d, r, 1.0), r);
}

// w <- w - lr*wd*w; m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
// w <- w - lr (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps), in float64 on the
// float32 state, each result rounded once to float32.  Float32 arithmetic lands
// several float32 ulps of the step from the exact update (its roundings of m,
// v, the square root and the quotient add up); in float64 the only error left
// is the final rounding.  The pass stays bound by memory: the float64 work is
// ~20 vector instructions per element against 29 bytes of traffic.
__device__ __forceinline__ void adam_elem(float &w, float g, float &m, float &v, const AdamConst &c) {
  const double wd = w, gd = g;
  const double md = fma(c.b1, (double)m, c.omb1 * gd);
  const double vd = fma(c.b2, (double)v, c.omb2 * (gd * gd));
  const double den = __builtin_sqrt(vd * c.rbc2) + c.eps;
  const double wn = fma(-c.lrwd, wd, wd);
  w = (float)fma(-c.lr * (md * c.rbc1), rcp64(den), wn);
  m = (float)md;
  v = (float)vd;
}

__global__ __launch_bounds__(256) void k_adamw(const ASeg *__restrict__ segs, float *__restrict__ w,
                                               const float *__restrict__ g, float *__restrict__ m,
                                               float *__restrict__ v, AdamConst c) {
  const ASeg s = segs[blockIdx.x];
  const int t = threadIdx.x;
  if ((s.base & 3) == 0) {
    const int nv = s.n >> 2;
    for (int i = t; i < nv; i += 256) {
      const int64_t e = s.base + 4 * (int64_t)i;
      float4 wv = load_nt(w + e);
      const float4 gv = load_nt(g + e);
      float4 mv = load_nt(m + e);
      float4 vv = load_nt(v + e);
      adam_elem(wv.x, gv.x, mv.x, vv.x, c);
      adam_elem(wv.y, gv.y, mv.y, vv.y, c);
      adam_elem(wv.z, gv.z, mv.z, vv.z, c);
      adam_elem(wv.w, gv.w, mv.w, vv.w, c);
      store_nt(w + e, wv);
      store_nt(m + e, mv);
      store_nt(v + e, vv);
    }
    for (int i = 4 * nv + t; i < s.n; i += 256) {
      const int64_t e = s.base + i;
      float wv = w[e], mv = m[e], vv = v[e];
      adam_elem(wv, g[e], mv, vv, c);
      w[e] = wv; m[e] = mv; v[e] = vv;
    }
  } else {
    for (int i = t; i < s.n; i += 256) {
      const int64_t e = s.base + i;
      float wv = w[e], mv = m[e], vv = v[e];
      adam_elem(wv, g[e], mv, vv, c);
      w[e] = wv; m[e] = mv; v[e] = vv;
    }
  }
}

// ----------------------------------------------------------------------------- G (+ AdamW)
// Quantise 4 elements per lane (8 lanes = one 32-element block) and store
// their codes and the block's scale byte.  All 64 lanes must call it (the
// block amax is a butterfly over lane groups of 8); `live` masks the stores.
__device__ __forceinline__ void quant_store(const float4 &wv, int64_t e, bool live, int t, const QChunk &q,
                                            const QRegion *__restrict__ regions, int tile_layout,
                                            uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const uint32_t a = mx_amax8(wv);
  if (!live) return;
  const uint32_t sb = mx_scale_byte(a);
  __builtin_nontemporal_store(mx_encode4(wv, sb), reinterpret_cast<uint32_t *>(codes + e));
  if ((t & 7) == 0) {
    int64_t idx = e >> 5;
    if (tile_layout) {
      // element e sits (e - base) < kChunk past the chunk's first element, whose
      // region row/column the planner stored: a 32-bit division by the row length
      const QRegion r = regions[q.region];
      const uint32_t col = (uint32_t)q.col0 + (uint32_t)(e - q.base);
      const uint32_t dn = col / (uint32_t)r.cols;
      idx = mx_tile32x4_index(r.abs, r.cols >> 5, (int64_t)q.row0 + dn, (col - dn * (uint32_t)r.cols) >> 5);
    }
    scales[idx] = (uint8_t)sb;
  }
}

// One chunk (<= kChunk elements, whole 32-blocks) per workgroup; four passes of
// 1024 elements, each lane owning 4 consecutive elements, 8 lanes per block.
// All loads of a chunk are issued before any arithmetic.  A chunk that is full
// and (when fused) wholly AdamW-updated takes a branch-free path; the others
// (region tails, runs that start or end inside the chunk) mask per element.
template <bool FUSED>
__global__ __launch_bounds__(256) void k_quant(const QChunk *__restrict__ chunks, const QRegion *__restrict__ regions,
                                               int tile_layout, float *__restrict__ w, const float *__restrict__ g,
                                               float *__restrict__ m, float *__restrict__ v,
                                               uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                               AdamConst c) {
  constexpr int P = kChunk / 1024;
  const QChunk q = chunks[blockIdx.x];
  const int t = threadIdx.x;
  float4 wv[P], gv[P], mv[P], vv[P];
  const bool full = q.n == kChunk && (!FUSED || (q.lo <= q.base && q.hi >= q.base + kChunk));
  if (full) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t e = q.base + p * 1024 + 4 * t;
      wv[p] = load_nt(w + e);
      if (FUSED) {
        gv[p] = load_nt(g + e);
        mv[p] = load_nt(m + e);
        vv[p] = load_nt(v + e);
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int64_t e = q.base + p * 1024 + 4 * t;
      if (FUSED) {
        adam_elem(wv[p].x, gv[p].x, mv[p].x, vv[p].x, c);
        adam_elem(wv[p].y, gv[p].y, mv[p].y, vv[p].y, c);
        adam_elem(wv[p].z, gv[p].z, mv[p].z, vv[p].z, c);
        adam_elem(wv[p].w, gv[p].w, mv[p].w, vv[p].w, c);
        store_nt(w + e, wv[p]);
        store_nt(m + e, mv[p]);
        store_nt(v + e, vv[p]);
      }
      quant_store(wv[p], e, true, t, q, regions, tile_layout, codes, scales);
    }
    return;
  }
  bool live[P], upd[P];
#pragma unroll
  for (int p = 0; p < P; ++p) wv[p] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int off = p * 1024 + 4 * t;
    const int64_t e = q.base + off;
    live[p] = off < q.n;
    upd[p] = FUSED && live[p] && e + 4 > q.lo && e < q.hi;
    if (live[p]) wv[p] = *reinterpret_cast<const float4 *>(w + e);
    if (upd[p]) {
      gv[p] = load_nt(g + e);
      mv[p] = *reinterpret_cast<const float4 *>(m + e);
      vv[p] = *reinterpret_cast<const float4 *>(v + e);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t e = q.base + p * 1024 + 4 * t;
    if (FUSED && upd[p]) {
      float *wp = reinterpret_cast<float *>(&wv[p]);
      const float *gp = reinterpret_cast<const float *>(&gv[p]);
      float *mp = reinterpret_cast<float *>(&mv[p]);
      float *vp = reinterpret_cast<float *>(&vv[p]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (e + j >= q.lo && e + j < q.hi) {
          adam_elem(wp[j], gp[j], mp[j], vp[j], c);
          w[e + j] = wp[j];
          m[e + j] = mp[j];
          v[e + j] = vp[j];
        }
      }
    }
    quant_store(wv[p], e, live[p], t, q, regions, tile_layout, codes, scales);
  }
}

// G with one scale per 32 x 32 block.  A workgroup takes one tile: 32 rows of
// up to 4 blocks (128 columns).  Lane t owns 4 consecutive columns (4*(t%32))
// of rows t/32 + 8p, p = 0..3, so a row of the tile is 32 lanes x 16 bytes.
// The block amax: a lane's 16 values, then lanes of the same block and row
// group (xor 1, 2, 4), then the two row groups of a wave (xor 32), then the 4
// waves through LDS.  Codes as in k_quant (hardware E4M3FN convert of the
// exactly scaled value); the scale byte is written once per block.
__global__ __launch_bounds__(256) void k_quant32(const Q32Tile *__restrict__ tiles, const float *__restrict__ w,
                                                 uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  __shared__ uint32_t red[4][4];
  const Q32Tile q = tiles[blockIdx.x];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c4 = t & 31, blk = c4 >> 3, rg = t >> 5;
  const bool act = blk < q.nb;
  float4 wv[4];
  uint32_t a = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    wv[p] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) wv[p] = load_nt(w + q.base + (int64_t)(rg + 8 * p) * q.cols + 4 * c4);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
    a = max(a, max(max(fbits(wv[p].x) & 0x7FFFFFFFu, fbits(wv[p].y) & 0x7FFFFFFFu),
                   max(fbits(wv[p].z) & 0x7FFFFFFFu, fbits(wv[p].w) & 0x7FFFFFFFu)));
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  a = max(a, (uint32_t)__shfl_xor((int)a, 4));
  a = max(a, (uint32_t)__shfl_xor((int)a, 32));
  if (lane < 32 && (lane & 7) == 0) red[wave][blk] = a;
  __syncthreads();
  a = max(max(red[0][blk], red[1][blk]), max(red[2][blk], red[3][blk]));
  if (!act) return;
  const uint32_t sb = mx_scale_byte(a);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    __builtin_nontemporal_store(mx_encode4(wv[p], sb),
                                reinterpret_cast<uint32_t *>(codes + q.base + (int64_t)(rg + 8 * p) * q.cols + 4 * c4));
  if (rg == 0 && (c4 & 7) == 0) scales[q.sidx + blk] = (uint8_t)sb;
}

// G as a bfloat16 cast: one chunk (<= kChunk elements, a multiple of 8) per
// workgroup, two passes of 2048; a lane converts 8 consecutive elements
// (v_cvt_pk_bf16_f32, round to nearest even) and stores 16 bytes.
__global__ __launch_bounds__(256) void k_cast_bf16(const CChunk *__restrict__ chunks, const float *__restrict__ w,
                                                   uint16_t *__restrict__ out) {
  const CChunk q = chunks[blockIdx.x];
  const int t = threadIdx.x;
  float4 a[2], b[2];
  bool live[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int off = p * 2048 + 8 * t;
    live[p] = off < q.n;
    if (live[p]) {
      a[p] = load_nt(w + q.base + off);
      b[p] = load_nt(w + q.base + off + 4);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (!live[p]) continue;
    u32x4_t h;
    h.x = pk_bf16(a[p].x, a[p].y);
    h.y = pk_bf16(a[p].z, a[p].w);
    h.z = pk_bf16(b[p].x, b[p].y);
    h.w = pk_bf16(b[p].z, b[p].w);
    __builtin_nontemporal_store(h, reinterpret_cast<u32x4_t *>(out + q.base + p * 2048 + 8 * t));
  }
}

AdamConst adam_const(const sshdp_adamw_hp &hp, int64_t step) {
  AdamConst c;
  c.b1 = hp.beta1;
  c.b2 = hp.beta2;
  c.omb1 = 1.0 - (double)hp.beta1;
  c.omb2 = 1.0 - (double)hp.beta2;
  c.lrwd = (double)hp.lr * (double)hp.weight_decay;
  c.lr = hp.lr;
  c.eps = hp.eps;
  c.rbc1 = 1.0 / (1.0 - std::pow((double)hp.beta1, (double)step));
  c.rbc2 = 1.0 / (1.0 - std::pow((double)hp.beta2, (double)step));
  return c;
}

}  // namespace

hipError_t launch_f0(const sshdp_plan &p, int lane, const float *g, float *m, float mu, int nesterov, char *ws,
                     hipStream_t s) {
  const int32_t b = p.f0_lane[lane], n = p.f0_lane[lane + 1] - b;
  if (n <= 0) return hipSuccess;
  // the lane's tiles and their partials (partial i of the launch belongs to tile b + i)
  hipLaunchKernelGGL(k_f0, dim3((unsigned)n), dim3(256), 0, s, p.d.munits, p.d.f0tiles + b, g, m, mu, nesterov, ws,
                     reinterpret_cast<float *>(ws + p.ws_partials) + b);
  return hipGetLastError();
}

hipError_t launch_norm(const sshdp_plan &p, int lane, char *ws, float eps, hipStream_t s) {
  const int32_t b = p.norm_lane[lane], n = p.norm_lane[lane + 1] - b;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_norm, dim3((unsigned)n), dim3(kNormThreads), 0, s, p.d.munits, p.d.norm_units + b,
                     reinterpret_cast<const float *>(ws + p.ws_partials), reinterpret_cast<float *>(ws + p.ws_uscale),
                     eps);
  return hipGetLastError();
}

hipError_t launch_adamw(const ASeg *segs, int64_t nseg, const sshdp_buffers &b, const sshdp_adamw_hp &hp,
                        int64_t step, hipStream_t s) {
  if (nseg <= 0) return hipSuccess;
  const AdamConst c = adam_const(hp, step);
  for (int64_t first = 0; first < nseg; first += 0x7FFFFFFF) {
    const int64_t cnt = std::min<int64_t>(nseg - first, 0x7FFFFFFF);
    hipLaunchKernelGGL(k_adamw, dim3((unsigned)cnt), dim3(256), 0, s, segs + first, b.w_main, b.grad, b.mom,
                       b.adam_v, c);
  }
  return hipGetLastError();
}

hipError_t launch_quant(const sshdp_plan &p, int64_t first, int64_t count, bool fused, const sshdp_buffers &b,
                        const sshdp_adamw_hp *hp, int64_t step, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const AdamConst c = fused ? adam_const(*hp, step) : AdamConst{};
  const int tile = p.opts.scale_layout == SSHDP_SCALE_TILE32X4;
  if (fused)
    hipLaunchKernelGGL(k_quant<true>, dim3((unsigned)count), dim3(256), 0, s, p.d.qchunks + first, p.d.qregions, tile,
                       b.w_main, b.grad, b.mom, b.adam_v, b.codes, b.scales, c);
  else
    hipLaunchKernelGGL(k_quant<false>, dim3((unsigned)count), dim3(256), 0, s, p.d.qchunks + first, p.d.qregions,
                       tile, b.w_main, nullptr, nullptr, nullptr, b.codes, b.scales, c);
  return hipGetLastError();
}

hipError_t launch_quant32(const sshdp_plan &p, const float *w, uint8_t *codes, uint8_t *scales, hipStream_t s) {
  const int64_t n = (int64_t)p.q32tiles.size();
  for (int64_t first = 0; first < n; first += 0x7FFFFFFF) {
    const int64_t cnt = std::min<int64_t>(n - first, 0x7FFFFFFF);
    hipLaunchKernelGGL(k_quant32, dim3((unsigned)cnt), dim3(256), 0, s, p.d.q32tiles + first, w, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const sshdp_plan &p, const float *w, uint16_t *out, hipStream_t s) {
  const int64_t n = (int64_t)p.cchunks.size();
  for (int64_t first = 0; first < n; first += 0x7FFFFFFF) {
    const int64_t cnt = std::min<int64_t>(n - first, 0x7FFFFFFF);
    hipLaunchKernelGGL(k_cast_bf16, dim3((unsigned)cnt), dim3(256), 0, s, p.d.cchunks + first, w, out);
  }
  return hipGetLastError();
}

}  // namespace sshdp
