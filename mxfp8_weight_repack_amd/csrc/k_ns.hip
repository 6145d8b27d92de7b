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
// Every product is one "NT" contraction O = alpha P Q^T + beta D with both
// operands K-contiguous, the layout the MFMA operands want:
//   Gram    A = X X^T            P = Q = X   (r x c)
//   poly    B = c A A + b A      P = Q = A   (A symmetric, so A A^T = A A; the
//                                b A term comes from the Q operand in LDS)
//   update  X' = a X + B X       P = B, Q = X^T (c x r); the a X term is
//           X^T read back from the Q operand's LDS stages (no extra memory
//           read); the epilogue writes X' and X'^T, the operands of the next
//           step (no transpose pass)
// Groups whose Gram runs in 128-tiles read it from X^T instead ("K-major":
// both operands staged k-row by k-row and turned into MFMA fragments by
// ds_read_b64_tr_b16 pairs), so their update stores X'^T alone and f0 stores
// u^T alone.
// A and B are symmetric: only tiles with tm <= tn are computed and each
// off-diagonal tile is also stored mirrored.  Groups of one 128-row tile
// (per-head units) keep B as a bf16 pair [B_hi | B_lo], B_lo the rounded
// remainder, and their update contracts over both halves (K = 2 r_pad, X^T
// read twice): rounding B is the iteration's largest storage error, and these
// short-K updates are latency-bound, so the doubled K costs little.  The normalisation is folded into
// the first step's scalars: with s = 1/(||u|| + eps), A0 = s^2 u u^T and
// X1 = s (B0 u) + a s u.  A unit whose momentum is all zero has s = 0 and skips
// every product (its direction is exactly zero).  A tall unit is iterated on
// its transpose (same map: X (X^T X) = (X X^T) X); its own layout plays the
// role of X^T.
//
// Per stage, one launch per tile size covers every group and unit on a stream
// (tile tables built by the planner, longest K first, in XCD-aware order);
// groups are dealt to up to four concurrent streams, so small per-head units
// run beside the large matrices instead of serialising latency-bound launches.
//
// Tile kernel: 256 x 256 per workgroup of 8 waves (2 x 4, each 128 x 64) or
// 128 x 128 per workgroup of 4 waves (2 x 2), as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators; K in steps of 64 through
// two LDS stages filled by buffer loads straight into LDS (no VGPR staging),
// each stage reloaded as soon as the barrier ending its step has passed;
// 128-byte LDS rows whose 16-byte chunks are XOR-swizzled so fragment reads
// are bank-conflict free; fragment reads and buffer loads are interleaved one
// per MFMA.  Epilogue through LDS (bf16 pack in hardware), 16-byte stores.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "lds_swizzle.h"
#include "tile_map.h"

namespace sshdp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for raw (untyped) gfx9-family buffer loads.
constexpr int kBufWord3 = 0x00020000;


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bfloat16 (a in the low half), one v_cvt_pk_bf16_f32:
// round to nearest even, identical to mx_bf16_bits for every non-NaN float32
// (checked exhaustively on the device).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Tile configuration: TM x TN output per workgroup of WM x WN waves, each
// wave (TM/WM) x (TN/WN) as 32x32 MFMA blocks; K moves through a ring of NST
// LDS stages of BK elements.  Both shipped configurations use BK = 64 and two
// stages: on the raw contraction, BK = 32 with a 4- or 6-stage ring and a
// 3-stage ring at BK = 64 (one workgroup per CU) all measured 15-30% slower.
template <int TM_, int TN_, int WM_, int WN_, int BK_ = 64, int NST_ = 2>
struct Cfg {
  static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_, BK = BK_, NST = NST_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WTM = TM / WM, WTN = TN / WN;
  static constexpr int MBM = WTM / 32, MBN = WTN / 32;
  static constexpr int RB = BK * 2;                                // bytes per LDS row
  static constexpr int CPR = RB / 16, RPI = 1024 / RB;             // 16-byte chunks per row, rows per load
  static constexpr int KS = BK / 16;                               // MFMA K slices per stage
  static constexpr int SEGA = TM * RB, SEGB = TN * RB;             // bytes of one operand stage
  static constexpr int NIA = TM / (RPI * NW), NIB = TN / (RPI * NW);   // buffer loads per wave per stage
  static constexpr int NV = NIA + NIB;
  static constexpr int STAGE = SEGA + SEGB;
  static constexpr int EPI = (TM * (TN + 8) > TN * (TM + 8) ? TM * (TN + 8) : TN * (TM + 8)) * 2;
  static constexpr int LDS = NST * STAGE > EPI ? NST * STAGE : EPI;
  static_assert(NW % 4 == 0 && NIA >= 1 && NIB >= 1 && (BK == 64 || BK == 32) && NST >= 2, "tile config");
  static_assert((NST - 2) * NV <= 63, "vmcnt range");
};

template <int BK>
__device__ __forceinline__ int swz(int r) { return lds_swz<BK>(r); }

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f32x4_t gf32x4_t;
// the main weight is read and written once per step: keep it out of the caches.
// The global address space keeps these off the LDS counter (a generic access
// would be waited for by every LDS wait in between).
__device__ __forceinline__ float4 load_nt4(const float *p) {
  const f32x4_t v = __builtin_nontemporal_load((const gf32x4_t *)p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt4(float *p, const float4 &v) {
  __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, (gf32x4_t *)p);
}

// acc = P[TM x K] Q[TN x K]^T, P and Q row-major with row pitch K elements
// (bf16) starting at byte addresses gP, gQ (uniform).
//
// CAPD (the update product, where Q = X^T and the added term is X itself):
// D[m][n] = Q[n][dk0 + m], so the D tile passes through LDS as the Q operand of
// the K steps covering [dk0, dk0 + TM).  While a stage is resident, the waves
// whose rows it covers add dscale * D into their accumulators straight from
// LDS, and the epilogue reads nothing more from memory.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// K-major stage rows (one k, T columns): 16-byte chunk c of row k sits at
// physical chunk c ^ km_swz(k), so the four rows a transposing read touches
// together fall on distinct bank groups.
__device__ __forceinline__ int km_swz(int k) { return (k & 3) << 2; }

// KM: both operands K-major (P stored [K][...] with row pitch ld elements, gP at
// element (k = 0, first row of the tile), likewise Q): the Gram read from X^T.
// Fragments come from ds_read_b64_tr_b16 pairs (each gives a lane 4 k of its row).
// SPLITQ: Q has row pitch kq = K/2 and is contracted twice: Q's element k is
// Q[n][k mod kq] (P = [P_hi | P_lo] against [Q | Q], the update with B held as a
// bf16 pair).
template <class C, bool CAPD = false, bool KM = false, bool SPLITQ = false>
__device__ __forceinline__ void gemm_core(const char *gP, const char *gQ, int64_t K, char *smem,
                                          f32x16_t (&acc)[C::MBM][C::MBN], int dk0 = 0, float dscale = 0.f,
                                          int64_t ld = 0) {
  static_assert(!(CAPD && KM), "the added term is read from an NT stage");
  static_assert(!(SPLITQ && KM), "the split contraction is NT");
  const int64_t kq = SPLITQ ? K / 2 : K;             // Q's row pitch and K period
  static_assert(!KM || (C::BK == 64 && C::TM % 32 == 0 && C::TN % 32 == 0), "K-major stages: 64 k-rows");
  constexpr int MBM = C::MBM, MBN = C::MBN, NW = C::NW, BK = C::BK, RB = C::RB, CPR = C::CPR, RPI = C::RPI;
  constexpr int NST = C::NST;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: LDS targets and offsets in SGPRs
  const int wm = wave / C::WN, wn = wave % C::WN;

  // DMA: buffer loads straight into LDS.  Load i of wave w fills rows
  // RPI*(NW*i + w) .. +RPI-1 of a stage segment, CPR lanes per row; lane i of a
  // load lands at LDS base + 16*i (M0).  The per-lane offset is fixed, the K
  // position and row block go in the scalar offset.  Each operand's buffer
  // resource covers exactly its TM (TN) x K panel.
  const int drow = RPI * wave + lane / CPR;
  const int dchunk = (lane % CPR) ^ swz<BK>(drow);   // rows drow + RPI*NW*i share the swizzle
  const int voff = (drow * (int)K + dchunk * 8) * 2;
  const int voffq = SPLITQ ? (drow * (int)kq + dchunk * 8) * 2 : voff;
  const __amdgpu_buffer_rsrc_t rP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(gP), 0, KM ? (int)(((K - 1) * ld + C::TM) * 2) : (int)(C::TM * K * 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(gQ), 0, KM ? (int)(((K - 1) * ld + C::TN) * 2) : (int)(C::TN * kq * 2), kBufWord3);
  // K-major DMA: a load fills RK = 1024 / (2 T) whole rows (k) of T columns; load i
  // of wave w fills rows RK*(NW*i + w) ..; the row's swizzle depends on k % 4 only
  constexpr int CKA = C::TM / 8, CKB = C::TN / 8;                  // 16-byte chunks per K-major row
  constexpr int RKA = 64 / CKA, RKB = 64 / CKB;                    // rows per load
  const int kra = RKA * wave + lane / CKA, krb = RKB * wave + lane / CKB;
  const int voffa = (int)(kra * ld * 2) + (((lane % CKA) ^ km_swz(kra)) << 4);
  const int voffb = (int)(krb * ld * 2) + (((lane % CKB) ^ km_swz(krb)) << 4);

  // fragment reads: lane holds row (lane & 31) of a 32-row block, logical chunk 2 kk + (lane >> 5)
  const int lrow = lane & 31;
  const int ra = (wm * C::WTM + lrow) * RB, rb = (wn * C::WTN + lrow) * RB;
  int cofs[C::KS];
#pragma unroll
  for (int kk = 0; kk < C::KS; ++kk) cofs[kk] = ((2 * kk + (lane >> 5)) ^ swz<BK>(lrow)) * 16;

#pragma unroll
  for (int i = 0; i < MBM; ++i)
#pragma unroll
    for (int j = 0; j < MBN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto dma_p = [&](int stage, int k0) __attribute__((always_inline)) {
    char *sa = smem + stage * C::STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < C::NIA; ++i) {
      if (KM)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (__attribute__((address_space(3))) void *)(sa + i * NW * 1024),
                                                 16, voffa, (int)((k0 + i * RKA * NW) * ld * 2), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (__attribute__((address_space(3))) void *)(sa + i * NW * 1024),
                                                 16, voff, (i * RPI * NW * (int)K + k0) * 2, 0, 0);
    }
  };
  auto dma_q = [&](int stage, int k0) __attribute__((always_inline)) {
    char *sa = smem + stage * C::STAGE + C::SEGA + wave * 1024;
    if (SPLITQ && k0 >= kq) k0 -= (int)kq;           // the second pass over Q
#pragma unroll
    for (int i = 0; i < C::NIB; ++i) {
      if (KM)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (__attribute__((address_space(3))) void *)(sa + i * NW * 1024),
                                                 16, voffb, (int)((k0 + i * RKB * NW) * ld * 2), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (__attribute__((address_space(3))) void *)(sa + i * NW * 1024),
                                                 16, voffq, (i * RPI * NW * (int)kq + k0) * 2, 0, 0);
    }
  };
  bf16x8_t fa0[MBM], fb0[MBN], fa1[MBM], fb1[MBN];
  // K-major fragment: in each 16-lane group, source lane s reads 4 columns of row
  // k0 + s/4; the transposing read hands lane i of the group column i at rows
  // k0 .. k0+3.  Lane l: row (in the 32-row block) l % 32, k = 16 kk + 8 (l/32) + 0..7
  // from two reads (k0 and k0 + 4).
  const int tk = 8 * (lane >> 5) + ((lane & 15) >> 2);             // k of this lane's read, slice-relative
  const int tm = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);          // first column it reads, block-relative
  const int tsw = km_swz(tk);                                       // = 4 * ((lane & 15) >> 2)
  auto ldtr = [&](const char *seg, int rowbytes, int col, int kk) __attribute__((always_inline)) {
    const char *base = seg + (16 * kk + tk) * rowbytes + (col & 7) * 2;
    const int c = col >> 3;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(base + ((c ^ tsw) << 4)));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(base + 4 * rowbytes + ((c ^ tsw) << 4)));
    const i16x4_t v[2] = {lo, hi};
    return *reinterpret_cast<const bf16x8_t *>(v);
  };
  auto ldfrag = [&](const char *sa, int kk, bf16x8_t(&fa_)[MBM], bf16x8_t(&fb_)[MBN]) __attribute__((always_inline)) {
    if (KM) {
#pragma unroll
      for (int i = 0; i < MBM; ++i) fa_[i] = ldtr(sa, C::TM * 2, wm * C::WTM + i * 32 + tm, kk);
#pragma unroll
      for (int j = 0; j < MBN; ++j) fb_[j] = ldtr(sa + C::SEGA, C::TN * 2, wn * C::WTN + j * 32 + tm, kk);
      return;
    }
#pragma unroll
    for (int i = 0; i < MBM; ++i) fa_[i] = *reinterpret_cast<const bf16x8_t *>(sa + ra + i * 32 * RB + cofs[kk]);
#pragma unroll
    for (int j = 0; j < MBN; ++j)
      fb_[j] = *reinterpret_cast<const bf16x8_t *>(sa + C::SEGA + rb + j * 32 * RB + cofs[kk]);
  };
  // one slice's MFMAs, each followed by one fragment read of the next slice
  // (nr of them) and one buffer load (nv of them)
  auto mma = [&](bf16x8_t(&fa_)[MBM], bf16x8_t(&fb_)[MBN], int nr, int nv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MBM; ++i)
#pragma unroll
      for (int j = 0; j < MBN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa_[i], fb_[j], acc[i][j], 0, 0, 0);
    constexpr int NM = MBM * MBN;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < nr) __builtin_amdgcn_sched_group_barrier(0x100, KM ? 2 : 1, 0);
      if (i < nv) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };
  // wait until stage `kt + 1` has landed: the newer NST - 2 stages' loads may still fly
  auto wait_next = [&]() __attribute__((always_inline)) {
    if (NST == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (NST == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::NV) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NST - 2) * C::NV) : "memory");
  };
  constexpr int NR = MBM + MBN;

  const int nk = (int)(K / BK);
  // CAPD: while stage `sa` (K step kt) is resident, add dscale * D from it
  auto capd = [&](const char *sa, int kt) __attribute__((always_inline)) {
    const int mb = kt * BK - dk0;                    // tile row held at K offset 0 of this stage
#pragma unroll
    for (int i = 0; i < MBM; ++i) {
      const int bm = wm * C::WTM + i * 32;           // wave-uniform
      if (CAPD && bm >= mb && bm < mb + BK) {
#pragma unroll
        for (int j = 0; j < MBN; ++j) {
          const int n = wn * C::WTN + j * 32 + lrow;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int kl = bm - mb + g4 * 8 + (lane >> 5) * 4;
            const uint2 d = *reinterpret_cast<const uint2 *>(sa + C::SEGA + n * RB +
                                                             (((kl >> 3) ^ swz<BK>(lrow)) << 4) + (kl & 7) * 2);
            acc[i][j][g4 * 4 + 0] = fmaf(dscale, __uint_as_float(d.x << 16), acc[i][j][g4 * 4 + 0]);
            acc[i][j][g4 * 4 + 1] = fmaf(dscale, __uint_as_float(d.x & 0xFFFF0000u), acc[i][j][g4 * 4 + 1]);
            acc[i][j][g4 * 4 + 2] = fmaf(dscale, __uint_as_float(d.y << 16), acc[i][j][g4 * 4 + 2]);
            acc[i][j][g4 * 4 + 3] = fmaf(dscale, __uint_as_float(d.y & 0xFFFF0000u), acc[i][j][g4 * 4 + 3]);
          }
        }
      }
    }
  };

  if (C::KS == 4 && NST == 2) {
    // Two stages, each reloaded as soon as the barrier that ends its step has
    // passed: the loads for step kt + 2 go out with the last slice of step kt,
    // so they have a whole step to land.
    dma_p(0, 0);
    dma_q(0, 0);
    dma_p(1, (nk > 1 ? 1 : 0) * BK);
    dma_q(1, (nk > 1 ? 1 : 0) * BK);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::NV) : "memory");   // stage 0 landed
    __syncthreads();
    ldfrag(smem, 0, fa0, fb0);
    for (int kt = 0; kt < nk; ++kt) {
      const char *sa = smem + (kt & 1) * C::STAGE;
      ldfrag(sa, 1, fa1, fb1);
      mma(fa0, fb0, NR, 0);
      __builtin_amdgcn_sched_barrier(0);
      ldfrag(sa, 2, fa0, fb0);
      mma(fa1, fb1, NR, 0);
      __builtin_amdgcn_sched_barrier(0);
      ldfrag(sa, 3, fa1, fb1);
      mma(fa0, fb0, NR, 0);
      __builtin_amdgcn_sched_barrier(0);
      capd(sa, kt);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");               // stage kt + 1 landed
      __syncthreads();                                                // stage kt consumed by all waves
      // near the end the reload repeats the last K slice into a stage nobody
      // reads again, so the body has no branch
      const int kn = (kt + 2 < nk ? kt + 2 : nk - 1) * BK;
      dma_p(kt & 1, kn);
      dma_q(kt & 1, kn);
      ldfrag(smem + ((kt + 1) & 1) * C::STAGE, 0, fa0, fb0);        // after the last step: unused
      mma(fa1, fb1, NR, C::NV);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                 // trailing reloads land before
    __syncthreads();                                                  // the caller reuses the LDS
    return;
  }

#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0) {
    const int k0 = (s0 < nk ? s0 : nk - 1) * BK;
    dma_p(s0, k0);
    dma_q(s0, k0);
  }
  wait_next();
  __syncthreads();
  ldfrag(smem, 0, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    const char *sa = smem + (kt % NST) * C::STAGE;
    // the next load goes into the stage consumed one step ago; near the end it
    // reloads the last K slice into a stage nobody reads again, so the body has
    // no branch and the loads interleave with the MFMAs
    const int tgt = (kt + NST - 1) % NST;
    const int kn = (kt + NST - 1 < nk ? kt + NST - 1 : nk - 1) * BK;
    if (C::KS == 4) {
      dma_p(tgt, kn);
      ldfrag(sa, 1, fa1, fb1);
      mma(fa0, fb0, NR, C::NIA);
      __builtin_amdgcn_sched_barrier(0);
      dma_q(tgt, kn);
      ldfrag(sa, 2, fa0, fb0);
      mma(fa1, fb1, NR, C::NIB);
      __builtin_amdgcn_sched_barrier(0);
      ldfrag(sa, 3, fa1, fb1);
      mma(fa0, fb0, NR, 0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      dma_p(tgt, kn);
      dma_q(tgt, kn);
      ldfrag(sa, 1, fa1, fb1);
      mma(fa0, fb0, NR, C::NV);
      __builtin_amdgcn_sched_barrier(0);
    }
    capd(sa, kt);
    wait_next();
    __syncthreads();
    ldfrag(smem + ((kt + 1) % NST) * C::STAGE, 0, fa0, fb0);   // after the last step: unused
    mma(fa1, fb1, NR, 0);
  }
  if (NST > 2) {                                 // trailing reloads land before the caller reuses the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// Copies an R x W bf16 tile from LDS (pitch W+8) to global rows of pitch ld,
// 16 bytes per lane.  NT: nontemporal stores, for outputs that would only
// evict operand lines; otherwise ordinary stores, so an output that the next
// stage reads and that fits the last-level cache stays there.
template <class C, int R, int W, bool NT>
__device__ __forceinline__ void copy_out(const uint16_t *lt, uint16_t *dst, int64_t ld) {
  constexpr int CH = W / 8, P = W + 8;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < R * CH / C::NT; ++k) {
    const int id = t + C::NT * k, row = id / CH, ch = id - row * CH;
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(&lt[row * P + ch * 8]);
    u32x4_t *q = reinterpret_cast<u32x4_t *>(dst + (int64_t)row * ld + ch * 8);
    if (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
  }
}

// Epilogue of a TM x TN product: x = alpha*acc + beta*D, rounded to bf16,
// stored row-major to O (leading dim ldo; skipped if O is null) and, if OT,
// transposed to OT[col*ldt + row].
// D is read through its transpose DT (DT[col*lddt + row] = D[row][col]): element
// (m, n) of a 32x32 MFMA block sits in lane n + 32*((m/4)%2), register
// (m/8)*4 + m%4, so a lane holds 4 consecutive rows of one column and the D^T
// read is 8 contiguous bytes.  Both stores go through LDS so that every lane
// writes 16 contiguous bytes and a wave writes whole rows: first the tile
// row-major (2-byte LDS writes), then, for O^T, column-major (8-byte LDS writes
// of the lane's 4 rows).  The global stores are nontemporal unless CACHED:
// ordinary stores would evict the operand lines that the other tiles of the
// launch are still streaming, which only pays off when the outputs fit the
// last-level cache and the next stage reads them there.  smem must be free
// (all fragment reads done) and hold max(TM*(TN+8), TN*(TM+8))*2 bytes.
// OL (optional, no D): the remainder x - bf16(x), rounded to bf16, stored like O
// with the same leading dimension (a bf16 pair holding x to ~16 bits).
template <class C, bool CACHED = false>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[C::MBM][C::MBN], float alpha, float beta,
                                           const uint16_t *DT, int64_t lddt, uint16_t *O, int64_t ldo, uint16_t *OT,
                                           int64_t ldt, int r0, int c0, char *smem, uint16_t *OL = nullptr) {
  constexpr int LP = C::TN + 8, LPT = C::TM + 8;
  static_assert(C::TM * LP * 2 <= C::LDS && C::TN * LPT * 2 <= C::LDS, "epilogue tile fits LDS");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave / C::WN, wn = wave % C::WN;
  uint16_t *lt = reinterpret_cast<uint16_t *>(smem);
  uint2 hp[C::MBM][C::MBN][4];                       // packed bf16 of the lane's 4-row runs
#pragma unroll
  for (int i = 0; i < C::MBM; ++i) {
#pragma unroll
    for (int j = 0; j < C::MBN; ++j) {
      const int lc = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int lr0 = wm * C::WTM + i * 32 + g4 * 8 + (lane >> 5) * 4;
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = alpha * acc[i][j][g4 * 4 + q];
        if (DT) {
          const uint2 d = *reinterpret_cast<const uint2 *>(DT + (int64_t)(c0 + lc) * lddt + r0 + lr0);
          x[0] = fmaf(beta, __uint_as_float(d.x << 16), x[0]);
          x[1] = fmaf(beta, __uint_as_float(d.x & 0xFFFF0000u), x[1]);
          x[2] = fmaf(beta, __uint_as_float(d.y << 16), x[2]);
          x[3] = fmaf(beta, __uint_as_float(d.y & 0xFFFF0000u), x[3]);
        }
        const uint32_t h01 = pk_bf16(x[0], x[1]), h23 = pk_bf16(x[2], x[3]);
        hp[i][j][g4] = make_uint2(h01, h23);
        if (O) {
          lt[(lr0 + 0) * LP + lc] = (uint16_t)h01;
          lt[(lr0 + 1) * LP + lc] = (uint16_t)(h01 >> 16);
          lt[(lr0 + 2) * LP + lc] = (uint16_t)h23;
          lt[(lr0 + 3) * LP + lc] = (uint16_t)(h23 >> 16);
        }
      }
    }
  }
  if (O) {
    __syncthreads();
    copy_out<C, C::TM, C::TN, !CACHED>(lt, O + (int64_t)r0 * ldo + c0, ldo);
  }
  if (OL) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::MBM; ++i)
#pragma unroll
      for (int j = 0; j < C::MBN; ++j) {
        const int lc = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int lr0 = wm * C::WTM + i * 32 + g4 * 8 + (lane >> 5) * 4;
          const uint2 h = hp[i][j][g4];
          const float hi[4] = {__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xFFFF0000u),
                               __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xFFFF0000u)};
          float lo[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) lo[q] = alpha * acc[i][j][g4 * 4 + q] - hi[q];
          const uint32_t l01 = pk_bf16(lo[0], lo[1]), l23 = pk_bf16(lo[2], lo[3]);
          lt[(lr0 + 0) * LP + lc] = (uint16_t)l01;
          lt[(lr0 + 1) * LP + lc] = (uint16_t)(l01 >> 16);
          lt[(lr0 + 2) * LP + lc] = (uint16_t)l23;
          lt[(lr0 + 3) * LP + lc] = (uint16_t)(l23 >> 16);
        }
      }
    __syncthreads();
    copy_out<C, C::TM, C::TN, !CACHED>(lt, OL + (int64_t)r0 * ldo + c0, ldo);
  }
  if (!OT) return;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::MBM; ++i)
#pragma unroll
    for (int j = 0; j < C::MBN; ++j) {
      const int lc = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int lr0 = wm * C::WTM + i * 32 + g4 * 8 + (lane >> 5) * 4;
        *reinterpret_cast<uint2 *>(&lt[lc * LPT + lr0]) = hp[i][j][g4];
      }
    }
  __syncthreads();
  copy_out<C, C::TN, C::TM, !CACHED>(lt, OT + (int64_t)c0 * ldt + r0, ldt);
}

// f2 on a tile of the last update product: w <- w*decay - lr*scale*x for the
// elements inside the unit (oriented r x c; a tall unit's view is the
// transpose).  The tile goes through LDS in fp32, half its rows at a time,
// laid out in the view's own orientation, so the read-modify-write of w is
// 16 contiguous bytes per lane along the view's contiguous dimension.
template <class C>
__device__ __forceinline__ void final_tile(const f32x16_t (&acc)[C::MBM][C::MBN], float alpha, const MuonUnit &u,
                                           float *w, float lr, float decay, int r0, int c0, bool zero, char *smem) {
  constexpr int HM = C::TM / 2;                      // rows per pass (= one wave row)
  static_assert(HM == C::WTM, "one pass per wave row");
  constexpr int PW = C::TN + 4, PT = HM + 4;         // fp32 LDS pitches (wide / tall layout)
  static_assert(HM * PW * 4 <= C::LDS && C::TN * PT * 4 <= C::LDS, "final tile fits LDS");
  if (zero && decay == 1.0f) return;                 // direction 0, no decay: w unchanged
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const int r_unit = u.tall ? u.cols : u.rows, c_unit = u.tall ? u.rows : u.cols;
  const float ls = lr * u.upd_scale;
  float *lt = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < C::MBM; ++i) {
#pragma unroll
        for (int j = 0; j < C::MBN; ++j) {
          const int lc = wn * C::WTN + j * 32 + (lane & 31);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int li0 = i * 32 + g4 * 8 + (lane >> 5) * 4;       // row within the pass
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (!zero) {
#pragma unroll
              for (int q = 0; q < 4; ++q) x[q] = alpha * acc[i][j][g4 * 4 + q];
            }
            if (u.tall) {
              *reinterpret_cast<float4 *>(&lt[lc * PT + li0]) = make_float4(x[0], x[1], x[2], x[3]);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) lt[(li0 + q) * PW + lc] = x[q];
            }
          }
        }
      }
    }
    __syncthreads();
    const int rb = r0 + h * HM;                      // first oriented row of this pass
    // each thread owns IT float4 of w per pass; they are read in batches of KB
    // loads before any store, so a batch's loads are in flight together
    constexpr int IT = C::TN * HM / 4 / C::NT, KB = 4;
    static_assert(C::TN * HM / 4 % C::NT == 0 && IT % KB == 0, "whole float4 batches per thread");
#pragma unroll
    for (int k0 = 0; k0 < IT; k0 += KB) {
      float *pw[KB];
      float4 xv[KB], wv[KB];
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        const int id = t + (k0 + q) * C::NT;
        int row, col, lofs;
        if (!u.tall) {
          // view row = oriented row, contiguous along oriented columns
          constexpr int CH = C::TN / 4;
          const int li = id / CH, j4 = (id - li * CH) * 4;
          row = rb + li; col = c0 + j4; lofs = li * PW + j4;
          pw[q] = w + u.abs + (int64_t)row * u.row_stride + col;
        } else {
          // view row = oriented column, contiguous along oriented rows
          constexpr int CH = HM / 4;
          const int lc = id / CH, i4 = (id - lc * CH) * 4;
          row = rb + i4; col = c0 + lc; lofs = lc * PT + i4;
          pw[q] = w + u.abs + (int64_t)col * u.row_stride + row;
        }
        if (!(row < r_unit && col < c_unit)) pw[q] = nullptr;
        xv[q] = *reinterpret_cast<const float4 *>(&lt[lofs]);
        if (pw[q]) wv[q] = load_nt4(pw[q]);
      }
#pragma unroll
      for (int q = 0; q < KB; ++q) {
        if (!pw[q]) continue;
        float4 o;
        o.x = fmaf(wv[q].x, decay, -ls * xv[q].x);
        o.y = fmaf(wv[q].y, decay, -ls * xv[q].y);
        o.z = fmaf(wv[q].z, decay, -ls * xv[q].z);
        o.w = fmaf(wv[q].w, decay, -ls * xv[q].w);
        store_nt4(pw[q], o);
      }
    }
    __syncthreads();
  }
}

struct NsArgs {
  char *ws;
  const NsGroupDev *groups;
  const NsTile *tiles;
  const float *uscale;
  const MuonUnit *units;
  float *w;
  float lr, decay;          // f2
  float ca, cb, cc;         // quintic coefficients
  int iter;
};

// STAGE: 0 Gram, 1 poly, 2 update, 3 update + f2.  CACHED: the stage's outputs
// are stored with ordinary stores (they and the rest of the step's NS working
// set fit the last-level cache, so the next stage reads them from there).
template <int STAGE, class C, bool CACHED>
__global__ __launch_bounds__(C::NT, C::NT == 256 ? 2 : 1) void k_ns(NsArgs a) {
  constexpr int TILE = C::TM;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const NsTile tl = a.tiles[blockIdx.x];
  const NsGroupDev g = a.groups[tl.group];
  const int unit = g.unit_base + tl.b;
  const float s = a.uscale[unit];
  const bool zero = s == 0.f;                       // all-zero momentum: direction is exactly 0
  if (zero && STAGE != 3) return;
  const int64_t rp = g.r_pad, cp = g.c_pad;
  // X is not stored for groups whose Gram reads X^T (K-major)
  uint16_t *X = g.km ? nullptr : reinterpret_cast<uint16_t *>(a.ws + g.off_x) + tl.b * rp * cp;
  uint16_t *XT0 = reinterpret_cast<uint16_t *>(a.ws + g.off_xt0) + tl.b * rp * cp;
  uint16_t *XT1 = reinterpret_cast<uint16_t *>(a.ws + g.off_xt1) + tl.b * rp * cp;
  uint16_t *A = reinterpret_cast<uint16_t *>(a.ws + g.off_a) + tl.b * rp * rp;
  // a split group keeps B as [B_hi | B_lo], row pitch 2 rp (one 128-tile: tm = tn = 0)
  const bool split = C::TM == kNsSmall && g.split;
  const int64_t ldb = split ? 2 * rp : rp;
  uint16_t *B = reinterpret_cast<uint16_t *>(a.ws + g.off_b) + tl.b * rp * ldb;
  const int r0 = tl.tm * TILE, c0 = tl.tn * TILE;
  f32x16_t acc[C::MBM][C::MBN];
  if (STAGE == 0) {
    if (g.km) {
      // from X^T (c_pad x r_pad): the tile's rows and columns are X^T columns
      const uint16_t *XTc = (a.iter & 1) ? XT1 : XT0;
      gemm_core<C, false, true>(reinterpret_cast<const char *>(XTc + r0), reinterpret_cast<const char *>(XTc + c0),
                                cp, smem, acc, 0, 0.f, rp);
    } else {
      gemm_core<C>(reinterpret_cast<const char *>(X + r0 * cp), reinterpret_cast<const char *>(X + c0 * cp), cp,
                   smem, acc);
    }
    const float al = a.iter == 0 ? s * s : 1.f;
    store_tile<C, CACHED>(acc, al, 0.f, nullptr, 0, A, rp, tl.tm != tl.tn ? A : nullptr, rp, r0, c0, smem);
  } else if (STAGE == 1) {
    // B = c (A A + (b/c) A); the A term is Q^T = A[c0.., r0..]^T, taken from LDS
    gemm_core<C, true>(reinterpret_cast<const char *>(A + r0 * rp), reinterpret_cast<const char *>(A + c0 * rp),
                       rp, smem, acc, r0, a.cb / a.cc);
    if (split)
      store_tile<C, CACHED>(acc, a.cc, 0.f, nullptr, 0, B, ldb, nullptr, 0, r0, c0, smem, B + rp);
    else
      store_tile<C, CACHED>(acc, a.cc, 0.f, nullptr, 0, B, rp, tl.tm != tl.tn ? B : nullptr, rp, r0, c0, smem);
  } else {
    const uint16_t *XTc = (a.iter & 1) ? XT1 : XT0;
    uint16_t *XTn = (a.iter & 1) ? XT0 : XT1;
    // X' = al (B X + a X): the a X term is taken from the Q operand in LDS
    const float al = a.iter == 0 ? s : 1.f;
    auto update = [&]() __attribute__((always_inline)) {
      if constexpr (C::TM == kNsSmall) {
        if (split) {
          gemm_core<C, true, false, true>(reinterpret_cast<const char *>(B + r0 * ldb),
                                          reinterpret_cast<const char *>(XTc + c0 * rp), ldb, smem, acc, r0, a.ca);
          return;
        }
      }
      gemm_core<C, true>(reinterpret_cast<const char *>(B + r0 * rp),
                         reinterpret_cast<const char *>(XTc + c0 * rp), rp, smem, acc, r0, a.ca);
    };
    if (STAGE == 2) {
      update();
      store_tile<C, CACHED>(acc, al, 0.f, nullptr, 0, X, cp, XTn, rp, r0, c0, smem);
    } else {
      if (!zero) update();
      const MuonUnit u = a.units[unit];
      final_tile<C>(acc, al, u, a.w, a.lr, a.decay, r0, c0, zero, smem);
    }
  }
}

// Raw batched contraction for tests: O[b] = alpha P[b] Q[b]^T + beta D[b].
struct RawArgs {
  const uint16_t *P, *Q, *D;
  uint16_t *O, *OT;
  int M, N, K;
  float alpha, beta;
};

template <class C>
__global__ __launch_bounds__(C::NT, 1) void k_gemm_raw(RawArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int b = blockIdx.y;
  int tm, tn;
  xcd_tile((int)blockIdx.x, a.M / C::TM, a.N / C::TN, &tm, &tn);
  const int64_t M = a.M, N = a.N, K = a.K;
  f32x16_t acc[C::MBM][C::MBN];
  gemm_core<C>(reinterpret_cast<const char *>(a.P + b * M * K + (int64_t)tm * C::TM * K),
               reinterpret_cast<const char *>(a.Q + b * N * K + (int64_t)tn * C::TN * K), K, smem, acc);
  // the raw entry takes D^T (N x M), the layout the update product reads X in
  store_tile<C>(acc, a.alpha, a.beta, a.D ? a.D + b * M * N : nullptr, M, a.O + b * M * N, N,
                a.OT ? a.OT + b * M * N : nullptr, M, tm * C::TM, tn * C::TN, smem);
}

// Raw K-major ("TN") contraction for tests: O[b] = alpha P[b]^T Q[b] with P[b]
// K x M and Q[b] K x N row-major (the Gram read from X^T).
template <class C>
__global__ __launch_bounds__(C::NT, 1) void k_gemm_raw_km(RawArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  const int b = blockIdx.y;
  int tm, tn;
  xcd_tile((int)blockIdx.x, a.M / C::TM, a.N / C::TN, &tm, &tn);
  const int64_t M = a.M, N = a.N, K = a.K;
  f32x16_t acc[C::MBM][C::MBN];
  gemm_core<C, false, true>(reinterpret_cast<const char *>(a.P + b * K * M + (int64_t)tm * C::TM),
                            reinterpret_cast<const char *>(a.Q + b * K * N + (int64_t)tn * C::TN), K, smem, acc, 0,
                            0.f, M);
  store_tile<C>(acc, a.alpha, 0.f, nullptr, 0, a.O + b * M * N, N, a.OT ? a.OT + b * M * N : nullptr, M,
                tm * C::TM, tn * C::TN, smem);
}

using CSmall = Cfg<kNsSmall, kNsSmall, 2, 2>;   // 4 waves, two workgroups per CU
using CLarge = Cfg<kNsLarge, kNsLarge, 2, 4>;   // 8 waves (two per SIMD), one workgroup per CU

template <int STAGE, class C>
hipError_t launch_list(const NsArgs &a, size_t n, bool cached, hipStream_t s) {
  // the last update stores no stage output: one instantiation
  if (cached && STAGE != 3)
    hipLaunchKernelGGL((k_ns<STAGE, C, STAGE != 3>), dim3((unsigned)n), dim3(C::NT), 0, s, a);
  else
    hipLaunchKernelGGL((k_ns<STAGE, C, false>), dim3((unsigned)n), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

template <int STAGE>
hipError_t launch_sizes(const sshdp_plan &p, NsArgs a, int ln, int st, hipStream_t s, int sizes) {
  hipError_t e = hipSuccess;
  if ((sizes & 1) && !p.ns_tiles[ln][st][1].empty()) {       // 256-tile work first: it is the long part
    a.tiles = p.d.ns_tiles[ln][st][1];
    e = launch_list<STAGE, CLarge>(a, p.ns_tiles[ln][st][1].size(), p.ns_cached, s);
    if (e != hipSuccess) return e;
  }
  if ((sizes & 2) && !p.ns_tiles[ln][st][0].empty()) {
    a.tiles = p.d.ns_tiles[ln][st][0];
    e = launch_list<STAGE, CSmall>(a, p.ns_tiles[ln][st][0].size(), p.ns_cached, s);
  }
  return e;
}

}  // namespace

hipError_t launch_ns_stage(const sshdp_plan &p, int lane, int stage, int iter, char *ws, float *w_main, float lr,
                           float wd, hipStream_t s, int sizes) {
  NsArgs a{};
  a.ws = ws;
  a.groups = p.d.ns_groups;
  a.uscale = reinterpret_cast<const float *>(ws + p.ws_uscale);
  a.units = p.d.munits;
  a.w = w_main;
  a.lr = lr;
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  a.ca = p.opts.ns_a;
  a.cb = p.opts.ns_b;
  a.cc = p.opts.ns_c;
  a.iter = iter;
  switch (stage) {
    case 0: return launch_sizes<0>(p, a, lane, 0, s, sizes);
    case 1: return launch_sizes<1>(p, a, lane, 1, s, sizes);
    case 2: return launch_sizes<2>(p, a, lane, 2, s, sizes);
    default: return launch_sizes<3>(p, a, lane, 2, s, sizes);
  }
}

hipError_t launch_gemm_raw(const void *P, const void *Q, const void *D, void *O, void *OT, int M, int N, int K,
                           int batch, float alpha, float beta, int tile, hipStream_t s) {
  RawArgs a{};
  a.P = static_cast<const uint16_t *>(P);
  a.Q = static_cast<const uint16_t *>(Q);
  a.D = static_cast<const uint16_t *>(D);
  a.O = static_cast<uint16_t *>(O);
  a.OT = static_cast<uint16_t *>(OT);
  a.M = M; a.N = N; a.K = K;
  a.alpha = alpha; a.beta = beta;
  if (tile == 128) {
    using C = CSmall;
    hipLaunchKernelGGL(k_gemm_raw<C>, dim3((unsigned)((M / 128) * (N / 128)), (unsigned)batch), dim3(C::NT), 0, s, a);
  } else if (tile == 256) {
    using C = CLarge;
    hipLaunchKernelGGL(k_gemm_raw<C>, dim3((unsigned)((M / 256) * (N / 256)), (unsigned)batch), dim3(C::NT), 0, s, a);
  } else if (tile == 1281) {   // K-major operands (M must equal N for the shared pitch rule below)
    using C = CSmall;
    hipLaunchKernelGGL(k_gemm_raw_km<C>, dim3((unsigned)((M / 128) * (N / 128)), (unsigned)batch), dim3(C::NT), 0, s, a);
  } else if (tile == 2561) {
    using C = CLarge;
    hipLaunchKernelGGL(k_gemm_raw_km<C>, dim3((unsigned)((M / 256) * (N / 256)), (unsigned)batch), dim3(C::NT), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sshdp
