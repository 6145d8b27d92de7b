// internal.h -- plan tables shared by the host planner and the HIP kernels.
#pragma once
#include <stdint.h>
#include <stddef.h>

#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/sshdp.h"

namespace sshdp {

constexpr int kF0Tile = 64;          // f0 transposing tile edge (elements)
constexpr int kNsSmall = 128;        // Newton-Schulz GEMM macro tiles: 128 x 128 (4 waves) ...
constexpr int kNsLarge = 256;        // ... or 256 x 256 (8 waves), chosen per group and stage
// Longest edge of a Muon unit: a 256-row operand panel of K bf16 elements is one
// buffer resource with 32-bit byte offsets (256 * K * 2 < 2^31), K a multiple of 128
constexpr int64_t kNsMaxEdge = (int64_t)0x7FFFFFFF / (2 * kNsLarge) / kNsSmall * kNsSmall;
constexpr int64_t kNsCacheBytes = 256ll << 20;  // last-level cache (MALL) of the chip
constexpr int kMaxLanes = 4;         // Newton-Schulz groups run on up to 4 concurrent streams
constexpr int kGpuCus = 256;         // compute units of an MI355X (workgroup slots for the stream rule)
constexpr int kChunk = 4096;         // elements per AdamW / requant work item
constexpr size_t kAlign = 256;       // workspace sub-buffer alignment (bytes)
constexpr int kRsMaxInputs = 8;      // slices one reduce-scatter reduction call takes

// One Muon unit as the kernels see it (device table, ordered by group).
struct MuonUnit {
  int64_t abs;          // absolute element offset of element (0,0) in the roots
  int64_t row_stride;   // elements between rows of the original view
  int32_t rows, cols;   // original view shape
  int32_t tall;         // rows > cols: oriented matrix X is the transpose of the view
  int32_t group;        // Newton-Schulz group
  int32_t idx;          // position inside the group (GEMM batch index)
  int32_t tile_begin;   // f0 tiles [tile_begin, tile_end) -> norm partials
  int32_t tile_end;
  int32_t Rp, Cp;       // padded original dims: the unit's own layout is Rp x Cp
  int64_t ws_orig;      // workspace byte offset of bf16 u in the unit's own layout (Rp x Cp), -1: not stored
  int64_t ws_trans;     // ... and of its transpose (Cp x Rp), -1: not stored
  float upd_scale;      // update scale (scale mode) of f2
  int32_t pad_;
};

// One f0 tile: a kF0Tile x kF0Tile block of the unit's original (padded) layout.
struct F0Tile {
  int32_t unit;
  int32_t tr, tc;       // tile row / column index
};

// Newton-Schulz group: units with the same oriented shape r x c (r <= c).
struct Group {
  int32_t r, c, r_pad, c_pad, n;
  // 256-tile regions (multiples of 256; 0 = none); the rest of each product in 128-tiles:
  // Gram/poly rows and columns [0, g256), update rows [0, u256r) x columns [0, u256c)
  int32_t g256, u256r, u256c;
  int32_t km;           // Gram from X^T with transposing LDS reads (128-tile Gram groups)
  int32_t split;        // r_pad == 128: B kept as a bf16 pair [B_hi | B_lo] (r_pad x 2 r_pad) and the
                        // update contracts over both halves (K = 2 r_pad, X^T read twice)
  int32_t unit_base;    // first MuonUnit of the group in the device table
  size_t off_x, off_xt0, off_xt1, off_a, off_b;   // workspace byte offsets
};

// Newton-Schulz group as the kernels see it.
struct NsGroupDev {
  int64_t off_x, off_xt0, off_xt1, off_a, off_b;   // workspace byte offsets
  int32_t r_pad, c_pad, unit_base, n;
  int32_t km;           // Gram read from X^T (K-major); X itself is never stored
  int32_t split;        // B stored as [B_hi | B_lo], row pitch 2 r_pad (see Group::split)
};

// One macro tile of one stage: group, unit within the group, tile row/column.
struct NsTile {
  int32_t group, b, tm, tn;
};

// AdamW work item: a contiguous run of unit elements (<= kChunk).
struct ASeg {
  int64_t base;
  int32_t n;
  int32_t pad_;
};

// Quantised region (runtime weight or quantised unit); contiguous, 32-aligned.
struct QRegion {
  int64_t abs;
  int64_t rows;
  int32_t cols;
  int32_t pad_;
};

// Requant work item: blocks [base, base + n) of one region (n % 32 == 0,
// n <= kChunk); elements in [lo, hi) are AdamW-updated first when fused.
struct QChunk {
  int64_t base;
  int64_t lo, hi;
  int32_t n;
  int32_t region;
  int32_t row0, col0;   // region row and column of `base` (for the TILE32X4 scale index)
};

// 32 x 32-block requant work item: 32 rows x up to 4 blocks of 32 columns of
// one region, starting at element `base`; its first block's scale sits at `sidx`.
struct Q32Tile {
  int64_t base;
  int64_t sidx;
  int32_t cols;         // the region's row pitch (= columns)
  int32_t nb;           // blocks in this tile (1..4)
};

// BF16-cast work item: elements [base, base + n) of one region (n <= kChunk, n % 8 == 0).
struct CChunk {
  int64_t base;
  int32_t n;
  int32_t pad_;
};

struct DeviceTables {
  MuonUnit *munits = nullptr;
  F0Tile *f0tiles = nullptr;
  ASeg *aseg_all = nullptr;
  ASeg *aseg_unfused = nullptr;
  QRegion *qregions = nullptr;
  QChunk *qchunks = nullptr;
  Q32Tile *q32tiles = nullptr;
  CChunk *cchunks = nullptr;
  NsGroupDev *ns_groups = nullptr;
  NsTile *ns_tiles[kMaxLanes][3][2] = {};   // [lane][stage: Gram, poly, update][tile: 128, 256]
  int32_t *norm_units = nullptr;
};

}  // namespace sshdp

struct sshdp_plan {
  int64_t root_numel = 0;
  sshdp_plan_opts opts{};
  std::vector<int64_t> node_abs;
  std::vector<int32_t> node_group;
  std::vector<sshdp::MuonUnit> munits;
  std::vector<sshdp::F0Tile> f0tiles;
  std::vector<sshdp::Group> groups;
  std::vector<double> group_unit_flops;   // MFMA flops the tile schedule executes per unit and step
  std::vector<sshdp::NsGroupDev> ns_groups;
  // Newton-Schulz groups are dealt to lanes (lane 0 = the caller's stream, others = plan-owned
  // streams joined back by events); per lane, stage and tile size a tile table, longest K first
  int n_lanes = 1;
  std::vector<int32_t> group_lane;
  bool ns_cached = false;             // NS stage outputs stored cacheable (working set fits the last-level cache)
  // f0 tiles and the units whose norms they feed, contiguous per lane: lane l owns tiles
  // [f0_lane[l], f0_lane[l+1]) and units norm_units[norm_lane[l] .. norm_lane[l+1])
  int32_t f0_lane[sshdp::kMaxLanes + 1] = {};
  int32_t norm_lane[sshdp::kMaxLanes + 1] = {};
  std::vector<int32_t> norm_units;
  std::vector<sshdp::NsTile> ns_tiles[sshdp::kMaxLanes][3][2];
  hipStream_t lane_stream[sshdp::kMaxLanes] = {};
  hipEvent_t ev_fork = nullptr, ev_join[sshdp::kMaxLanes] = {};
  std::vector<sshdp::ASeg> aseg_all, aseg_unfused;
  std::vector<sshdp::QRegion> qregions;
  std::vector<sshdp::QChunk> qchunks;   // fused-eligible chunks first
  int64_t n_qchunks_fused = 0;
  std::vector<sshdp::Q32Tile> q32tiles; // BLOCK32X32 layout: all requant work
  std::vector<sshdp::CChunk> cchunks;   // BF16 regions
  size_t ws_uscale = 0, ws_partials = 0, ws_bytes = 0;
  sshdp_plan_stats stats{};
  bool host_only = true;
  int device = -1;
  void *dblock = nullptr;
  sshdp::DeviceTables d;
  // measurement
  bool prof = false;
  double prof_ms[SSHDP_PROF_CLASSES] = {};
  int64_t prof_n[SSHDP_PROF_CLASSES] = {};
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> prof_pending;
  std::vector<hipEvent_t> prof_pool;
};

// Kernel launchers (defined in the .hip translation units).
namespace sshdp {
hipError_t launch_f0(const sshdp_plan &p, int lane, const float *g, float *m, float mu, int nesterov, char *ws,
                     hipStream_t s);
hipError_t launch_norm(const sshdp_plan &p, int lane, char *ws, float eps, hipStream_t s);
// stage: 0 Gram, 1 poly, 2 update, 3 final update (+f2); one launch per tile size covers all
// groups of the lane; sizes: 1 = the 256-tile launch, 2 = the 128-tile launch, 3 = both
hipError_t launch_ns_stage(const sshdp_plan &p, int lane, int stage, int iter, char *ws, float *w_main, float lr,
                           float wd, hipStream_t s, int sizes = 3);
hipError_t launch_gemm_raw(const void *P, const void *Q, const void *D, void *O, void *OT, int M, int N,
                           int K, int batch, float alpha, float beta, int tile, hipStream_t s);
hipError_t launch_adamw(const ASeg *segs, int64_t nseg, const sshdp_buffers &b, const sshdp_adamw_hp &hp,
                        int64_t step, hipStream_t s);
hipError_t launch_quant(const sshdp_plan &p, int64_t first, int64_t count, bool fused, const sshdp_buffers &b,
                        const sshdp_adamw_hp *hp, int64_t step, hipStream_t s);
hipError_t launch_quant32(const sshdp_plan &p, const float *w, uint8_t *codes, uint8_t *scales, hipStream_t s);
hipError_t launch_cast_bf16(const sshdp_plan &p, const float *w, uint16_t *out, hipStream_t s);
hipError_t launch_rs_reduce(const void *const *inputs, int n_in, int in_bf16, void *out, int out_sr, int64_t n,
                            uint64_t seed, uint64_t ctr, int64_t g0, hipStream_t s);
hipError_t launch_rs_accumulate(const void *const *inputs, int n_in, int in_bf16, float *g, int64_t n, int first,
                                hipStream_t s);
}  // namespace sshdp
