/*
 * sshdp.h -- C ABI of libsshdp.so: one GPU's share of the SS-HSDP update phase
 * on MI355X (gfx950).
 *
 * Sources, cited by title and section:
 *   [SS-HSDP]  "SS-HSDP: Efficient and Flexible Sharded Data Parallelism via
 *              Runtime-Update Decoupling" (arXiv:2611.16467v1)
 *   [OCP-MX]   OCP Microscaling Formats (MX) v1.0, the MXFP format cited there
 *
 * What the library computes.  [SS-HSDP §2.1]: an optimizer update F maps
 * (main weight, main gradient, optimizer state) to new main weight and state,
 * and weight preparation G casts or quantises the main weight into the
 * low-precision runtime weight and its scales.  [SS-HSDP §3.1, EG1]: for Muon,
 * F = [f0, f1, f2] per update unit (one attention head, one matrix): f0 updates
 * the momentum and writes a BF16 intermediate u, f1 runs Newton-Schulz on u and
 * produces an FP32 direction v, f2 updates the main weight from v; G produces
 * FP8 (E4M3) weights with UE8M0 scales, and the weight transform Tw packs the
 * head weights into the runtime weight (a view, no copy [SS-HSDP §3.2, §4.2])
 * and relays the scales out for the GEMM kernel.  [SS-HSDP §5.2]: AdamW updates
 * the parameters Muon does not.
 *
 * Data model.  Every field (main weight, gradient, momentum, AdamW second
 * moment, FP8 codes) is ONE flat root allocation indexed by the same element
 * offsets; views are described by a data tree [SS-HSDP §3.2 "Data Tree"]: a
 * child is a view at an element offset inside its parent, only the root owns
 * storage.  Codes mirror the fp32 root byte-for-element, so a head's codes are a
 * sub-range of its packed projection's codes.  Scales are one E8M0 byte per
 * 1x32 block (row-major or the 32x128 tile layout) or per 32x32 block (see
 * SSHDP_SCALE_*).
 *
 * Conventions.  All functions return an int status: SSHDP_OK (0) or a negative
 * SSHDP_ERR_* code; sshdp_status_string() names it.  Device pointers are
 * caller-owned, must stay valid until the enqueued work has run, and must be
 * 16-byte aligned.  `stream` is a hipStream_t passed as void* (NULL = the
 * default stream); every launching call is asynchronous on it, performs no
 * allocation and no synchronisation.  Newton-Schulz groups of one call may run
 * on up to three plan-owned side streams (default priority) that are forked
 * from and joined back into `stream` with events, so the call behaves as one
 * ordered unit of work on `stream` (and can be captured into a HIP graph).
 * Calls with one plan use its side streams: issue them from one host thread,
 * in order (their work is then ordered as issued).  Calls sharing a workspace
 * are serialised by the caller's stream order.  The library keeps no state
 * between calls: the step counter is an argument.
 */
#ifndef SSHDP_H
#define SSHDP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSHDP_ABI_VERSION 6

/* Status codes.  The planning errors are the rejections of [SS-HSDP Appendix A,
 * Table 4]: incompatible metadata, invalid geometry, storage overlap. */
enum {
  SSHDP_OK = 0,
  SSHDP_ERR_ARG = -1,       /* null pointer, empty table, step < 1, bad option value   */
  SSHDP_ERR_TREE = -2,      /* a parent index is not an earlier node                   */
  SSHDP_ERR_BOUNDS = -3,    /* a view leaves its parent or the root                    */
  SSHDP_ERR_OVERLAP = -4,   /* two units, or two quantised regions, share an element   */
  SSHDP_ERR_SCHEMA = -5,    /* geometry/metadata the kernels cannot take (see below)   */
  SSHDP_ERR_ALIGN = -6,     /* a device pointer is not 16-byte aligned                 */
  SSHDP_ERR_WORKSPACE = -7, /* workspace missing or smaller than sshdp_plan_info says  */
  SSHDP_ERR_HIP = -8,       /* a HIP runtime call or kernel launch failed              */
  SSHDP_ERR_STATE = -9,     /* the plan was made host-only and cannot launch           */
  SSHDP_ERR_SCRATCH = -10   /* the plan needs more workspace than the built-in scratch  */
};

enum { SSHDP_OPT_NONE = 0, SSHDP_OPT_MUON = 1, SSHDP_OPT_ADAMW = 2 };

/* Scale layouts.  For a quantised region at absolute element offset o with N
 * rows and K columns (KB = K/32 blocks per row), the scale of block (n, kb):
 *   ROWMAJOR : o/32 + n*KB + kb             (= index of its first element / 32)
 *   TILE32X4 : o/32 + ((n/32)*(KB/4) + kb/4)*128 + (n%32)*4 + kb%4
 * TILE32X4 stores each 32-row x 128-column tile's scales as one 128-byte run,
 * one 4-byte word per row holding 4 consecutive K-blocks: the operand a 32-row
 * scaled-MFMA tile reads in one coalesced load.  It is this library's own
 * layout (the [SS-HSDP] kernels' layout belongs to other hardware).  Both
 * layouts keep a head's scales a sub-range of its projection's when the head's
 * row count is a multiple of 32.
 *
 * BLOCK32X32 is the other block shape [SS-HSDP §3.1 EG1] (and [veScale §6])
 * describe: one scale per 32-row x 32-column block, the least-e rule over the
 * block's 1024 elements, codes as above; block (bn, bk) of a region at o with
 * K columns has its scale at  o/1024 + bn*(K/32) + bk.  The blocks of X^T are
 * the transposes of X's, so the same codes serve the transposed operand.  The
 * scale array then holds (root_numel + 1023)/1024 bytes, and AdamW is never
 * fused with G (the AdamW units run first, then G). */
enum { SSHDP_SCALE_ROWMAJOR = 0, SSHDP_SCALE_TILE32X4 = 1, SSHDP_SCALE_BLOCK32X32 = 2 };

/* Plan flags.  The Newton-Schulz tile policy is a tuning knob (results stay
 * within the Newton-Schulz tolerance either way, not bit-identical): by default
 * a group's products run in 256 x 256 tiles over their largest 256-aligned
 * leading block when the group is large enough to fill the GPU with them, and
 * in 128 x 128 tiles elsewhere.  Setting both tile flags is an argument error.
 * Gram products that run in 128-tiles read X^T (so only X^T is stored) unless
 * SSHDP_PLAN_NS_GRAM_NT is set or X^T of the unit exceeds 2^31 bytes.  Groups
 * other than the largest run on side streams while the largest group's
 * launches fill fewer than two rounds of the GPU's workgroup slots in some
 * stage; otherwise only the groups with r_pad == 128 do (on one side stream)
 * and the rest share the caller's stream.  SSHDP_PLAN_NS_ONE_STREAM keeps
 * every group on the caller's stream. */
enum {
  SSHDP_PLAN_HOST_ONLY = 1,       /* plan and validate on the host; no device tables (cannot launch) */
  SSHDP_PLAN_NS_TILES_SMALL = 2,  /* every Newton-Schulz product in 128 x 128 tiles                  */
  SSHDP_PLAN_NS_TILES_LARGE = 4,  /* 256 x 256 tiles over every 256-aligned leading block            */
  SSHDP_PLAN_NS_GRAM_NT = 8,      /* every Gram reads X row-major (X and X^T stored); for comparison */
  SSHDP_PLAN_NS_ONE_STREAM = 16   /* every Newton-Schulz group on the caller's stream, none on side streams */
};

/* One data-tree node [SS-HSDP §3.2]: a 2-D view (rows x cols, cols contiguous,
 * rows `row_stride` elements apart) at `offset` elements from its parent's first
 * element.  A 1-D tensor is rows = 1.  `is_unit` marks an update parameter (a
 * leaf of the optimisation [SS-HSDP §3.1]) with `optimizer` SSHDP_OPT_MUON or
 * SSHDP_OPT_ADAMW; `quantize` marks a region (a runtime weight, or a unit)
 * that G turns into its runtime form [SS-HSDP §2.1: G casts or quantises the
 * main weight]: SSHDP_G_MXFP8 requantises it to MXFP8 (codes + scales),
 * SSHDP_G_BF16 casts it to bfloat16 (w_bf16).  Rules (else the error named):
 *   parent is -1 or an earlier node index                          (TREE)
 *   rows, cols >= 1, offset >= 0, row_stride >= cols if rows > 1   (SCHEMA)
 *   the view lies inside its parent's extent and the root           (BOUNDS)
 *   a Muon unit is 2-D (rows, cols >= 2) and its first element, row_stride
 *     and cols are multiples of 4 (16-byte vectors); rows, cols <= 4194176
 *     (a 256-row bf16 panel of that length spans < 2^31 bytes)     (SCHEMA)
 *   quantize is SSHDP_G_NONE, SSHDP_G_MXFP8 or SSHDP_G_BF16          (SCHEMA)
 *   an MXFP8 region is contiguous (row_stride == cols), with cols and its
 *     first element multiples of 32; for TILE32X4 also rows % 32 == 0 and
 *     cols % 128 == 0; for BLOCK32X32 also rows % 32 == 0 and the
 *     first element a multiple of 1024                              (SCHEMA)
 *   a BF16 region is contiguous, with cols and its first element
 *     multiples of 8 (16-byte stores)                               (SCHEMA)
 *   units are pairwise disjoint; G regions (both kinds) too        (OVERLAP)
 * Checks run node by node in index order; overlap is checked last. */
typedef struct {
  int32_t parent;
  int32_t is_unit;
  int64_t offset;
  int64_t rows;
  int64_t cols;
  int64_t row_stride;
  int32_t optimizer;
  int32_t quantize;
} sshdp_node;

enum { SSHDP_G_NONE = 0, SSHDP_G_MXFP8 = 1, SSHDP_G_BF16 = 2 };

/* Plan options.  Defaults (sshdp_default_opts): 5 Newton-Schulz steps with
 * (a, b, c) = (3.4445, -4.7750, 2.0315) on the Frobenius-normalised u, ns_eps =
 * 1e-7 added to the norm, heavy-ball momentum (nesterov = 0), update scale mode
 * 0 (scale 1; mode 1: sqrt(max(1, rows/cols)); mode 2: 0.2*sqrt(max(rows,
 * cols))), ROWMAJOR scales, flags 0. */
typedef struct {
  int32_t ns_steps;
  float ns_a, ns_b, ns_c;
  float ns_eps;
  int32_t scale_layout;
  int32_t nesterov;
  int32_t muon_scale_mode;
  uint32_t flags;
} sshdp_plan_opts;

/* Muon: m <- momentum*m + g; u = bf16(m) (nesterov: bf16(g + momentum*m));
 * v = NS(u); w <- w - lr*weight_decay*w - lr*scale*v. */
typedef struct { float lr, momentum, weight_decay; } sshdp_muon_hp;

/* AdamW: w <- w - lr*wd*w; m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
 * w <- w - lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps). */
typedef struct { float lr, beta1, beta2, eps, weight_decay; } sshdp_adamw_hp;

/* Caller-owned device roots, all indexed by the same element offsets.
 * w_main, grad, mom (Muon momentum and AdamW first moment): fp32, root_numel
 * elements.  adam_v: fp32 root or NULL when the plan has no AdamW units.
 * codes: uint8 root of root_numel bytes (E4M3FN).  scales: uint8, at least
 * sshdp_plan_stats.scale_bytes bytes (E8M0).  w_bf16: bfloat16 root of
 * root_numel elements, or NULL when the plan has no BF16 regions.  Only unit
 * elements of w_main, mom, adam_v, MXFP8-region bytes of codes/scales and
 * BF16-region elements of w_bf16 are written. */
typedef struct {
  float *w_main;
  const float *grad;
  float *mom;
  float *adam_v;
  uint8_t *codes;
  uint8_t *scales;
  uint16_t *w_bf16;
} sshdp_buffers;

typedef struct sshdp_plan sshdp_plan;   /* opaque; owns host tables and one device table block */

/* Figures a caller needs to size buffers, and the algorithmic work per step. */
typedef struct {
  int64_t root_numel;
  int64_t scale_bytes;        /* bytes of the scale root: ceil(root_numel / 32)            */
  int64_t workspace_bytes;    /* device workspace sshdp_update_muon/_step need (256-aligned) */
  int32_t n_nodes, n_units, n_muon_units, n_adamw_units, n_quant_regions, n_groups;
  int64_t muon_elems, adamw_elems, quant_elems;
  int64_t fused_quant_elems;  /* MXFP8 elements G handles inside the AdamW pass           */
  double ns_flops;            /* steps*(4 r^2 c + 2 r^3) summed over Muon units: the dense count */
  double ns_tile_flops;       /* MFMA flops the tile schedule executes per step (symmetric Gram and
                                 poly computed as tm <= tn tiles; padding to the tile included; units
                                 whose momentum is all zero skip theirs at run time)             */
  int64_t cast_elems;         /* elements of BF16 regions                                  */
  int32_t n_cast_regions;
  int32_t pad_;
} sshdp_plan_stats;

/* One Newton-Schulz batch: the Muon units sharing an oriented shape r x c
 * (r = min(rows, cols)), run as one batched GEMM per stage [SS-HSDP §4.1]. */
typedef struct {
  int32_t r, c;               /* oriented shape                                            */
  int32_t r_pad, c_pad;       /* padded to a multiple of 128                               */
  int32_t n_units;
  int32_t tile;               /* largest macro-tile edge of the update product (128 or 256) */
  int32_t tile_gram;          /* largest macro-tile edge of the Gram and polynomial products */
  int32_t gram256;            /* Gram/poly rows and columns [0, gram256) run in 256-tiles,  */
                              /* the rest in 128-tiles (0: all 128)                          */
  int32_t upd256_rows;        /* update rows [0, upd256_rows) x columns [0, upd256_cols)    */
  int32_t upd256_cols;        /* run in 256-tiles, the rest in 128-tiles                     */
  int32_t gram_kmajor;        /* 1: the Gram reads X^T (K-major) and X itself is not stored  */
  int32_t split_b;            /* 1 (groups with r_pad == 128): the polynomial B goes to memory  */
                              /* as a bf16 pair, its rounding and the remainder, and the update */
                              /* contracts over both (twice the update's K)                     */
  int32_t lane;               /* stream the group runs on: 0 = the caller's, 1.. = side streams */
} sshdp_group_info;

/* Fill *opts with the defaults above. */
int sshdp_default_opts(sshdp_plan_opts *opts);

/* Resolve the data tree and build a plan [SS-HSDP §3.2 "Data Tree"; §3.3
 * groups; Appendix A Table 4 rejections].  Host-synchronous; unless
 * SSHDP_PLAN_HOST_ONLY, allocates and uploads one block of device descriptor
 * tables on the current HIP device.  Errors leave *out_plan NULL and touch no
 * device memory.  The plan is freed by sshdp_plan_destroy, which releases its
 * device tables and side streams: call it only once the work enqueued with the
 * plan has completed. */
int sshdp_plan_views(const sshdp_node *nodes, int32_t n_nodes, int64_t root_numel,
                     const sshdp_plan_opts *opts, sshdp_plan **out_plan);

int sshdp_plan_info(const sshdp_plan *plan, sshdp_plan_stats *stats);
int sshdp_plan_group(const sshdp_plan *plan, int32_t group, sshdp_group_info *info);
/* Absolute element offset of node `node` (accumulated along its chain) and the
 * Newton-Schulz group of a Muon unit (-1 otherwise). */
int sshdp_plan_node(const sshdp_plan *plan, int32_t node, int64_t *abs_offset, int32_t *group);
void sshdp_plan_destroy(sshdp_plan *plan);

/* F for every Muon unit: f0 (momentum, bf16 u, ||u||^2), f1 (Newton-Schulz,
 * batched bf16 MFMA GEMMs per group) and f2 (main-weight update, fused into the
 * last Newton-Schulz product) [SS-HSDP §3.1 EG1, §4.1].  Reads grad, mom,
 * w_main; writes mom, w_main.  `workspace`: device memory of at least
 * stats.workspace_bytes, 256-byte aligned; its contents on entry are ignored.
 * Errors (nothing is launched): ARG (null plan/bufs/hp/grad/mom/w_main, or the
 * current device is not the plan's), STATE (host-only plan), ALIGN, WORKSPACE
 * (null or too small); HIP if a launch fails. */
int sshdp_update_muon(const sshdp_plan *plan, const sshdp_buffers *bufs, const sshdp_muon_hp *hp,
                      void *workspace, size_t workspace_bytes, void *stream);

/* F for every AdamW unit at step `step` (>= 1, caller-owned, same for all
 * units) [SS-HSDP §5.2: the parameters Muon does not take -- 1-D and
 * elementwise ones -- are updated by AdamW; Appendix B.1: AdamW is the
 * optimizer of every performance run].  The pages write no AdamW formula; the
 * form is the sshdp_adamw_hp one above (decay lr*wd on the pre-update weight,
 * bias-corrected moments, eps after the square root), elementwise in fp32.
 * Reads grad, mom, adam_v, w_main; writes mom, adam_v, w_main.
 * Errors: ARG (null pointers, step < 1, wrong device), STATE, ALIGN; HIP. */
int sshdp_update_adamw(const sshdp_plan *plan, const sshdp_buffers *bufs, const sshdp_adamw_hp *hp,
                       int64_t step, void *stream);

/* G + the scale part of Tw for every quantised region [SS-HSDP §3.1 EG1; OCP-MX]:
 * per 1x32 block along K, e = least integer with amax <= 448*2^e (clamped to
 * [-127,127]; all-zero block -> -127), scale byte e+127 at the layout's index,
 * codes = E4M3FN round-to-nearest-even of x*2^-e, written at the elements' own
 * offsets.  A block holding NaN/Inf gets scale 0xFF and codes 0x7F.  Reads
 * w_main; writes codes and scales.  A plan without MXFP8 regions returns OK at
 * once.  Errors: ARG (null pointers, wrong device), STATE, ALIGN (w_main or
 * codes); HIP. */
int sshdp_requant_mxfp8(const sshdp_plan *plan, const float *w_main, uint8_t *codes, uint8_t *scales,
                        void *stream);

/* G for every BF16 region [SS-HSDP §2.1]: w_bf16 = bfloat16(w_main), round to
 * nearest even, at the elements' own offsets (a runtime view of a BF16 weight
 * is the same sub-range of w_bf16).  Reads w_main; writes w_bf16.  A plan
 * without BF16 regions returns OK at once.  Errors: ARG, STATE, ALIGN; HIP. */
int sshdp_cast_bf16(const sshdp_plan *plan, const float *w_main, uint16_t *w_bf16, void *stream);

/* The reduce-scatter tail [SS-HSDP §4.3 "Reduce-Scatter", Figure 5(e)]: within
 * a node, the slices of one output partition arriving from several ranks are
 * summed in FP32 by a local reducer; the partial stays FP32 or, for BF16
 * gradients, is stored as BF16 with stochastic rounding; the final FP32
 * reduction accumulates straight into the persistent gradient buffer (G'z2),
 * with no result buffer and no separate addition pass.  On one GPU the slices
 * are device buffers (what peer copies deliver).
 *
 * `inputs`: host array of n_inputs (1..8) device pointers, each n elements of
 * in_dtype (SSHDP_RS_FP32 or SSHDP_RS_BF16), summed left to right, every
 * addition rounded to FP32.  n % 16 == 0 and every pointer 16-byte aligned.
 *
 * sshdp_rs_reduce writes the sum to `out` as FP32 (SSHDP_RS_OUT_FP32) or as
 * BF16 with stochastic rounding (SSHDP_RS_OUT_BF16_SR): the fp32 bit pattern
 * plus a 16-bit random, truncated to its upper half (NaN kept), i.e. away from
 * zero with probability (discarded bits)/2^16.  The randoms come from
 * Philox4x64-10 [Salmon et al., SC 2011] with key (seed, 0): element j of the
 * call is element g = g0 + j of the whole tensor (g0 % 16 == 0) and uses word
 * (g/4) % 4, bits 16*(g%4), of the block at counter (g/16 + 1, ctr, 0, 0) --
 * so a rank that restores (seed, ctr) reproduces its partials.
 *
 * sshdp_rs_accumulate: g = in_0 + in_1 + ... when `first` (the first
 * microbatch initialises the buffer), else g = (g + in_0) + in_1 + ....
 *
 * Errors: ARG (null pointer, n_inputs out of range, n < 0, bad dtype/mode),
 * SCHEMA (n or g0 not a multiple of 16), ALIGN. */
enum { SSHDP_RS_FP32 = 0, SSHDP_RS_BF16 = 1 };
enum { SSHDP_RS_OUT_FP32 = 0, SSHDP_RS_OUT_BF16_SR = 1 };
int sshdp_rs_reduce(const void *const *inputs, int32_t n_inputs, int32_t in_dtype, void *out, int32_t out_mode,
                    int64_t n, uint64_t seed, uint64_t ctr, int64_t g0, void *stream);
int sshdp_rs_accumulate(const void *const *inputs, int32_t n_inputs, int32_t in_dtype, float *g, int64_t n,
                        int32_t first, void *stream);

/* The whole update phase in order [SS-HSDP §3.4 "Update"]: Muon F, AdamW F
 * (fused with G for MXFP8 regions holding only AdamW units; the other AdamW
 * units may run on a plan-owned side stream beside the Newton-Schulz work, as
 * they share no element with a Muon unit), then G for the remaining MXFP8
 * regions and the BF16 regions.  Equivalent to
 * sshdp_update_muon; sshdp_update_adamw; sshdp_requant_mxfp8; sshdp_cast_bf16.
 * Every argument the plan's parts need is checked before anything is launched
 * (the errors of those calls); mh may be NULL for a plan without Muon units
 * and ah for one without AdamW units. */
int sshdp_update_step(const sshdp_plan *plan, const sshdp_buffers *bufs, const sshdp_muon_hp *mh,
                      const sshdp_adamw_hp *ah, int64_t step, void *workspace, size_t workspace_bytes,
                      void *stream);

/* sshdp_update_step without caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a device array built
 * into the library, SSHDP_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the
 * library runs on, held until the process ends; its address is looked up on
 * the first call on each device.  The call allocates nothing (with
 * sshdp_profile_enable on, its timing events are created on first use, as in
 * every launching call).  Plans whose stats.workspace_bytes exceed the array
 * are refused (SSHDP_ERR_SCRATCH) before anything is launched.  Every call on
 * a GPU shares that GPU's array and leaves its contents behind (nothing in it
 * needs to start at zero: each step writes the whole region it reads), so
 * calls that may overlap on one GPU -- on different streams or from different
 * threads -- race; order them on one stream.  Otherwise it is exactly
 * sshdp_update_step: same arguments, results and other errors. */
#define SSHDP_NOALLOC_SCRATCH_BYTES (64u << 20)
int sshdp_update_step_noalloc(const sshdp_plan *plan, const sshdp_buffers *bufs, const sshdp_muon_hp *mh,
                              const sshdp_adamw_hp *ah, int64_t step, void *stream);

/* Diagnostics.  The batched NT contraction used by Newton-Schulz, exposed to
 * test it alone: for b < batch, O[b] = bf16(alpha * P[b] Q[b]^T + beta * D[b])
 * with P[b] M x K, Q[b] N x K, O[b] M x N (bf16, row-major, dense, batch strides
 * M*K, N*K, M*N).  D is passed TRANSPOSED, DT[b] N x M (the layout in which the
 * update product reads X), or NULL (beta ignored); OT (optional) receives
 * O[b]^T (N x M).  M, N must be multiples of `tile` (128 or 256), K of 64.
 * tile 1281 / 2561: the same 128 / 256 tiles with both operands K-major (the
 * Gram read from X^T): P[b] K x M, Q[b] K x N row-major, M == N, D NULL.
 * Errors: ARG (null P, Q or O, non-positive sizes, unknown tile, K-major with D
 * or M != N), SCHEMA (sizes not multiples of the tile, or an operand panel that
 * one buffer resource cannot address: tile * K * 2 bytes, K-major
 * ((K - 1) * M + tile) * 2 bytes, at least 2^31), ALIGN. */
int sshdp_gemm_bf16_nt(const void *P, const void *Q, const void *D, void *O, void *OT, int32_t M,
                       int32_t N, int32_t K, int32_t batch, float alpha, float beta, int32_t tile,
                       void *stream);

/* Diagnostics.  What the Newton-Schulz tile schedule executed in the last
 * sshdp_update_muon / sshdp_update_step that used `workspace`: a unit whose
 * momentum was all zero has direction 0 and skips every product, so only the
 * other units count.  `units_per_group` (n_groups entries, or NULL) receives
 * each group's count of such units; `flops` (or NULL) the MFMA flops their
 * tiles executed in that step (stats.ns_tile_flops split per unit, summed over
 * them).  Reads the per-unit normalisation scales the call left in the
 * workspace: enqueues a copy on `stream` and synchronises with it.  Errors: ARG
 * (null plan, wrong device), STATE, WORKSPACE (null or smaller than
 * stats.workspace_bytes); HIP. */
int sshdp_ns_executed(const sshdp_plan *plan, const void *workspace, size_t workspace_bytes,
                      int32_t *units_per_group, double *flops, void *stream);

/* Per-stage kernel timing for benchmarking: when enabled on a plan, launching
 * calls bracket each kernel class with HIP events on the launch stream and
 * accumulate durations (milliseconds) and bracket counts; reading synchronises
 * on those events, returns the sums since the previous read and clears them.
 * Classes: 0 momentum (f0), 1 norm, 2 NS Gram, 3 NS poly,
 * 4 NS update (+f2), 5 AdamW, 6 AdamW+G fused, 7 G requant, 8 the whole
 * Newton-Schulz phase on the caller's stream (fork to join: NS launches of
 * different groups run concurrently on plan-owned streams, so classes 2-4 can
 * overlap in time), 9 G bf16 cast, and the Newton-Schulz launches of the
 * caller's stream alone (the groups whose sshdp_group_info.lane is 0): 10 Gram
 * and 11 poly (both tile sizes), 12 the update's 256-tile launch in the steps
 * before the last, 13 that launch in the last step (+f2).
 * Not thread-safe; for measurement only. */
enum { SSHDP_PROF_CLASSES = 14 };
int sshdp_profile_enable(sshdp_plan *plan, int32_t enable);
int sshdp_profile_read(sshdp_plan *plan, double *ms, int64_t *launches);

const char *sshdp_status_string(int code);
int sshdp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSHDP_H */
