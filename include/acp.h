/*
 * acp.h -- pipelined asynchronous tile copy + elementwise for AMD MI355X (gfx950).
 *
 * A small C ABI over operations on multi-dimensional tiles staged in LDS:
 *
 *   acp_tile_copy           global -> LDS -> global
 *   acp_tile_ewise          elementwise op on LDS-resident operand tiles
 *   acp_stream_ewise        tiles streamed through a 2..4-stage LDS ring
 *   acp_tile_reduce         staged tiles added into a destination
 *   acp_stream_binary       two tensors streamed through one ring (add, mul)
 *   acp_stream_reduce_rows  row sums of ring-staged tiles
 *
 * plus the host-side descriptor encoder / planner they share.  The method
 * follows four pages:
 *   [tma]    "copy_async -> tma"            (TVM TIRx docs)
 *   [smem]   "elementwise -> smem"          (TVM TIRx docs)
 *   [ldgsts] "copy_async -> ldgsts"         (TVM TIRx docs)
 *   [cb]     "Add TMA support for circular buffering pass" (nvFuser PR #2833)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Status.  Every call returns an acp_status; nothing throws across the ABI.
 *   ACP_ERR_INVALID      malformed request (null pointer, bad enum, shape or
 *                        operand mismatch) -- the "anything else is an error"
 *                        class of [tma] "Algorithm" step 1;
 *   ACP_ERR_DECLINED     well formed, but no legal plan exists ([tma] final
 *                        paragraph of "How inputs change the algorithm";
 *                        [ldgsts] "the variant declines");
 *   ACP_ERR_UNSUPPORTED  op / dtype combination outside the registry
 *                        ([smem] "What it accepts": check_extras), or a plan
 *                        beyond this library's kernel limits;
 *   ACP_ERR_LDS          the staged tiles do not fit the device's LDS;
 *   ACP_ERR_HIP          a HIP runtime call or kernel launch failed.
 *   acp_last_error() returns the reason for the calling thread's last
 *   non-OK status (the pages' predicates return an (ok, reason) pair).
 * Ownership.  Descriptors are caller-owned plain data; the library keeps no
 *   reference to them after a call returns.  A descriptor embeds the tensor's
 *   device address, so the tensor must outlive every enqueued use and moving
 *   the tensor means encoding again ([tma] "Algorithm" step 3: encoded once
 *   on the host, reused by the caller).  Device pointers and streams are
 *   borrowed.
 * Asynchrony.  Compute calls validate and plan on the host (errors return
 *   synchronously), then enqueue one kernel on `hip_stream` (a hipStream_t;
 *   NULL = the null stream) and return.  Nothing is allocated and nothing
 *   else is enqueued, so a call can be captured into a HIP graph.  Completion is stream order; the
 *   caller synchronizes.  Inside a kernel the library owns every wait: unlike
 *   the pages' copy_async (whose caller commits and waits), completion of
 *   the staged loads is tracked by the kernel itself.
 * Threads.  `threads` is the workgroup size: a multiple of 64 (one gfx950
 *   wavefront) from 64 to 1024.
 * Layout.  Shapes, strides and boxes are outermost-first; strides are in
 *   elements; the innermost stride must be 1.  Out-of-bounds elements of a
 *   partial tile read as zero and are never written.
 */
#ifndef ACP_H
#define ACP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ACP_ABI_VERSION 1
#define ACP_MAX_INPUT_RANK 8   /* rank of a tensor handed to the encoder */
#define ACP_MAX_RANK 5         /* descriptor rank after planning ([tma] "What it accepts") */
#define ACP_MAX_BOX 256        /* per-dimension box limit ([cb] "Lowering Details") */
#define ACP_MAX_ISSUES 256     /* loads per tile the kernels index (a library limit) */
#define ACP_MAX_IMAGE_AXES 12  /* axes of a tile's LDS image the kernels index (a library limit) */
#define ACP_MAX_EWISE_INPUTS 3

typedef enum {
  ACP_OK = 0,
  ACP_ERR_INVALID = 1,
  ACP_ERR_DECLINED = 2,
  ACP_ERR_UNSUPPORTED = 3,
  ACP_ERR_LDS = 4,
  ACP_ERR_HIP = 5
} acp_status;

typedef enum { ACP_U8 = 0, ACP_U16 = 1, ACP_U32 = 2, ACP_U64 = 3, ACP_F16 = 4, ACP_F32 = 5 } acp_dtype;

/* LDS layout of a staged tile.  ACP_SWIZZLE_128B carries the mode number of
 * [tma]'s worked example (3): 16-byte chunk index XOR (128-byte row index
 * mod 8) on stage-relative LDS byte offsets.  Modes 1 and 2 follow the mode
 * numbering ([tma] "How inputs change the algorithm": the mode sets the
 * innermost-box constraint): mode m permutes the 2^m 16-byte chunks of each
 * 16 * 2^m-byte span by XOR with the 128-byte row index mod 2^m, and an
 * innermost box wider than 16 * 2^m bytes is split into atoms of that width. */
typedef enum { ACP_SWIZZLE_NONE = 0, ACP_SWIZZLE_32B = 1, ACP_SWIZZLE_64B = 2, ACP_SWIZZLE_128B = 3 } acp_swizzle;

/* Out-of-bounds fill: zero, the last encode argument of [tma]'s example. */
typedef enum { ACP_OOB_ZERO = 0 } acp_oob;

/* Op registry ([smem] "What it accepts", "How inputs change the algorithm"):
 *   ZERO  y = +0                     SQRT  y = sqrt(x)      EXP  y = exp(x)
 *   ADD   y = x0 + x1                MUL   y = x0 * x1
 *   FMA   y = x0 * x1 + x2 (fused, one rounding)
 * For acp_stream_ewise the second and third operands are per-row scalars:
 *   ADD y = x + b[row], MUL y = a[row] * x, FMA y = a[row] * x + b[row].
 * COPY (acp_tile_copy only) moves raw bytes. */
typedef enum {
  ACP_OP_ZERO = 0,
  ACP_OP_SQRT = 1,
  ACP_OP_EXP = 2,
  ACP_OP_ADD = 3,
  ACP_OP_MUL = 4,
  ACP_OP_FMA = 5,
  ACP_OP_COPY = 6
} acp_op;

/* Host-encoded tile descriptor (the cuTensorMap of [tma], re-designed):
 * plain data, caller-owned, 256 bytes, 64-byte aligned; contents private. */
typedef struct {
  __attribute__((aligned(64))) unsigned char opaque[256];
} acp_tile_desc;

/* What the planner chose for one tile of a descriptor ([tma] "Algorithm"
 * step 2, [smem] "Algorithm" step 2, [ldgsts] "Algorithm" step 1). */
typedef struct {
  int32_t rank;              /* descriptor rank, <= 5 */
  int32_t desc_elem_bytes;   /* element size after promotion (copies only) */
  int64_t dims[ACP_MAX_RANK];    /* innermost-first, in desc elements */
  int64_t strides[ACP_MAX_RANK]; /* bytes, innermost-first; strides[0] == desc_elem_bytes */
  int32_t box[ACP_MAX_RANK];     /* innermost-first, in desc elements */
  int32_t issues;            /* loads per tile (product of the issue axes) */
  int32_t n_issue_axes;
  int32_t n_image_axes;      /* axes of the tile's LDS image */
  int32_t swizzle;           /* acp_swizzle */
  int32_t promoted;          /* 1 when the element type was widened */
  int32_t threads;           /* partition; all four are 0 when threads == 0 */
  int32_t vec;               /* elements per thread per round */
  int32_t vec_bytes;         /* bytes per thread per round (16 or 4 on gfx950) */
  int32_t outer;             /* rounds: tile elements / (threads * vec) */
  int64_t tile_bytes;        /* bytes of one tile's LDS image */
  int64_t n_tiles;           /* tiles covering the tensor */
} acp_plan_info;

/* ABI version of the loaded library (ACP_ABI_VERSION). */
int acp_abi_version(void);

/* Reason for the calling thread's last non-OK status; "" if none.  The
 * pointer stays valid until the thread's next acp_* call. */
const char* acp_last_error(void);

/* The kernel and launch shape of this thread's last launch attempt of a
 * pipelined entry point, as text ("stream linear grid vec 16 rounds 2 srow
 * 1 variant 0 grid 256 ..."): "none" when that call launched nothing (no
 * tiles, or the launch failed), empty before the first.  A row reduction
 * ends in "wave-local" or "lds partials", the path its stage layout takes.
 * Calls rejected before the launch step leave it unchanged.  Owned by the
 * library; valid until the thread's next such call. */
const char* acp_last_kernel(void);

/* Encode a descriptor for tiles of `box` over a tensor at `gbase`
 * ([tma] "Algorithm" step 3; "Generated TIRx IR" shows the worked call).
 *   out      caller-owned descriptor to fill
 *   dtype    element type
 *   rank     1..ACP_MAX_INPUT_RANK
 *   gbase    device address of element (0, ..., 0); never dereferenced here
 *   shape    rank extents >= 1
 *   strides  rank element strides >= 1, innermost == 1
 *   box      rank tile extents >= 1 (may exceed 256: the planner splits it)
 *   swizzle  LDS layout of the staged tile
 *   oob      ACP_OOB_ZERO
 * Runs the box-level plan search.  The search always shrinks a plan to rank
 * <= 5 (outer dims become loads of their own) and cuts an innermost box that
 * does not fit the swizzle atom into loads that do ([tma] "Algorithm" step
 * 2), so it returns ACP_ERR_DECLINED only when no legal descriptor exists:
 * innermost stride != 1, or under a swizzle an innermost box (merged rows
 * included) that is no whole number of 16-byte chunks.  A legal plan beyond
 * what the kernels index (more than ACP_MAX_ISSUES loads per tile or
 * ACP_MAX_IMAGE_AXES image axes) is ACP_ERR_UNSUPPORTED.  Pure host code. */
acp_status acp_encode_tiled(acp_tile_desc* out, acp_dtype dtype, int rank, const void* gbase,
                            const int64_t* shape, const int64_t* strides, const int32_t* box,
                            acp_swizzle swizzle, acp_oob oob);

/* Report the plan of `desc` for a workgroup of `threads` (0: descriptor
 * only).  `copy_only` != 0 allows element-type promotion (byte copies);
 * elementwise plans never promote.  Pure host code. */
acp_status acp_plan_query(const acp_tile_desc* desc, int threads, int copy_only, acp_plan_info* out);

/* Copy every tile of `src` to the same coordinates of `dst` through LDS:
 * direct-to-LDS loads (16 or 4 bytes per lane, swizzled per `src`), a
 * per-wave completion wait, then LDS reads and coalesced stores
 * ([tma] and [ldgsts] "Demonstration program").  One workgroup per tile
 * while the tiles fit one grid of one workgroup per CU; beyond that a
 * persistent grid (one workgroup per CU, environment ACP_TILE_WG_PER_CU)
 * walks tiles w, w+G, ... through a 2-slot ring (ACP_TILE_STAGES); tiles
 * narrower than a 128-byte line are staged side by side in pairs (or
 * fours), and a workgroup whose staged rows are whole lines takes a run of
 * consecutive tiles instead (ACP_BLOCKED_COPY=0: the cyclic walk).  The
 * result does not depend on the walk.
 * `src` and `dst` must have equal dtype, shape and box ([tma]
 * validate_copy_op); `dst` may have other strides.  ACP_ERR_INVALID when
 * the byte ranges of src and dst (base to last element) intersect. */
acp_status acp_tile_copy(const acp_tile_desc* src, const acp_tile_desc* dst, int threads,
                         void* hip_stream);

/* out = op(in[0], ..., in[n_in-1]) tile by tile with every operand staged
 * in LDS and the result written to an LDS tile before it is copied out
 * ([smem]).  n_in: ZERO 0 or 1, SQRT/EXP 1, ADD/MUL 2, FMA 3.  All inputs
 * share dtype, shape, strides, box and swizzle (one anchor layout); `out`
 * has the same shape and box.  Types: SQRT/EXP f16|f32 -> f16|f32,
 * computed in f32 and rounded to the output type; ADD/MUL/FMA inputs and
 * output one of f16|f32; ZERO -> f16|f32.  Large
 * tile counts run on a persistent grid whose ring trips stage 1, 2 or 4
 * consecutive tiles (about 16 KiB per trip; ACP_TILES_PER_TRIP): one
 * workgroup per CU when the tiles form a linear grid, else about 32 KiB of
 * loads in flight per CU (ACP_TILE_WG_PER_CU overrides both).  `out`
 * may be an input element for element (same base, element size and
 * strides: the op runs in place); any other intersection of the output's
 * byte range with an input's is ACP_ERR_INVALID. */
acp_status acp_tile_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* const* in,
                          int n_in, int threads, void* hip_stream);

/* Stream the tiles of `x` through an LDS ring of `stages` (2..4) buffers
 * ([cb] "Loop Structure"): a prologue issues stages-1 loads, the main loop
 * issues the load of trip i+stages-1 into stage (i+stages-1) % stages and
 * then waits for stage i % stages, the epilogue drains.  Each trip stages a
 * `stage_box` sub-box of x's box (x's box is the workgroup tile; stage_box
 * must divide it per dim; its planned load count may exceed one).
 *   op          ZERO, SQRT, EXP (x f16|f32 -> out f16|f32) or
 *               ADD, MUL, FMA (x and out f32, per-row scalars)
 *   out         same shape and box as x; any strides; its byte range must
 *               not intersect x's or a row array's (else ACP_ERR_INVALID)
 *   row_a/row_b device float32 arrays over x's outer dims (shape[:-1],
 *               packed row-major); FMA needs both, MUL row_a, ADD row_b;
 *               NULL otherwise
 *   workgroups  0: one workgroup per tile of x; G > 0: G persistent
 *               workgroups, workgroup w walks tiles w, w+G, ... with one
 *               continuous ring
 * Completion per stage is the wave's in-order count of outstanding memory
 * operations (s_waitcnt vmcnt) in place of the pages' per-stage barriers. */
acp_status acp_stream_ewise(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x,
                            const float* row_a, const float* row_b, const int32_t* stage_box,
                            int stages, int threads, int workgroups, void* hip_stream);

/* Store with reduce-add ([tma] "How inputs change the algorithm": a shared
 * -> global copy with a reduce op, e.g. add): every tile of `src` is staged
 * in LDS by direct-to-LDS loads and added element by element into `dst`
 * with no-return buffer atomics.
 *   op    ACP_OP_ADD
 *   src   u32, f32 or f16
 *   dst   same dtype, rank and box; each extent equal to src's, or 1 where
 *         src's box is 1: every source tile along such a dim adds into the
 *         same destination elements (a sum over that dim); its byte range
 *         must not intersect src's (else ACP_ERR_INVALID)
 * dst'[j] = dst[j] + sum of the src elements mapped to j; u32 wraps modulo
 * 2^32.  Floating-point additions land in no fixed order: the result is
 * the exactly rounded sum whenever every partial sum is representable (in
 * particular with one contribution per element).  Tile counts above the
 * grid run on a persistent grid: workgroup w walks tiles w, w+G, ..., or,
 * when contributions are summed over a dim, a run of whole groups of the
 * tiles that add into one destination tile.  When dst
 * has src's shape and strides (one contribution per element) and the dtype
 * is a float, no atomics are needed: both tensors ride the LDS ring and the
 * sum is stored into dst in place.
 * ACP_ERR_UNSUPPORTED unless the plan has 16-byte rounds and 1, 2, 4 or 8
 * rounds per thread. */
acp_status acp_tile_reduce(acp_op op, const acp_tile_desc* dst, const acp_tile_desc* src, int threads,
                           void* hip_stream);

/* Row reduction over ring-staged tiles ([cb] "Testing Setup": the
 * Reduction and InnerPersistent schedules; a stage may need several loads):
 * out[row] = sum of x[row, :] over the innermost dim, every row of x.
 *   op          ACP_OP_ADD
 *   out         device float32 array over x's outer dims (shape[:-1],
 *               packed row-major, 4-byte aligned, not intersecting x),
 *               written (not accumulated)
 *   x           float16 or float32, rank >= 2; its box and `stage_box` hold
 *               whole rows (innermost box = innermost extent)
 *   stages      2..4; workgroups as for acp_stream_ewise
 * Each lane sums its 16-byte chunks (fixed pairwise order, binary32).  When
 * every 1 KiB wave block of a stage lies in one row and every row in one
 * wave, the wave sums its blocks with cross-lane moves and writes its rows
 * with no barrier; otherwise the chunk partials go through LDS and, after a
 * workgroup barrier, each wave reduces whole rows (lane-strided sums, then
 * the same cross-lane sum).  The order is fixed, so results are
 * deterministic; their error against the exact sum is within the
 * recursive-summation bound for the row length.
 * ACP_ERR_UNSUPPORTED unless the plan has 16-byte rounds and 1, 2, 4 or 8
 * rounds per thread. */
acp_status acp_stream_reduce_rows(acp_op op, float* out, const acp_tile_desc* x, const int32_t* stage_box, int stages,
                                  int threads, int workgroups, void* hip_stream);

/* How the second tensor of a two-tensor stream reaches its ring slot
 * ([cb] "Testing Setup", Pointwise: one tensor on the asynchronous ring,
 * the other "Set", i.e. loaded by ordinary loads and stored into the
 * circular buffer; PointwiseCpAsync: both asynchronous). */
typedef enum { ACP_STAGE_RING = 0, ACP_STAGE_SET = 1 } acp_staging;

/* Stream out = x OP z (op ADD or MUL) through an LDS ring of `stages`
 * (2..4) buffers, as acp_stream_ewise does for one tensor.  x is staged by
 * direct-to-LDS loads; z with ACP_STAGE_RING the same way (both loads of a
 * trip in flight together), with ACP_STAGE_SET by ordinary loads into
 * registers, a wait for all of the wave's outstanding loads, and a store
 * into z's image in the slot.
 *   x, z        float16 or float32, one layout (dtype, shape, strides, box,
 *               swizzle); x's box is the workgroup tile
 *   out         same dtype, shape and box; any strides; its byte range must
 *               not intersect x's or z's (else ACP_ERR_INVALID)
 *   stage_box   sub-box of the tile staged per trip (divides it per dim)
 *   workgroups  0: one workgroup per tile; G > 0: G persistent workgroups
 * Results are the IEEE sum or product of each element pair, rounded once
 * to the operand type.  ACP_ERR_UNSUPPORTED unless the plan has 16-byte
 * rounds and 1, 2, 4 or 8 rounds per thread. */
acp_status acp_stream_binary(acp_op op, const acp_tile_desc* out, const acp_tile_desc* x, const acp_tile_desc* z,
                             const int32_t* stage_box, int stages, int threads, int workgroups,
                             acp_staging z_staging, void* hip_stream);

/* Test export: the raw LDS bytes of tile `tile_index` of `src` after its
 * direct-to-LDS load, written to `out_bytes` (device, tile_bytes long). */
acp_status acp_debug_lds_image(const acp_tile_desc* src, int64_t tile_index, int threads,
                               void* out_bytes, void* hip_stream);

/* Test export: run the ring control of acp_stream_ewise for one wave with
 * `n_iters` trips, `stages` buffers, `loads` and `stores` memory operations
 * per trip, recording 3 * n_iters events of 4 int32 each
 * (kind 0 load / 1 wait / 2 consume, trip, stage, outstanding-op count
 * allowed at the wait) into device memory `out_events`.  The pairs
 * (loads, stores) = (1,1), (2,1), (2,2), (4,1), (4,4) run the ring form whose
 * per-trip counts are compile-time constants (the one the linear-grid kernels
 * use), any other pair the general form; both follow the same schedule. */
acp_status acp_debug_ring_trace(int n_iters, int stages, int loads, int stores, int32_t* out_events,
                                void* hip_stream);

/* Measurement reference (not part of the pipelined path): copy `bytes`
 * (a multiple of 16) from device memory `src` to the non-overlapping device
 * memory `dst` with a plain register-path kernel: no LDS and no ring, each
 * workgroup of 256 threads moving 16 KiB blocks (four 16-byte non-temporal
 * loads per lane, then four stores) in a grid-stride loop.  `workgroups` 0
 * takes one per compute unit.  The caller owns both buffers; the copy is
 * asynchronous on `hip_stream`.  It gives the bandwidth a plain 1:1
 * read/write stream reaches on the device, the practical ceiling against
 * which the ring's streams are compared.  ACP_ERR_INVALID on null pointers,
 * a size that is negative, not a multiple of 16 or at least 2^40, or
 * overlapping buffers. */
acp_status acp_debug_stream_copy(void* dst, const void* src, int64_t bytes, int workgroups, void* hip_stream);

/* Measurement reference (not part of the pipelined path): acp_debug_stream_copy
 * in other shapes and cache policies, so that a sweep shows what a plain
 * register-path copy reaches on the device.  Workgroups of `threads` lanes
 * copy blocks of threads * unroll * 16 bytes w, w+G, ... (each lane issues
 * `unroll` 16-byte loads, then the stores); `load_nt` / `store_nt` 1 give
 * the loads / stores the non-temporal cache policy, 0 the default one;
 * `workgroups` 0 takes one per compute unit (never more than the blocks).
 * Built shapes (threads x unroll): 64x16, 128x8, 256x2, 256x4, 256x8,
 * 512x2, 512x4, 512x8, 1024x2, 1024x4, each with the four policy pairs;
 * 256x4 with both policies non-temporal is acp_debug_stream_copy's kernel
 * shape.  ACP_ERR_UNSUPPORTED for any other combination; ACP_ERR_INVALID as
 * for acp_debug_stream_copy, or for policies other than 0 / 1. */
acp_status acp_debug_stream_copy_shape(void* dst, const void* src, int64_t bytes, int workgroups, int threads,
                                       int unroll, int load_nt, int store_nt, void* hip_stream);

/* Measurement reference with the walk of a persistent tiled copy (not part
 * of the pipelined path): dst = src over a rank-3 tensor `src` (element
 * `src_strides`, innermost 1, 16-byte multiples in bytes) of `esize`-byte
 * elements into a packed tensor `dst` of the same `shape`, with no LDS and
 * no ring.  Tiles are `box` = (1, rows, cols); `tiles_per_trip` neighbouring
 * tiles along the innermost dim form a group, and workgroup w of
 * `workgroups` (0: one per compute unit, never more than the groups) walks
 * the groups in row-major order as acp_tile_copy's persistent grid does: a
 * run of ceil(groups / G) consecutive groups from w * ceil(groups / G) when
 * a group row is whole 128-byte lines, else groups w, w+G, ...  It issues
 * the next group's 16-byte non-temporal loads before the current group's
 * stores (two groups in flight, as in a 2-slot ring).  Edge tiles are
 * clipped to the tensor.  It gives the rate a plain register-path copy
 * reaches over the same tiles and order as acp_tile_copy's persistent grid.  ACP_ERR_INVALID for null
 * pointers, esize not 1/2/4/8, threads not 128/256, tiles_per_trip not
 * 1/2/4, box[0] != 1, rows or groups not whole 16-byte chunks, more than 8
 * chunks per lane and group, misaligned pointers or strides, or
 * overlapping buffers. */
acp_status acp_debug_copy_tiles(void* dst, const void* src, int esize, const int64_t* shape,
                                const int64_t* src_strides, const int32_t* box, int tiles_per_trip, int threads,
                                int workgroups, void* hip_stream);

/* Measurement references for one direction (not part of the pipelined
 * path), with acp_debug_stream_copy's walk: 256-thread workgroups, 16 KiB
 * blocks w, w+G, ..., four 16-byte non-temporal accesses per lane;
 * `workgroups` 0 takes one per compute unit (never more than the blocks).
 * They give the bandwidth the device reaches when it only reads or only
 * writes, the two limits a mixed read/write stream lies between.
 *   acp_debug_stream_read   reads `bytes` from device memory `src`; each
 *                           workgroup w writes the XOR of the 16-byte words
 *                           it read to sums[w] (device, 16 bytes per
 *                           workgroup, not intersecting src)
 *   acp_debug_stream_fill   writes the 32-bit `pattern` over `bytes` of
 *                           device memory `dst`
 * ACP_ERR_INVALID on null pointers, a size that is negative, not a multiple
 * of 16 or at least 2^40, or sums intersecting the source. */
acp_status acp_debug_stream_read(const void* src, int64_t bytes, void* sums, int workgroups, void* hip_stream);
acp_status acp_debug_stream_fill(void* dst, int64_t bytes, uint32_t pattern, int workgroups, void* hip_stream);

/* Measurement reference for a stream that writes two bytes per byte read
 * (not part of the pipelined path): dst[i] = (float)src[i] for `elements`
 * float16 values of contiguous device memory `src` into contiguous device
 * memory `dst` (exact: every float16 is a float32).  256-thread workgroups
 * take 8 KiB input blocks w, w+G, ... (four 8-byte non-temporal loads per
 * lane, each widened into one 16-byte non-temporal store, so every wave
 * instruction covers a contiguous span); `workgroups` 0 takes one per
 * compute unit.  ACP_ERR_INVALID on null pointers, an element count that is
 * negative, not a multiple of 8 or at least 2^38, or overlapping buffers. */
acp_status acp_debug_stream_widen(float* dst, const void* src, int64_t elements, int workgroups, void* hip_stream);

/* Measurement reference with the walk of a tiled widening stream (not part
 * of the pipelined path): dst = (float)src over a rank-5 float16 tensor
 * `src` (element `src_strides`, innermost 1, 8-byte multiples in bytes) into
 * a packed float32 tensor `dst` of the same `shape`, with no LDS and no
 * ring.  One 256-thread workgroup per `box` tile (consecutive tiles on one
 * XCD when the tile count is a multiple of 8) walks the tile's `stage_box`
 * stages in row-major order; a stage spans the two innermost dims only.
 * Each lane takes 4-element pieces of a stage (8-byte loads, two stages in
 * flight) and writes each as one 16-byte non-temporal store.  It gives the
 * rate a plain register-path stream reaches over the same tiles, stages and
 * row pitch as acp_stream_ewise's widening ops.  ACP_ERR_INVALID unless
 * every tile and stage is whole, a stage row holds whole 4-element pieces
 * (at most 2048 per stage), src is 8-byte and dst 16-byte aligned, and the
 * two do not overlap. */
acp_status acp_debug_widen_tiles(float* dst, const void* src, const int64_t* shape, const int64_t* src_strides,
                                 const int32_t* box, const int32_t* stage_box, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* ACP_H */
