// Launch contract between the host API and the stage-ring engine kernels.
//
// One engine runs all three operations: a workgroup walks "trips" (one staged
// sub-box each) through a ring of LDS slots.  tile_copy and tile_ewise run
// one trip per workgroup in a single slot; stream_ewise runs a 2..4-slot ring
// over many trips ("Add TMA support for circular buffering pass", "Loop
// Structure").  Every field is computed on the host by the planner.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace acp {

constexpr int kDims = 8;       // tensor dims the engine indexes
constexpr int kAxes = 12;      // LDS-image axes
constexpr int kMaxOuter = 8;   // rounds per thread per trip
constexpr int kPartial = 4;    // dims that may end in a partial stage
constexpr uint32_t kOobOffset = 0x80000000u;  // buffer offset past num_records: loads 0, stores dropped

struct EngineArgs {
  const char* in[3];   // staged operands (same layout)
  char* out;
  const float* row_a;  // per-row scalars (row ops), never null when staged
  const float* row_b;
  // per tensor dim d < rank
  int64_t xstep[kDims];      // input bytes per stage step along d
  int64_t ostep[kDims];      // output bytes per stage step along d
  int64_t rstep[kDims];      // packed rows per stage step along d (d < rank-1)
  uint32_t sbox[kDims];      // stage box
  uint32_t nst[kDims];       // stages covering the tensor along d
  uint32_t sub[kDims], sub_mag[kDims], sub_sh[kDims];   // stages per tile along d
  uint32_t tgrid[kDims], tg_mag[kDims], tg_sh[kDims];   // tiles along d
  int32_t pslot_of_dim[kDims];  // partial-stage slot of dim d, -1 if its stages are all full
  // partial slots: dims whose last stage is cut by the tensor edge
  uint32_t prem[kPartial];   // valid extent of that last stage (0xFFFFFFFF for unused slots)
  // LDS image axes, outermost-first; strides are per index of the axis
  uint32_t ax_count[kAxes], ax_mag[kAxes], ax_sh[kAxes], ax_step[kAxes];
  uint32_t ax_xs[kAxes];     // input bytes
  uint32_t ax_os[kAxes];     // output bytes
  uint32_t ax_rs[kAxes];     // packed stage rows
  int32_t ax_pslot[kAxes];   // partial slot of the axis' dim, -1 if none
  int32_t rank, n_axes;
  uint32_t subs, subs_mag, subs_sh;  // stages per tile
  uint32_t n_tiles;
  uint32_t tile0;                    // first tile (debug image)
  int32_t esize_log2;                // staged element size
  int32_t outer, waves, stages, n_in;
  int32_t swizzle;           // 0 (none), 1, 3 or 7: row bits XORed into the 16-byte chunk index
  // LDS slot layout (bytes)
  uint32_t in_image_bytes;   // stride between operand images in a slot
  uint32_t out_image_off;    // output image (staged output only), after the ring slots
  uint32_t ab_off;           // per-row scalar area
  uint32_t ab_wave_bytes;    // per wave
  uint32_t slot_bytes;
  int32_t n_rows, ab_instr;  // rows per stage; 4-byte loads per wave per stage for a/b
  int32_t row_ops;
  int32_t xcd_remap;
  // extents (bytes from the tensor base to one past its last element): the
  // buffer resources end there, so no access can leave its tensor
  uint64_t in_span, out_span;
  uint64_t total_rows;       // rows of the per-row scalar arrays
  // Linear stage grid: one stage per tile, no partial stage and a row-major
  // contiguous grid, so stage t starts at t * lin_x input bytes, t * lin_o
  // output bytes and row t * lin_r.  lin == 0 selects the general path.
  int32_t lin;
  int64_t lin_x, lin_o, lin_r;
  // cache policy of the direct-to-LDS loads and of the stores: 0 default,
  // 1 non-temporal (streamed data, no reuse expected)
  int32_t load_nt, store_nt;
  // Row ops whose every 1 KiB wave block lies inside one row: the per-row
  // scalars are read through the scalar cache instead of being staged.
  int32_t row_uniform;
  // General kernel, tile copy / tile ewise on a persistent grid: every ring
  // trip stages 2^tpt_log2 consecutive tiles (each with its own images in
  // the slot), so tiles that share cache lines at their edges are loaded
  // back to back.  Workgroup w takes tile groups w, w+G, ...
  uint32_t tpt_log2;
  // Row reduction: the innermost dim's image axes (bit k for axis k), the
  // 16-byte chunks of one row, rows per stage, the packed row stride of
  // each outer dim, and the LDS double buffer of per-chunk partial sums.
  uint32_t ax_inner_mask;
  uint32_t row_chunks, red_rows, part_off, part_bytes;
  int32_t red_local;         // every wave block lies in one row and every row in one wave
  // Store with reduce-add over batch dims: workgroup w takes the contiguous
  // tiles w * per_wg ... (the per-dim tile arrays list the summed dims
  // last, so consecutive tiles are the red_group contributions to one
  // destination tile); the contributions are summed in registers and added
  // to the destination once per group.  0: round-robin tiles, no grouping.
  uint32_t per_wg, red_group;
  uint32_t rowstr[kDims];
  // Tile ewise on a linear tile grid (linear kernel): a stage is 2^k tiles
  // of 2^tile_rounds_log2 rounds each; round f belongs to tile
  // f >> tile_rounds_log2 of the stage, whose input and output start
  // tile_x and tile_o bytes after the previous tile's.
  uint32_t tile_rounds_log2;
  int64_t tile_x, tile_o;
};

// Which kernel variant a launch needs.
struct KernelKey {
  int op;        // acp_op
  int tin;       // acp_dtype of staged operands
  int tout;      // acp_dtype of the output
  int vec_bytes; // 16 or 4
  int mode;      // 0 copy, 1 tile ewise (output staged in LDS), 2 stream, 3 stream on a linear grid,
                 // 4 / 5 / 6 / 7 / 8: copy / tile ewise / stream / store with reduce-add /
                 // row reduction in the general lean kernel, 9 tile ewise on a linear grid,
                 // 10 wave-local row reduction on a linear grid
  int outer;     // modes 3..10: rounds per thread (1, 2, 4 or 8); 0 otherwise
  int srow;      // modes 3 and 6, row ops: per-row scalars through the scalar cache
  int variant = 0;  // modes 3 and 6, add / mul of two streamed tensors: 1 both on the direct-to-LDS
                    // ring, 2 the second one loaded synchronously ("Set") into its slot
};

// Kernel for `key`, or nullptr when that combination is not built.
const void* engine_kernel(const KernelKey& key);
hipError_t engine_launch(const void* kernel, const EngineArgs& args, unsigned grid, unsigned block,
                         unsigned lds_bytes, hipStream_t stream);
const void* lds_image_kernel(int vec_bytes);
hipError_t lds_image_launch(const void* kernel, const EngineArgs& args, unsigned block, unsigned lds_bytes,
                            void* out_bytes, uint32_t image_bytes, hipStream_t stream);
hipError_t stream_copy_launch(const void* src, void* dst, uint64_t bytes, unsigned grid, hipStream_t stream);
hipError_t stream_read_launch(const void* src, uint64_t bytes, void* sums, unsigned grid, hipStream_t stream);
hipError_t stream_fill_launch(void* dst, uint64_t bytes, uint32_t pattern, unsigned grid, hipStream_t stream);
hipError_t stream_widen_launch(const void* src, void* dst, uint64_t in_bytes, unsigned grid, hipStream_t stream);
hipError_t widen_tiles_launch(const void* src, void* dst, const int64_t* in_stride_b, const int64_t* out_stride_b,
                              const uint32_t* tgrid, const uint32_t* box, const uint32_t* sbox, uint32_t n_tiles,
                              hipStream_t stream);
// Reference copies of other shapes: the kernel for (threads, unroll, cache
// policies), or nullptr when that combination is not built.
const void* copy_shape_kernel_for(int threads, int unroll, int load_nt, int store_nt);
hipError_t copy_shape_launch(const void* kernel, const void* src, void* dst, uint64_t bytes, unsigned grid,
                             unsigned threads, hipStream_t stream);
// Same-walk tiled copy reference (rank 3, packed output); threads 128 or
// 256 with at most 8 chunks of 16 bytes per lane and group, else
// hipErrorInvalidValue before any launch.
hipError_t copy_tiles_launch(const void* src, void* dst, const int64_t* in_stride_b, const int64_t* out_stride_b,
                             uint32_t rows_total, uint32_t row_bytes_total, uint32_t rows, uint32_t group_bytes,
                             uint32_t tiles_1, uint32_t groups_2, uint32_t n_groups, unsigned threads, unsigned grid,
                             hipStream_t stream);
hipError_t ring_trace_launch(int n_iters, int stages, int loads, int stores, int32_t* out,
                             hipStream_t stream);

// Magic numbers for n / d with n < 2^31: q = (n * mag) >> (31 + sh).
inline void magic_for(uint32_t d, uint32_t* mag, uint32_t* sh) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const unsigned __int128 num = (static_cast<unsigned __int128>(1) << (31 + s)) + d - 1;
  *mag = static_cast<uint32_t>(num / d);
  *sh = s;
}

}  // namespace acp
