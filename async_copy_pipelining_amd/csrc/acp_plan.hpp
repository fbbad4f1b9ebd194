// Host-side descriptor store and plan search for acp (pure C++17, no HIP).
//
// Plan search ("copy_async -> tma", "Algorithm" step 2): canonicalize (L1),
// split the inner axis into 128-byte swizzle atoms and cut boxes over 256
// into several loads (L2), merge adjacent fully-boxed contiguous dims,
// promote the element type of an over-256 copy box, validate rank <= 5 and
// shrink the descriptor from the outside when it is too deep (L3).
// Partition ("elementwise -> smem" and "copy_async -> ldgsts", "Algorithm"
// step 1): [outer, threads, vec] with vec the widest legal aligned width.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace acp {

constexpr int kMaxInputRank = 8;
constexpr int kMaxRank = 5;
constexpr int64_t kMaxBox = 256;
constexpr int64_t kMaxIssues = 256;   // loads per tile the kernels index (a library limit)
constexpr int kMaxImageAxes = 12;     // axes of a tile's LDS image the kernels index (a library limit)
constexpr uint32_t kDescMagic = 0x44504341u;  // "ACPD"

enum class PlanStatus { Ok, Invalid, Declined, Unsupported };

// Contents of acp_tile_desc::opaque.
struct DescData {
  uint32_t magic;
  uint8_t dtype, esize, rank, swizzle;
  uint8_t oob, reserved[3];
  uint64_t gbase;
  int64_t shape[kMaxInputRank];
  int64_t strides[kMaxInputRank];  // elements
  int32_t box[kMaxInputRank];
};
static_assert(sizeof(DescData) <= 256, "descriptor payload must fit acp_tile_desc");

// One axis of a tile's LDS image: `count` indices along tensor dim `dim`,
// each advancing that coordinate by `step` elements.
struct Axis {
  int64_t count;
  int dim;
  int64_t step;
};

struct DescDim {
  int64_t extent;        // desc elements
  int64_t stride;        // bytes
  int64_t box;           // desc elements
  std::vector<Axis> parts;
  bool atom = false;
  bool segmented = false;
  Axis seg{0, 0, 0};
};

struct Plan {
  int esize = 0, desc_esize = 0, swizzle = 0;
  bool promoted = false;
  int rank_t = 0;                        // tensor rank as encoded
  int64_t shape[kMaxInputRank] = {};
  int64_t strides[kMaxInputRank] = {};   // elements
  int64_t box[kMaxInputRank] = {};
  std::vector<DescDim> dims;             // the descriptor, outermost-first
  std::vector<Axis> issue_axes;          // outermost-first
  int threads = 0, vec_bytes = 0, vec = 0, outer = 0;

  std::vector<Axis> image_axes() const;  // issue axes then box parts; count-1 axes dropped
  int64_t issues() const;
  int64_t tile_elems() const;
  int64_t tile_bytes() const { return tile_elems() * esize; }
  int64_t n_tiles() const;
};

PlanStatus plan_box(const DescData& d, bool copy_only, Plan* out, std::string* reason);
// Same as plan_box for a different box over the same tensor.
PlanStatus plan_box_with(const DescData& d, const int32_t* box, bool copy_only, Plan* out,
                         std::string* reason);
PlanStatus plan_partition(Plan* p, int threads, uint64_t base_addr, std::string* reason);

int dtype_size(int dtype);  // -1 if unknown

}  // namespace acp
