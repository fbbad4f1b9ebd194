// Measurement references: plain register-path copies (no LDS, no ring) in
// other shapes and cache policies than stream_copy_kernel, so that a sweep
// can show what a plain copy of the same bytes reaches on this device.
#include "acp_dev_base.hpp"

namespace acp {
namespace dev {

// Workgroup w copies blocks w, w+G, ... of T * U * 16 bytes: each lane
// issues U 16-byte loads, then the U stores.  LNT / SNT select the
// non-temporal cache policy for the loads / the stores.  A block's buffer
// resources end at the copy's end, so a short last block reads zeros past it
// and its stores there are dropped.
template <int T, int U, int LNT, int SNT>
__global__ __launch_bounds__(T) void copy_shape_kernel(const char* src, char* dst, uint64_t bytes) {
  constexpr uint64_t kBlock = static_cast<uint64_t>(T) * U * 16u;
  const uint64_t blocks = (bytes + kBlock - 1) / kBlock;
  for (uint64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const uint64_t off = b * kBlock;
    const uint64_t left = bytes - off;
    const int range = static_cast<int>(left < kBlock ? left : kBlock);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + off, 0, range, 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(dst + off, 0, range, 0x00020000);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (u * T + threadIdx.x) * 16, 0, LNT ? 2 : 0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], ry, (u * T + threadIdx.x) * 16, 0, SNT ? 2 : 0);
  }
}

// Same-walk reference of a tiled copy: the tiles of a rank-3 tensor (dim 0
// one slab per tile, `rows` rows along dim 1, the innermost dim contiguous)
// go to a packed output of the same shape in groups of neighbouring tiles
// along the innermost dim, with no LDS and no ring.  Group g is tile row
// g / groups_per_row and group g % groups_per_row of it; workgroup w takes
// groups w, w+G, ... with the next group's loads issued before the current
// group's stores, so two groups are in flight as in a 2-slot ring.  Lane
// chunk c = u * T + lane of a group is row c / chunks_per_row and 16-byte
// column c % chunks_per_row; chunks past the tensor's edge take the
// out-of-bounds offset (loads read zeros, stores are dropped).
struct CopyTilesArgs {
  const char* src;
  char* dst;
  int64_t in_stride[2], out_stride[2];  // bytes per index of dims 0 and 1
  uint32_t rows_total;                  // extent of dim 1
  uint32_t row_bytes_total;             // innermost extent in bytes
  uint32_t rows;                        // tile rows
  uint32_t group_bytes;                 // bytes of one group row (a multiple of 16)
  uint32_t tiles_1, groups_2;           // tiles along dim 1, groups along the innermost dim
  uint32_t n_groups;
  uint32_t per;                         // groups per workgroup of a blocked walk (0: cyclic walk)
};

template <int T, int R>
struct TileGroup {
  __amdgpu_buffer_rsrc_t rin, rout;
  uint32_t xo[R], oo[R];

  __device__ __forceinline__ void locate(const CopyTilesArgs& A, uint32_t g) {
    const uint32_t c2 = g % A.groups_2;
    const uint32_t q = g / A.groups_2;
    const uint32_t t1 = q % A.tiles_1;
    const uint32_t t0 = q / A.tiles_1;
    const uint32_t row0 = t1 * A.rows;
    const uint32_t nrows = A.rows_total - row0 < A.rows ? A.rows_total - row0 : A.rows;
    const uint32_t col0 = c2 * A.group_bytes;
    const uint32_t ncol = A.row_bytes_total - col0 < A.group_bytes ? A.row_bytes_total - col0 : A.group_bytes;
    const int64_t ib = t0 * A.in_stride[0] + row0 * A.in_stride[1] + col0;
    const int64_t ob = t0 * A.out_stride[0] + row0 * A.out_stride[1] + col0;
    const uint32_t cpr = A.group_bytes / 16u;
    rin = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(A.src) + ib, 0, 0x7FFFFFFF, 0x00020000);
    rout = __builtin_amdgcn_make_buffer_rsrc(A.dst + ob, 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const uint32_t c = u * T + threadIdx.x;
      const uint32_t r = c / cpr, k = (c % cpr) * 16u;
      const bool ok = r < nrows && k < ncol;
      xo[u] = ok ? static_cast<uint32_t>(r * A.in_stride[1]) + k : kOobOffset;
      oo[u] = ok ? static_cast<uint32_t>(r * A.out_stride[1]) + k : kOobOffset;
    }
  }
  __device__ __forceinline__ void load(u32x4 (&v)[R]) const {
#pragma unroll
    for (int u = 0; u < R; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rin, xo[u], 0, 2);
  }
  __device__ __forceinline__ void store(const u32x4 (&v)[R]) const {
#pragma unroll
    for (int u = 0; u < R; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rout, oo[u], 0, 2);
  }
};

// Workgroup w takes groups w, w+G, ... (cyclic walk) or the run w * per,
// ..., (w + 1) * per - 1 (blocked walk).
template <int T, int R>
__global__ __launch_bounds__(T) void copy_tiles_kernel(const CopyTilesArgs A) {
  const uint32_t grid = gridDim.x;
  const uint32_t step = A.per ? 1u : grid;
  uint32_t g = A.per ? blockIdx.x * A.per : blockIdx.x;
  const uint32_t end = A.per ? min(A.n_groups, g + A.per) : A.n_groups;
  if (g >= end) return;
  TileGroup<T, R> a, b;
  u32x4 va[R], vb[R];
  a.locate(A, g);
  a.load(va);
  for (;;) {
    const uint32_t g1 = g + step;
    const bool more1 = g1 < end;
    if (more1) {
      b.locate(A, g1);
      b.load(vb);
    }
    a.store(va);
    if (!more1) break;
    const uint32_t g2 = g1 + step;
    const bool more2 = g2 < end;
    if (more2) {
      a.locate(A, g2);
      a.load(va);
    }
    b.store(vb);
    if (!more2) break;
    g = g2;
  }
}

}  // namespace dev

namespace {

struct CopyShape {
  int threads, unroll, load_nt, store_nt;
  const void* kernel;
};

#define ACP_COPY_SHAPE(T, U)                                                             \
  CopyShape{T, U, 1, 1, reinterpret_cast<const void*>(&dev::copy_shape_kernel<T, U, 1, 1>)}, \
  CopyShape{T, U, 1, 0, reinterpret_cast<const void*>(&dev::copy_shape_kernel<T, U, 1, 0>)}, \
  CopyShape{T, U, 0, 1, reinterpret_cast<const void*>(&dev::copy_shape_kernel<T, U, 0, 1>)}, \
  CopyShape{T, U, 0, 0, reinterpret_cast<const void*>(&dev::copy_shape_kernel<T, U, 0, 0>)}

const CopyShape kCopyShapes[] = {
    ACP_COPY_SHAPE(64, 16),  ACP_COPY_SHAPE(128, 8),  ACP_COPY_SHAPE(256, 2),  ACP_COPY_SHAPE(256, 4),
    ACP_COPY_SHAPE(256, 8),  ACP_COPY_SHAPE(512, 2),  ACP_COPY_SHAPE(512, 4),  ACP_COPY_SHAPE(512, 8),
    ACP_COPY_SHAPE(1024, 2), ACP_COPY_SHAPE(1024, 4),
};

#undef ACP_COPY_SHAPE

}  // namespace

const void* copy_shape_kernel_for(int threads, int unroll, int load_nt, int store_nt) {
  for (const CopyShape& c : kCopyShapes)
    if (c.threads == threads && c.unroll == unroll && c.load_nt == load_nt && c.store_nt == store_nt) return c.kernel;
  return nullptr;
}

hipError_t copy_tiles_launch(const void* src, void* dst, const int64_t* in_stride_b, const int64_t* out_stride_b,
                             uint32_t rows_total, uint32_t row_bytes_total, uint32_t rows, uint32_t group_bytes,
                             uint32_t tiles_1, uint32_t groups_2, uint32_t n_groups, unsigned threads, unsigned grid,
                             hipStream_t stream) {
  dev::CopyTilesArgs A{};
  A.src = static_cast<const char*>(src);
  A.dst = static_cast<char*>(dst);
  for (int d = 0; d < 2; ++d) {
    A.in_stride[d] = in_stride_b[d];
    A.out_stride[d] = out_stride_b[d];
  }
  A.rows_total = rows_total;
  A.row_bytes_total = row_bytes_total;
  A.rows = rows;
  A.group_bytes = group_bytes;
  A.tiles_1 = tiles_1;
  A.groups_2 = groups_2;
  A.n_groups = n_groups;
  // the library's walk for persistent tile copies: blocked runs when a
  // group row is whole 128-byte lines, else every G-th group
  A.per = (group_bytes % 128u == 0 && n_groups > grid) ? (n_groups + grid - 1) / grid : 0u;
  const uint32_t chunks = rows * (group_bytes / 16u);
  const void* k = nullptr;
  if (threads == 128 && chunks <= 512) k = reinterpret_cast<const void*>(&dev::copy_tiles_kernel<128, 4>);
  else if (threads == 128 && chunks <= 1024) k = reinterpret_cast<const void*>(&dev::copy_tiles_kernel<128, 8>);
  else if (threads == 256 && chunks <= 1024) k = reinterpret_cast<const void*>(&dev::copy_tiles_kernel<256, 4>);
  else if (threads == 256 && chunks <= 2048) k = reinterpret_cast<const void*>(&dev::copy_tiles_kernel<256, 8>);
  if (!k) return hipErrorInvalidValue;
  void* params[] = {&A};
  return hipLaunchKernel(k, dim3(grid), dim3(threads), params, 0, stream);
}

hipError_t copy_shape_launch(const void* kernel, const void* src, void* dst, uint64_t bytes, unsigned grid,
                             unsigned threads, hipStream_t stream) {
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  void* params[] = {&s, &d, &bytes};
  return hipLaunchKernel(kernel, dim3(grid), dim3(threads), params, 0, stream);
}

}  // namespace acp
