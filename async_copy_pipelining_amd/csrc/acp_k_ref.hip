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

hipError_t copy_shape_launch(const void* kernel, const void* src, void* dst, uint64_t bytes, unsigned grid,
                             unsigned threads, hipStream_t stream) {
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  void* params[] = {&s, &d, &bytes};
  return hipLaunchKernel(kernel, dim3(grid), dim3(threads), params, 0, stream);
}

}  // namespace acp
