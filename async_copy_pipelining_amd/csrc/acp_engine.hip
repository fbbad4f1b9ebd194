// Kernel registry, launch helpers, the two debug kernels of the engine and the
// register-path reference copy.
#include <mutex>
#include <unordered_map>

#include "acp_engine_impl.hpp"

namespace acp {

const void* lookup_copy(const KernelKey& k);
const void* lookup_tile(const KernelKey& k);
const void* lookup_tile_gen(const KernelKey& k);
const void* lookup_tile_lin(const KernelKey& k);
const void* lookup_stream_f32(const KernelKey& k);
const void* lookup_stream_f16(const KernelKey& k);

namespace dev {

// Debug: load one tile (A->tile0) into slot 0, wait, then dump the slot's
// first operand image.  The dump reads chunks that other waves loaded, so it
// is the one place that needs a workgroup barrier.
template <int VB>
__global__ __launch_bounds__(1024) void lds_image_kernel_t(const EngineArgs, unsigned char* out, uint32_t bytes) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  CArgs* A = kargs();
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const Loc L = load_loc(A);
  LaneMap m;
  build_map<VB>(A, wave, lane, m);
  uint64_t row_ptr[3] = {0, 0, 0};
  uint32_t row_bad[2] = {~0u, ~0u};
  const Trip t = trip_geometry(A, L, 0, 1, 0);
  issue_loads<VB>(L, m, t, lds0, wave, row_ptr, row_bad);
  wait_vmcnt(0);
  __syncthreads();
  for (uint32_t o = threadIdx.x * 4u; o < bytes; o += blockDim.x * 4u)
    *reinterpret_cast<uint32_t*>(out + o) = *reinterpret_cast<const uint32_t*>(lds + o);
}

// Debug: the ring control of the engine for one wave, recording its events.
struct TracePolicy {
  int32_t* out;
  int pos;
  __device__ void put(int kind, int i, int s, int k) {
    out[pos * 4 + 0] = kind;
    out[pos * 4 + 1] = i;
    out[pos * 4 + 2] = s;
    out[pos * 4 + 3] = k;
    ++pos;
  }
  __device__ void load(int j, int s) { put(0, j, s, 0); }
  __device__ void pre_wait(int i, int s, int k) { put(1, i, s, k); }
  __device__ void consume(int i, int s) { put(2, i, s, 0); }
};

// Per-trip counts that the linear-grid kernels fix at compile time run the
// ring with those counts; any other pair runs the general ring.
__global__ void ring_trace_kernel(int n, int s, int loads, int stores, int32_t* out) {
  if (threadIdx.x != 0) return;
  TracePolicy p{out, 0};
  if (loads == 1 && stores == 1) run_ring_fixed<1, 1>(p, n, s);
  else if (loads == 2 && stores == 1) run_ring_fixed<2, 1>(p, n, s);
  else if (loads == 2 && stores == 2) run_ring_fixed<2, 2>(p, n, s);
  else if (loads == 4 && stores == 1) run_ring_fixed<4, 1>(p, n, s);
  else if (loads == 4 && stores == 4) run_ring_fixed<4, 4>(p, n, s);
  else run_ring(p, n, s, loads, stores);
}

// Measurement reference: a plain register-path copy (no LDS, no ring).
// Workgroup w copies 16 KiB blocks w, w+G, ...: four 16-byte non-temporal
// loads per lane, then the four stores.  The block's buffer resources end at
// the copy's end, so a short last block reads zeros past it and its stores
// there are dropped.
__global__ __launch_bounds__(256) void stream_copy_kernel(const char* src, char* dst, uint64_t bytes) {
  const uint64_t blocks = (bytes + 16383u) / 16384u;
  for (uint64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const uint64_t off = b * 16384u;
    const uint64_t left = bytes - off;
    const int range = static_cast<int>(left < 16384u ? left : 16384u);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + off, 0, range, 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(dst + off, 0, range, 0x00020000);
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (u * 256 + threadIdx.x) * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], ry, (u * 256 + threadIdx.x) * 16, 0, 2);
  }
}

// Measurement references for one direction at a time, with the copy's walk
// (16 KiB blocks w, w+G, ..., four non-temporal 16-byte accesses per lane):
// a read-only stream whose lanes fold what they read into one 16-byte XOR per
// lane (the workgroup's XOR goes to sums[w], so no load can be dropped), and
// a write-only stream of one 32-bit pattern.
__global__ __launch_bounds__(256) void stream_read_kernel(const char* src, uint64_t bytes, u32x4* sums) {
  __shared__ u32x4 part[256];
  const uint64_t blocks = (bytes + 16383u) / 16384u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const uint64_t off = b * 16384u;
    const uint64_t left = bytes - off;
    const int range = static_cast<int>(left < 16384u ? left : 16384u);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + off, 0, range, 0x00020000);
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rx, (u * 256 + threadIdx.x) * 16, 0, 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (unsigned h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) part[threadIdx.x] ^= part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[blockIdx.x] = part[0];
}

__global__ __launch_bounds__(256) void stream_fill_kernel(char* dst, uint64_t bytes, uint32_t pattern) {
  const uint64_t blocks = (bytes + 16383u) / 16384u;
  const u32x4 v = {pattern, pattern, pattern, pattern};
  for (uint64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const uint64_t off = b * 16384u;
    const uint64_t left = bytes - off;
    const int range = static_cast<int>(left < 16384u ? left : 16384u);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(dst + off, 0, range, 0x00020000);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_amdgcn_raw_buffer_store_b128(v, ry, (u * 256 + threadIdx.x) * 16, 0, 2);
  }
}

// Measurement reference for a widening stream (two bytes written per byte
// read): float16 -> float32 conversion of a contiguous tensor, workgroup w
// taking 8 KiB input blocks w, w+G, ...: four 8-byte non-temporal loads per
// lane, each widened into one 16-byte store, so every wave instruction reads
// 512 contiguous bytes and writes 1 KiB.
__global__ __launch_bounds__(256) void stream_widen_kernel(const char* src, char* dst, uint64_t in_bytes) {
  const uint64_t blocks = (in_bytes + 8191u) / 8192u;
  for (uint64_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const uint64_t off = b * 8192u;
    const uint64_t left = in_bytes - off;
    const int range = static_cast<int>(left < 8192u ? left : 8192u);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + off, 0, range, 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(dst + 2 * off, 0, 2 * range, 0x00020000);
    u32x2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b64(rx, (u * 256 + threadIdx.x) * 8, 0, 2);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      _Float16 h[4];
      __builtin_memcpy(h, &v[u], 8);
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(h[e]);
      u32x4 w;
      __builtin_memcpy(&w, f, 16);
      __builtin_amdgcn_raw_buffer_store_b128(w, ry, (u * 256 + threadIdx.x) * 16, 0, 2);
    }
  }
}

// Measurement reference with the walk of a tiled widening stream: tiles of a
// rank-5 float16 tensor (any strides, innermost 1) go to float32 in a packed
// output with no LDS and no ring.  Workgroup b takes the tile whose index is
// b remapped so that consecutive tiles run on one XCD (as the library's
// streams do when the tile count is a multiple of 8), and walks the tile's
// stages in row-major order; a stage is stage_rows rows of stage_cols
// elements (the two innermost dims).  Each lane takes 4-element pieces (up
// to eight per stage): two stages per iteration, their 8-byte loads in
// flight together, each piece widened into one 16-byte non-temporal store.
// Geometry (validated on the host): stage_cols a multiple of 4, at most 2048
// pieces per stage, every tile and stage whole, 8-byte aligned input rows.
struct WidenTilesArgs {
  const char* src;
  char* dst;
  int64_t in_stride[5], out_stride[5];  // bytes
  uint32_t tgrid[5], box[5], sbox[5], sub[5];
  uint32_t n_tiles, subs, remap;
};

__global__ __launch_bounds__(256) void widen_tiles_kernel(const WidenTilesArgs A) {
  uint32_t b = blockIdx.x;
  const uint32_t grid = gridDim.x;
  if (A.remap) b = (b % 8u) * (grid / 8u) + b / 8u;
  if (b >= A.n_tiles) return;
  // tile coordinates, last dim fastest
  uint32_t tc[5], t = b;
  for (int d = 4; d >= 0; --d) {
    tc[d] = t % A.tgrid[d];
    t /= A.tgrid[d];
  }
  const uint32_t cols = A.sbox[4], rows = A.sbox[3];
  const uint32_t pieces_per_row = cols / 4u;
  const uint32_t pieces = rows * pieces_per_row;
  for (uint32_t j0 = 0; j0 < A.subs; j0 += 2) {
    u32x2 v[2][8];
    int64_t ob[2];
    uint32_t np = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t j = j0 + h;
      if (j >= A.subs) break;
      // stage coordinates inside the tile, last dim fastest
      uint32_t sj = j, sc[5];
      for (int d = 4; d >= 0; --d) {
        sc[d] = sj % A.sub[d];
        sj /= A.sub[d];
      }
      int64_t ib = 0, o = 0;
      for (int d = 0; d < 5; ++d) {
        const int64_t c = static_cast<int64_t>(tc[d]) * A.box[d] + static_cast<int64_t>(sc[d]) * A.sbox[d];
        ib += c * A.in_stride[d];
        o += c * A.out_stride[d];
      }
      ob[h] = o;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = u * 256u + threadIdx.x;
        const uint32_t r = p / pieces_per_row, q = p % pieces_per_row;
        if (p < pieces)
          v[h][u] = *reinterpret_cast<const u32x2*>(A.src + ib + r * A.in_stride[3] + q * 8u);
      }
      ++np;
    }
    for (uint32_t h = 0; h < np; ++h) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = u * 256u + threadIdx.x;
        if (p >= pieces) continue;
        const uint32_t r = p / pieces_per_row, q = p % pieces_per_row;
        _Float16 hh[4];
        __builtin_memcpy(hh, &v[h][u], 8);
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(hh[e]);
        u32x4 w;
        __builtin_memcpy(&w, f, 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(A.dst + ob[h] + r * A.out_stride[3] + q * 16u));
      }
    }
  }
}

}  // namespace dev

hipError_t widen_tiles_launch(const void* src, void* dst, const int64_t* in_stride_b, const int64_t* out_stride_b,
                              const uint32_t* tgrid, const uint32_t* box, const uint32_t* sbox, uint32_t n_tiles,
                              hipStream_t stream) {
  dev::WidenTilesArgs A{};
  A.src = static_cast<const char*>(src);
  A.dst = static_cast<char*>(dst);
  A.subs = 1;
  for (int d = 0; d < 5; ++d) {
    A.in_stride[d] = in_stride_b[d];
    A.out_stride[d] = out_stride_b[d];
    A.tgrid[d] = tgrid[d];
    A.box[d] = box[d];
    A.sbox[d] = sbox[d];
    A.sub[d] = box[d] / sbox[d];
    A.subs *= A.sub[d];
  }
  A.n_tiles = n_tiles;
  A.remap = (n_tiles % 8 == 0 && n_tiles >= 16) ? 1u : 0u;
  hipLaunchKernelGGL(dev::widen_tiles_kernel, dim3(n_tiles), dim3(256), 0, stream, A);
  return hipGetLastError();
}

hipError_t stream_widen_launch(const void* src, void* dst, uint64_t in_bytes, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL(dev::stream_widen_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const char*>(src),
                     static_cast<char*>(dst), in_bytes);
  return hipGetLastError();
}

hipError_t stream_read_launch(const void* src, uint64_t bytes, void* sums, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL(dev::stream_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const char*>(src), bytes,
                     static_cast<dev::u32x4*>(sums));
  return hipGetLastError();
}

hipError_t stream_fill_launch(void* dst, uint64_t bytes, uint32_t pattern, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL(dev::stream_fill_kernel, dim3(grid), dim3(256), 0, stream, static_cast<char*>(dst), bytes,
                     pattern);
  return hipGetLastError();
}

hipError_t stream_copy_launch(const void* src, void* dst, uint64_t bytes, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL(dev::stream_copy_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const char*>(src),
                     static_cast<char*>(dst), bytes);
  return hipGetLastError();
}

const void* engine_kernel(const KernelKey& k) {
  if (const void* f = lookup_copy(k)) return f;
  if (const void* f = lookup_tile(k)) return f;
  if (const void* f = lookup_tile_gen(k)) return f;
  if (const void* f = lookup_tile_lin(k)) return f;
  if (const void* f = lookup_stream_f32(k)) return f;
  return lookup_stream_f16(k);
}

// Raise a kernel's dynamic-LDS limit when a launch needs more than any
// earlier one on this device.  The attribute is process state shared by
// every calling thread, so it only ever grows: one process-wide record,
// changed under a lock, holds the limit set per (kernel, device), and a
// thread-local copy answers repeat launches without the lock (a limit once
// set is never lowered, so the copy stays valid).
hipError_t ensure_lds_limit(const void* kernel, unsigned lds_bytes) {
  thread_local std::unordered_map<uint64_t, unsigned> seen;  // (kernel, device) -> limit known to be set
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const uint64_t key = (static_cast<uint64_t>(reinterpret_cast<uintptr_t>(kernel)) << 8) ^ static_cast<uint64_t>(dev);
  const auto it = seen.find(key);
  if (it != seen.end() && it->second >= lds_bytes) return hipSuccess;
  static std::mutex lock;
  static std::unordered_map<uint64_t, unsigned> set;  // (kernel, device) -> limit set in this process
  std::lock_guard<std::mutex> guard(lock);
  unsigned& limit = set[key];
  if (limit < lds_bytes) {
    const hipError_t err =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_bytes));
    if (err != hipSuccess) return err;
    limit = lds_bytes;
  }
  seen[key] = limit;
  return hipSuccess;
}

hipError_t engine_launch(const void* kernel, const EngineArgs& args, unsigned grid, unsigned block,
                         unsigned lds_bytes, hipStream_t stream) {
  const hipError_t err = ensure_lds_limit(kernel, lds_bytes);
  if (err != hipSuccess) return err;
  void* params[] = {const_cast<EngineArgs*>(&args)};
  return hipLaunchKernel(kernel, dim3(grid), dim3(block), params, lds_bytes, stream);
}

const void* lds_image_kernel(int vec_bytes) {
  return vec_bytes == 16 ? reinterpret_cast<const void*>(&dev::lds_image_kernel_t<16>)
                         : reinterpret_cast<const void*>(&dev::lds_image_kernel_t<4>);
}

hipError_t lds_image_launch(const void* kernel, const EngineArgs& args, unsigned block, unsigned lds_bytes,
                            void* out_bytes, uint32_t image_bytes, hipStream_t stream) {
  const hipError_t err = ensure_lds_limit(kernel, lds_bytes);
  if (err != hipSuccess) return err;
  unsigned char* out = static_cast<unsigned char*>(out_bytes);
  void* params[] = {const_cast<EngineArgs*>(&args), &out, &image_bytes};
  return hipLaunchKernel(kernel, dim3(1), dim3(block), params, lds_bytes, stream);
}

hipError_t ring_trace_launch(int n, int s, int loads, int stores, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(dev::ring_trace_kernel, dim3(1), dim3(64), 0, stream, n, s, loads, stores, out);
  return hipGetLastError();
}

}  // namespace acp
