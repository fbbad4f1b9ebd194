// Kernel registry, launch helpers and the two debug kernels of the engine.
#include "acp_engine_impl.hpp"

namespace acp {

const void* lookup_copy(const KernelKey& k);
const void* lookup_tile(const KernelKey& k);
const void* lookup_tile_gen(const KernelKey& k);
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
  __device__ void wait(int i, int s, int k) { put(1, i, s, k); }
  __device__ void consume(int i, int s) { put(2, i, s, 0); }
};

__global__ void ring_trace_kernel(int n, int s, int loads, int stores, int32_t* out) {
  if (threadIdx.x != 0) return;
  TracePolicy p{out, 0};
  run_ring(p, n, s, loads, stores);
}

}  // namespace dev

const void* engine_kernel(const KernelKey& k) {
  if (const void* f = lookup_copy(k)) return f;
  if (const void* f = lookup_tile(k)) return f;
  if (const void* f = lookup_tile_gen(k)) return f;
  if (const void* f = lookup_stream_f32(k)) return f;
  return lookup_stream_f16(k);
}

hipError_t engine_launch(const void* kernel, const EngineArgs& args, unsigned grid, unsigned block,
                         unsigned lds_bytes, hipStream_t stream) {
  hipError_t err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_bytes));
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
  hipError_t err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_bytes));
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
