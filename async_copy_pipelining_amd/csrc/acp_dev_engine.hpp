// The rolled fallback engine: any round count and 4-byte rounds.
#pragma once

#include "acp_dev_map.hpp"

namespace acp {
namespace dev {

// Loads of one trip into one slot: every staged operand (outer rounds of
// VB-byte direct-to-LDS loads) and, for row ops, the stage's per-row scalars.
template <int VB>
__device__ __forceinline__ void issue_loads(const Loc& L, const LaneMap& m, const Trip& t, uint32_t slot_lds, int wave,
                                            const uint64_t* row_ptr, const uint32_t* row_bad) {
  const bool nt = L.load_nt != 0;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (k >= L.n_in) continue;
    const v4i rs = rsrc_v4(L.in[k] + t.xbase, range_from(L.in_span, t.xbase));
    const uint32_t img = slot_lds + k * L.in_image_bytes;
#pragma unroll
    for (int f = 0; f < kMaxOuter; ++f) {
      if (f >= L.outer) continue;
      const bool ok = !t.beyond && (m.oobm[f] & t.last) == 0;
      const uint32_t voff = ok ? m.xoff[f] : kOobOffset;
      const uint32_t m0 = img + (f * L.waves + wave) * 64u * VB;
      if constexpr (VB == 16)
        dma_b128(rs, voff, m0, nt);
      else
        dma_b32(rs, voff, m0, nt);
    }
  }
  if (L.row_ops) {
    // rows that do not exist (or lie past the edge) read row 0 of the array
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q >= L.ab_instr) continue;
      const bool ok = !t.beyond && (row_bad[q] & t.last) == 0;
      uint64_t row = ok ? t.rbase + row_ptr[1 + q] / 4u : 0u;
      if (row >= L.total_rows) row = 0;
      const uint64_t addr = row_ptr[0] + row * 4u;
      dma_global_b32(reinterpret_cast<const void*>(addr), slot_lds + L.ab_off + wave * L.ab_wave_bytes + q * 256u);
    }
  }
}

// Consume one trip: read the staged chunks, apply the op, (tile ewise) write
// the result into the slot's output image and read it back, store.
template <class OP, int VB, bool STAGE_OUT>
__device__ __forceinline__ void consume_trip(const Loc& L, int esize_log2, int swizzle, const LaneMap& m,
                                             const Trip& t, unsigned char* lds, uint32_t slot, int wave, int lane) {
  typedef ChunkShape<OP, VB> CS;
  typedef typename OP::TI TI;
  typedef typename OP::TO TO;
  const int outer = L.outer, waves = L.waves;
  const uint32_t in_img = L.in_image_bytes;
  const __amdgpu_buffer_rsrc_t rs = rsrc_store(L.out + t.obase, range_from(L.out_span, t.obase));
#pragma unroll
  for (int f = 0; f < kMaxOuter; ++f) {
    if (f >= outer) continue;
    const uint32_t chunk = slot + ((f * waves + wave) * 64u + lane) * VB;
    TI in[3][CS::NE];
#pragma unroll
    for (int k = 0; k < (OP::NIN ? OP::NIN : 1); ++k) {
      if (k >= OP::NIN) {
        __builtin_memset(in[k], 0, sizeof(in[k]));
      } else if constexpr (VB == 16) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(__builtin_assume_aligned(lds + chunk + k * in_img, 16));
        __builtin_memcpy(in[k], &v, 16);
      } else {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(__builtin_assume_aligned(lds + chunk + k * in_img, 4));
        __builtin_memcpy(in[k], &v, 4);
      }
    }
    float ra = 0.f, rb = 0.f;
    if constexpr (OP::ROW) {
      const uint32_t ab = slot + L.ab_off + wave * L.ab_wave_bytes + m.abo[f];
      ra = *reinterpret_cast<const float*>(lds + ab);
      rb = *reinterpret_cast<const float*>(lds + ab + 128u);
    }
    TO res[CS::NE];
#pragma unroll
    for (int e = 0; e < CS::NE; ++e)
      res[e] = OP::f(in[0][e], in[OP::NIN > 1 ? 1 : 0][e], in[OP::NIN > 2 ? 2 : 0][e], ra, rb);
    uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    __builtin_memcpy(words, res, CS::OB);
    if constexpr (STAGE_OUT) {
      // the output tile lives in LDS ("elementwise -> smem": every operand,
      // the output included, is in shared memory) and is copied out from there
      const uint32_t lo = (m.lpos[f] >> esize_log2) * CS::EO;
      constexpr int P = (CS::OB + 15) / 16;
      constexpr int PB = CS::OB < 16 ? CS::OB : 16;
#pragma unroll
      for (int piece = 0; piece < P; ++piece) {
        const uint32_t lp = lo + piece * 16;
        __builtin_memcpy(lds + L.out_image_off + swz(lp, swizzle), words + piece * 4, PB);
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int piece = 0; piece < P; ++piece) {
        const uint32_t lp = lo + piece * 16;
        __builtin_memcpy(words + piece * 4, lds + L.out_image_off + swz(lp, swizzle), PB);
      }
    }
    const bool ok = !t.beyond && (m.oobm[f] & t.last) == 0;
    store_chunk<CS::OB>(rs, ok ? m.ooff[f] : kOobOffset, words, L.store_nt != 0);
  }
}

template <class OP, int VB, bool STAGE_OUT>
struct EnginePolicy {
  CArgs* A;
  const Loc& L;
  const LaneMap& m;
  unsigned char* lds;
  uint32_t lds0, wg, grid;
  int wave, lane, esize_log2, swizzle;
  uint64_t row_ptr[3];   // by value: a pointer to the caller's arrays would keep them in scratch memory
  uint32_t row_bad[2];

  __device__ __forceinline__ void load(int j, int slot) {
    const Trip t = trip_geometry(A, L, wg, grid, j);
    issue_loads<VB>(L, m, t, lds0 + slot * L.slot_bytes, wave, row_ptr, row_bad);
  }
  __device__ __forceinline__ void pre_wait(int, int, int) {}
  __device__ __forceinline__ void consume(int i, int slot) {
    const Trip t = trip_geometry(A, L, wg, grid, i);
    consume_trip<OP, VB, STAGE_OUT>(L, esize_log2, swizzle, m, t, lds, slot * L.slot_bytes, wave, lane);
  }
};

// The engine kernel.  The EngineArgs parameter fixes the launch ABI; the
// body reads it through the kernarg segment pointer.
template <class OP, int VB, bool STAGE_OUT>
__global__ __launch_bounds__(1024) void engine_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  prefetch_kargs();
  CArgs* A = kargs();
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t n_tiles = A->n_tiles;
  const uint32_t tiles = wg < n_tiles ? (n_tiles - wg + grid - 1) / grid : 0;
  const int n = static_cast<int>(tiles * A->subs);
  if (n == 0) return;
  const Loc L = load_loc(A);
  const int esize_log2 = A->esize_log2, swizzle = A->swizzle, stages = A->stages;
  LaneMap m;
  build_map<VB>(A, wave, lane, m);
  uint64_t row_ptr[3];
  uint32_t row_bad[2];
  build_rows(A, lane, row_ptr, row_bad);
  EnginePolicy<OP, VB, STAGE_OUT> pol{A, L, m, lds, lds0, wg, grid, wave, lane, esize_log2, swizzle,
                                      {row_ptr[0], row_ptr[1], row_ptr[2]}, {row_bad[0], row_bad[1]}};
  typedef ChunkShape<OP, VB> CS;
  const int d = L.n_in * L.outer + (L.row_ops ? L.ab_instr : 0);
  const int st = L.outer * CS::ST;
  run_ring(pol, n, stages, d, st);
}

}  // namespace dev
}  // namespace acp
