// Linear-grid kernels: streams, tile ewise and wave-local row sums whose
// stages sit on a row-major contiguous grid.
#pragma once

#include "acp_dev_map.hpp"

namespace acp {
namespace dev {

// ---------------------------------------------------------------------------
// Linear stage grid (one full stage per tile, row-major contiguous), 16-byte
// rounds, OUTER rounds per thread known at compile time.  Same ring schedule
// and wait counts as the general engine, the per-trip counts fixed at compile
// time; per trip only the stage bases change (by one grid stride), and no
// chunk can be out of bounds.
// * Streaming (STAGE_OUT false): one staged operand (x and z for two-tensor ops).
// * Tile ewise (STAGE_OUT true, "elementwise -> smem"): OP::NIN staged
//   operands, and the result goes through the LDS output image before the
//   store.  A stage is 2^k consecutive tiles (one ring trip), round f
//   belonging to tile f >> tile_rounds_log2 of it.

template <class OP, int OUTER, bool SROW, bool STAGE_OUT, bool NT>
struct LinPolicy {
  // staged operands per trip (a stream stages x, and z for two-tensor ops)
  static constexpr int NL = STAGE_OUT ? OP::NIN : (OP::NIN > 1 ? OP::NIN : 1);
  unsigned char* lds;
  const char* in[3];
  char* out;
  uint64_t in_span, out_span;
  uint64_t lin_x, lin_o, lin_r, total_rows;
  uint32_t lds0, slot_bytes, in_image_bytes, out_image_off, ab_base, wg, grid, waves_kb;  // waves_kb: LDS bytes of one round
  int wave, lane, ab_instr, swizzle, esize_log2;
  bool load_nt, store_nt;     // NT: both known to be set
  uint64_t ld_xb, ld_rb, step_x, step_r;  // byte and row offsets of the next stage loaded
  uint32_t xoff[OUTER], ooff[OUTER], abo[OUTER], lpos[OUTER];
  const uint64_t* row_ptr;   // [0] lane's array, [1 + q] row byte offset in the stage
  const uint32_t* row_ok;    // lane has a row in load q
  // SROW: this wave's row (relative to the stage) of each round, and the
  // scalars of the trip being consumed, read through the scalar cache
  const float __attribute__((address_space(4)))* ca;
  const float __attribute__((address_space(4)))* cb;
  uint32_t row_of[OUTER];
  float sa[OUTER], sb[OUTER];

  __device__ __forceinline__ uint64_t stage(int j) const { return wg + static_cast<uint64_t>(j) * grid; }
  __device__ __forceinline__ bool lnt() const { return NT || load_nt; }
  __device__ __forceinline__ bool snt() const { return NT || store_nt; }

  // the ring loads trips 0, 1, 2, ... in order: the stage offsets advance by
  // one grid stride per load
  __device__ __forceinline__ void load(int, int slot) {
    const uint64_t xb = ld_xb;
    ld_xb += step_x;
    const uint32_t range = range_from(in_span, xb);
    const uint32_t base = lds0 + slot * slot_bytes + wave * 1024u;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const v4i rs = rsrc_v4(in[k] + xb, range);
#pragma unroll
      for (int f = 0; f < OUTER; ++f) dma_b128(rs, xoff[f], base + k * in_image_bytes + f * waves_kb, lnt());
    }
    if constexpr (OP::ROW && !SROW) {
      const uint64_t rb = ld_rb;
      ld_rb += step_r;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= ab_instr) continue;
        uint64_t row = row_ok[q] ? rb + row_ptr[1 + q] / 4u : 0u;
        if (row >= total_rows) row = 0;
        const uint64_t addr = row_ptr[0] + row * 4u;
        dma_global_b32(reinterpret_cast<const void*>(addr), lds0 + slot * slot_bytes + ab_base + q * 256u);
      }
    }
  }
  __device__ __forceinline__ void pre_wait(int i, int, int) {
    if constexpr (OP::ROW && SROW) {
      // scalar loads of trip i's rows go out before the stage wait, so their
      // latency hides behind it
      const uint64_t rb = stage(i) * lin_r;
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        sa[f] = ca[rb + row_of[f]];
        sb[f] = cb[rb + row_of[f]];
      }
    }
  }

  __device__ __forceinline__ void consume(int i, int slot) {
    typedef ChunkShape<OP, 16> CS;
    typedef typename OP::TI TI;
    typedef typename OP::TO TO;
    const uint64_t s = stage(i);
    const uint64_t ob = s * lin_o;
    const __amdgpu_buffer_rsrc_t rs = rsrc_store(out + ob, range_from(out_span, ob));
    const uint32_t sl = slot * slot_bytes;
    // rounds in groups whose staged operands fit in registers together
    constexpr int GRP = round_group(OUTER, NL, 16);
    static_assert(OUTER % GRP == 0, "round groups must tile the rounds");
#pragma unroll
    for (int g0 = 0; g0 < OUTER; g0 += GRP) {
      u32x4 v[NL > 0 ? NL : 1][GRP];
      float ra[GRP], rb[GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int f = g0 + u;
#pragma unroll
        for (int k = 0; k < NL; ++k)
          v[k][u] = *reinterpret_cast<const u32x4*>(
              __builtin_assume_aligned(lds + sl + k * in_image_bytes + f * waves_kb + wave * 1024u + lane * 16u, 16));
        if constexpr (NL == 0) v[0][u] = u32x4{0, 0, 0, 0};
        if constexpr (OP::ROW && SROW) {
          ra[u] = sa[f];
          rb[u] = sb[f];
        } else if constexpr (OP::ROW) {
          ra[u] = *reinterpret_cast<const float*>(lds + sl + ab_base + abo[f]);
          rb[u] = *reinterpret_cast<const float*>(lds + sl + ab_base + abo[f] + 128u);
        } else {
          ra[u] = rb[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int f = g0 + u;
        TI in0[CS::NE], in1[CS::NE], in2[CS::NE];
        __builtin_memcpy(in0, &v[0][u], 16);
        __builtin_memcpy(in1, &v[NL > 1 ? 1 : 0][u], 16);
        __builtin_memcpy(in2, &v[NL > 2 ? 2 : 0][u], 16);
        TO res[CS::NE];
#pragma unroll
        for (int e = 0; e < CS::NE; ++e) res[e] = OP::f(in0[e], in1[e], in2[e], ra[u], rb[u]);
        uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        __builtin_memcpy(words, res, CS::OB);
        if constexpr (STAGE_OUT) {
          // the output tile is LDS-resident ("elementwise -> smem") and is
          // copied out from there; the lane reads back the bytes it wrote
          const uint32_t lo = (lpos[f] >> esize_log2) * CS::EO;
          constexpr int P = (CS::OB + 15) / 16;
          constexpr int PB = CS::OB < 16 ? CS::OB : 16;
#pragma unroll
          for (int piece = 0; piece < P; ++piece)
            __builtin_memcpy(lds + out_image_off + swz(lo + piece * 16, swizzle), words + piece * 4, PB);
          asm volatile("" ::: "memory");
#pragma unroll
          for (int piece = 0; piece < P; ++piece)
            __builtin_memcpy(words + piece * 4, lds + out_image_off + swz(lo + piece * 16, swizzle), PB);
        }
        store_chunk<CS::OB>(rs, ooff[f], words, snt());
      }
    }
  }
};

template <class OP, int OUTER, bool SROW, bool STAGE_OUT, bool NT>
__device__ __forceinline__ void stream_lin_body(CArgs* A, unsigned char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t n_tiles = A->n_tiles;
  const int n = static_cast<int>(wg < n_tiles ? (n_tiles - wg + grid - 1) / grid : 0);
  if (n == 0) return;
  LaneMap m;
  build_map_c<16, OUTER>(A, wave, lane, m);
  uint64_t row_ptr[3] = {0, 0, 0};
  uint32_t row_bad[2] = {~0u, ~0u};
  if constexpr (OP::ROW && !SROW) build_rows(A, lane, row_ptr, row_bad);
  uint32_t row_ok[2] = {row_bad[0] == 0u, row_bad[1] == 0u};
  const Loc L = load_loc(A);
  LinPolicy<OP, OUTER, SROW, STAGE_OUT, NT> p;
  p.lds = lds;
  for (int k = 0; k < 3; ++k) p.in[k] = L.in[k];
  p.out = L.out;
  p.in_span = L.in_span;
  p.out_span = L.out_span;
  p.lin_x = static_cast<uint64_t>(L.lin_x);
  p.lin_o = static_cast<uint64_t>(L.lin_o);
  p.lin_r = static_cast<uint64_t>(L.lin_r);
  p.total_rows = L.total_rows;
  p.lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  p.slot_bytes = L.slot_bytes;
  p.in_image_bytes = L.in_image_bytes;
  p.out_image_off = L.out_image_off;
  p.ab_base = L.ab_off + wave * L.ab_wave_bytes;
  p.wg = wg;
  p.grid = grid;
  p.wave = wave;
  p.lane = lane;
  p.ab_instr = L.ab_instr;
  p.swizzle = uni(A->swizzle);
  p.esize_log2 = uni(A->esize_log2);
  p.load_nt = L.load_nt != 0;
  p.store_nt = L.store_nt != 0;
  p.ld_xb = static_cast<uint64_t>(wg) * p.lin_x;
  p.ld_rb = static_cast<uint64_t>(wg) * p.lin_r;
  p.step_x = static_cast<uint64_t>(grid) * p.lin_x;
  p.step_r = static_cast<uint64_t>(grid) * p.lin_r;
  p.waves_kb = static_cast<uint32_t>(L.waves) * 1024u;
  // tile ewise: round f lies in tile f >> tile_rounds_log2 of the stage
  const uint32_t trl = STAGE_OUT ? uni(A->tile_rounds_log2) : 0u;
  const uint64_t tx = STAGE_OUT ? uni64(static_cast<uint64_t>(A->tile_x)) : 0u;
  const uint64_t to = STAGE_OUT ? uni64(static_cast<uint64_t>(A->tile_o)) : 0u;
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    const uint32_t t = static_cast<uint32_t>(f) >> trl;
    p.xoff[f] = m.xoff[f] + static_cast<uint32_t>(t * tx);
    p.ooff[f] = m.ooff[f] + static_cast<uint32_t>(t * to);
    p.abo[f] = m.abo[f];
    p.lpos[f] = m.lpos[f];
  }
  p.row_ptr = row_ptr;
  p.row_ok = row_ok;
  p.ca = (const float __attribute__((address_space(4)))*)(unip(A->row_a));
  p.cb = (const float __attribute__((address_space(4)))*)(unip(A->row_b));
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    // the whole 1 KiB block of this wave and round lies in one row
    const uint32_t abo = uni(m.abo[f]);
    p.row_of[f] = (abo >> 8) * 32u + (abo & 255u) / 4u;
    p.sa[f] = p.sb[f] = 0.f;
  }
  typedef ChunkShape<OP, 16> CS;
  constexpr int DL = LinPolicy<OP, OUTER, SROW, STAGE_OUT, NT>::NL * OUTER;
  if constexpr (OP::ROW && !SROW)
    run_ring(p, n, uni(A->stages), DL + L.ab_instr, OUTER * CS::ST);
  else
    run_ring_fixed<DL, OUTER * CS::ST>(p, n, uni(A->stages));
}

// Non-temporal loads and stores (the default for contiguous stages) get a
// body with the cache policy fixed at compile time, so the trip carries no
// branch on it.
template <class OP, int OUTER, bool SROW, bool STAGE_OUT = false>
__global__ __launch_bounds__(1024) void stream_lin_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  prefetch_kargs<kLinArgLines>();
  CArgs* A = kargs();
  if (A->load_nt && A->store_nt)
    stream_lin_body<OP, OUTER, SROW, STAGE_OUT, true>(A, lds);
  else
    stream_lin_body<OP, OUTER, SROW, STAGE_OUT, false>(A, lds);
}

// ---------------------------------------------------------------------------
// Row reduction on a linear stage grid whose wave blocks each lie in one row
// and whose rows each lie in one wave (the wave-local case): the linear
// kernel's lean trip (stage base advanced by one grid stride) with the wave-local
// reduction of the general kernel.  Stage s holds rows s * lin_r + (the
// packed offsets of its rows); lane k of a wave owns the wave's k-th
// distinct row.

template <class OP, int OUTER, bool NT>
struct LinRowsPolicy {
  unsigned char* lds;
  const char* in0;
  __amdgpu_buffer_rsrc_t out_rs;  // the whole row array
  uint64_t in_span, lin_x, lin_r;
  uint32_t lds0, slot_bytes, wg, grid, waves_kb;
  int wave, lane;
  bool load_nt, one_row;  // NT: load_nt known to be set
  uint64_t ld_xb, step_x;  // byte offset of the next stage loaded
  uint32_t xoff[OUTER], row_of[OUTER];
  uint32_t lrow, loff;  // this lane's row of the stage (~0: none) and its packed offset

  __device__ __forceinline__ uint64_t stage(int j) const { return wg + static_cast<uint64_t>(j) * grid; }

  // trips load in order: the stage offset advances by one grid stride
  __device__ __forceinline__ void load(int, int slot) {
    const uint64_t xb = ld_xb;
    ld_xb += step_x;
    const v4i rs = rsrc_v4(in0 + xb, range_from(in_span, xb));
    const uint32_t base = lds0 + slot * slot_bytes + wave * 1024u;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) dma_b128(rs, xoff[f], base + f * waves_kb, NT || load_nt);
  }
  __device__ __forceinline__ void pre_wait(int, int, int) {}

  __device__ __forceinline__ void consume(int i, int slot) {
    const uint32_t sl = slot * slot_bytes;
    float part[OUTER];
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
      part[f] = OP::chunk(v);
    }
    float acc = 0.f;
    if (one_row) {
      float p = part[0];
#pragma unroll
      for (int f = 1; f < OUTER; ++f) p += part[f];
      acc = wave_sum(p);
    } else {
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const float s = wave_sum(part[f]);
        acc += (lrow == row_of[f]) ? s : 0.f;
      }
    }
    const uint64_t g = stage(i) * lin_r + loff;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), out_rs,
                                          lrow != ~0u ? static_cast<uint32_t>(g * 4u) : kOobOffset, 0, 0);
  }
};

template <class OP, int OUTER, bool NT>
__device__ __forceinline__ void rows_lin_body(CArgs* A, unsigned char* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t n_tiles = A->n_tiles;
  const int n = static_cast<int>(wg < n_tiles ? (n_tiles - wg + grid - 1) / grid : 0);
  if (n == 0) return;
  LaneMap m;
  build_map_c<16, OUTER>(A, wave, lane, m);
  const Loc L = load_loc(A);
  LinRowsPolicy<OP, OUTER, NT> p;
  p.lds = lds;
  p.in0 = L.in[0];
  p.out_rs = rsrc_store(L.out, range_from(L.out_span, 0));
  p.in_span = L.in_span;
  p.lin_x = static_cast<uint64_t>(L.lin_x);
  p.lin_r = static_cast<uint64_t>(L.lin_r);
  p.lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  p.slot_bytes = L.slot_bytes;
  p.wg = wg;
  p.grid = grid;
  p.waves_kb = static_cast<uint32_t>(L.waves) * 1024u;
  p.wave = wave;
  p.lane = lane;
  p.load_nt = L.load_nt != 0;
  p.ld_xb = static_cast<uint64_t>(wg) * p.lin_x;
  p.step_x = static_cast<uint64_t>(grid) * p.lin_x;
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    p.xoff[f] = m.xoff[f];
    const uint32_t abo = uni(m.abo[f]);
    p.row_of[f] = (abo >> 8) * 32u + (abo & 255u) / 4u;
  }
  p.one_row = true;
#pragma unroll
  for (int f = 1; f < OUTER; ++f) p.one_row = p.one_row && p.row_of[f] == p.row_of[0];
  // the wave's distinct rows in round order; lane k takes the k-th
  p.lrow = ~0u;
  uint32_t n_local = 0;
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    bool seen = false;
#pragma unroll
    for (int g = 0; g < f; ++g) seen = seen || (p.row_of[g] == p.row_of[f]);
    if (!seen) {
      if (static_cast<uint32_t>(lane) == n_local) p.lrow = p.row_of[f];
      ++n_local;
    }
  }
  uint32_t rr = p.lrow != ~0u ? p.lrow : 0u, off = 0;
  for (int dd = uni(A->rank) - 2; dd >= 0; --dd) {
    const uint32_t sb = A->sbox[dd];
    off += (rr % sb) * A->rowstr[dd];
    rr /= sb;
  }
  p.loff = off;
  run_ring_fixed<OUTER, 1>(p, n, uni(A->stages));
}

template <class OP, int OUTER>
__global__ __launch_bounds__(1024) void rows_lin_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  prefetch_kargs<kLinArgLines>();
  CArgs* A = kargs();
  if (A->load_nt)
    rows_lin_body<OP, OUTER, true>(A, lds);
  else
    rows_lin_body<OP, OUTER, false>(A, lds);
}

}  // namespace dev
}  // namespace acp
