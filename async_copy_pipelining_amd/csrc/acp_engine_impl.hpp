// Stage-ring engine for gfx950 (CDNA4): direct-to-LDS tile loads, a per-wave
// completion count in place of per-stage barriers, elementwise ops on the
// staged tile, and coalesced buffer stores.  Included by the kernel
// translation units only.
//
// Design (what the pages describe, re-built for gfx950):
// * "copy_async -> tma" moves a whole tile with one descriptor-driven
//   instruction that completes on a barrier; "copy_async -> ldgsts" has every
//   thread issue 16-byte asynchronous copies to its own shared address.
//   gfx950 has neither a tensor engine nor per-thread LDS destinations for
//   asynchronous loads: its direct-to-LDS buffer loads write lane l's 16 (or
//   4) bytes at M0 + 16 * l (4 * l), so one wave instruction fills one
//   contiguous 1 KiB (256 B) of LDS.  A tile's LDS image is therefore filled
//   in contiguous blocks and the swizzle is applied on the GLOBAL side: lane
//   l fetches the logical chunk the swizzle maps onto its physical slot (the
//   swizzle is an involution).
// * The [outer, threads, vec] partition of "elementwise -> smem" is also the
//   load partition: round f of thread t loads, and later consumes, the same
//   physical chunk (f * threads + t).  Every wave thus consumes only bytes it
//   loaded itself, completion is the wave's own in-order count of
//   outstanding memory operations (s_waitcnt vmcnt) and the ring needs no
//   workgroup barrier.  Reusing a slot (the hazard the circular-buffer
//   pseudo-code leaves implicit) is safe because the wave's LDS reads of the
//   previous occupant completed before that data was stored.
// * Out-of-bounds chunks get a buffer offset past the resource's range: the
//   hardware writes zeros into LDS (the descriptor's zero fill) and drops
//   such stores, so every wave issues the same number of memory operations
//   and the wait counts stay exact.
// * Direct-to-LDS loads and the waits are inline asm: the compiler treats any
//   pending direct-to-LDS load as aliasing every LDS read and would put a
//   full vmcnt(0) wait before each one, collapsing the ring.
// * Launch arguments are read through the kernarg segment pointer (address
//   space 4): scalar loads, no per-lane copy of the argument block.
#pragma once

#include <hip/hip_runtime.h>

#include "acp_engine.hpp"

namespace acp {
namespace dev {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const EngineArgs __attribute__((address_space(4))) CArgs;

constexpr int kOpZero = 0, kOpSqrt = 1, kOpExp = 2, kOpAdd = 3, kOpMul = 4, kOpFma = 5, kOpCopy = 6;
constexpr int kU32 = 2, kF16 = 4, kF32 = 5;

__device__ __forceinline__ CArgs* kargs() {
  return (CArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
}

// XOR swizzle of a stage-relative LDS byte offset: the 16-byte chunk index
// within its span takes the 128-byte row index modulo the span's chunk
// count (mask 1, 3, 7 for the 32-, 64-, 128-byte modes; 0 is no swizzle).
__device__ __forceinline__ uint32_t swz(uint32_t o, uint32_t mask) { return o ^ (((o >> 7) & mask) << 4); }

__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint32_t mag, uint32_t sh) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * mag) >> (31 + sh));
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}

// Range of a buffer resource starting `off` bytes into a tensor of `span`
// bytes: it ends at the tensor's end (and below the out-of-bounds offset).
// Both values lie below 2^63, so span - off read as a signed number tells
// whether off is past the span; the clamp works on 32-bit halves, which
// keeps the whole computation in scalar instructions.
__device__ __forceinline__ uint32_t range_from(uint64_t span, uint64_t off) {
  const uint64_t d = span - off;
  const uint32_t hi = static_cast<uint32_t>(d >> 32), lo = static_cast<uint32_t>(d);
  if (static_cast<int32_t>(hi) < 0) return 0u;
  if (hi != 0u || lo >= kOobOffset) return kOobOffset - 16u;
  return lo;
}

// Buffer resource for the asm loads: raw (stride 0), 32-bit data format.
__device__ __forceinline__ v4i rsrc_v4(const void* base, uint32_t range) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r.x = uni(static_cast<int>(static_cast<uint32_t>(a)));
  r.y = uni(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu));
  r.z = uni(static_cast<int>(range));
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_store(void* base, uint32_t range) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(range), 0x00020000);
}

// s_nop 4 covers the wait states between an SGPR / M0 write and a
// direct-to-LDS instruction reading it.
__device__ __forceinline__ void dma_b128(v4i rsrc, uint32_t voff, uint32_t m0, bool nt) {
  if (nt)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
__device__ __forceinline__ void dma_b32(v4i rsrc, uint32_t voff, uint32_t m0, bool nt) {
  if (nt)
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
__device__ __forceinline__ void dma_global_b32(const void* addr, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "{m0}"(m0) : "memory");
}

// Wait until at most k of this wave's memory operations are outstanding.
// Completion is in issue order, so this retires everything issued before the
// k most recent operations.  k above the 6-bit field clamps to 63 (a
// stronger wait).
__device__ __forceinline__ void wait_vmcnt(int k) {
  switch (k < 63 ? k : 63) {
#define ACP_W(n) \
  case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;
    ACP_W(0) ACP_W(1) ACP_W(2) ACP_W(3) ACP_W(4) ACP_W(5) ACP_W(6) ACP_W(7)
    ACP_W(8) ACP_W(9) ACP_W(10) ACP_W(11) ACP_W(12) ACP_W(13) ACP_W(14) ACP_W(15)
    ACP_W(16) ACP_W(17) ACP_W(18) ACP_W(19) ACP_W(20) ACP_W(21) ACP_W(22) ACP_W(23)
    ACP_W(24) ACP_W(25) ACP_W(26) ACP_W(27) ACP_W(28) ACP_W(29) ACP_W(30) ACP_W(31)
    ACP_W(32) ACP_W(33) ACP_W(34) ACP_W(35) ACP_W(36) ACP_W(37) ACP_W(38) ACP_W(39)
    ACP_W(40) ACP_W(41) ACP_W(42) ACP_W(43) ACP_W(44) ACP_W(45) ACP_W(46) ACP_W(47)
    ACP_W(48) ACP_W(49) ACP_W(50) ACP_W(51) ACP_W(52) ACP_W(53) ACP_W(54) ACP_W(55)
    ACP_W(56) ACP_W(57) ACP_W(58) ACP_W(59) ACP_W(60) ACP_W(61) ACP_W(62) ACP_W(63)
#undef ACP_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// ---------------------------------------------------------------------------
// Ring control ("Add TMA support for circular buffering pass", "Loop
// Structure" and "Detailed Pseudo-Code"): the prologue loads min(S-1, N)
// trips; the main loop loads trip i+S-1 into slot (i+S-1) % S, waits for
// trip i in slot i % S and consumes it; the epilogue only waits and
// consumes.  `allowed` is the number of this wave's memory operations issued
// after the last load of trip i when its wait executes: the loads of trips
// i+1..min(i+S-1, N-1) (d each) and the stores of every consume since trip
// i's load (st each).  With S == 1 the ring is load, wait, consume.

__device__ __forceinline__ int allowed(int i, int n, int s, int d, int st) {
  int ahead = n - 1 - i;
  if (ahead > s - 1) ahead = s - 1;
  const int behind = i < s - 1 ? i : s - 1;
  return ahead * d + behind * st;
}

template <class P>
__device__ __forceinline__ void run_ring(P& p, int n, int s, int d, int st) {
  const int pro = n < s - 1 ? n : s - 1;
  for (int j = 0; j < pro; ++j) p.load(j, j);
  const int nmain = n - (s - 1) > 0 ? n - (s - 1) : 0;
  int cur = 0, ld = s - 1;
  int i = 0;
  for (; i < nmain; ++i) {
    p.load(i + s - 1, ld);
    p.wait(i, cur, allowed(i, n, s, d, st));
    p.consume(i, cur);
    cur = (cur + 1 == s) ? 0 : cur + 1;
    ld = (ld + 1 == s) ? 0 : ld + 1;
  }
  for (; i < n; ++i) {
    p.wait(i, cur, allowed(i, n, s, d, st));
    p.consume(i, cur);
    cur = (cur + 1 == s) ? 0 : cur + 1;
  }
}

// ---------------------------------------------------------------------------
// Op registry ("elementwise -> smem", "What it accepts" and "How inputs
// change the algorithm").  IEEE binary32 / binary16 arithmetic with
// round-to-nearest-even and no flush of denormals; fma is fused.

template <int DT> struct DType;
template <> struct DType<kF32> { typedef float T; };
template <> struct DType<kF16> { typedef _Float16 T; };
template <> struct DType<kU32> { typedef uint32_t T; };

template <typename T> __device__ __forceinline__ float to_f(T v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f(float v) { return static_cast<T>(v); }

template <int OP, int TIN, int TOUT> struct Op;

template <int TIN, int TOUT> struct Op<kOpSqrt, TIN, TOUT> {
  typedef typename DType<TIN>::T TI;
  typedef typename DType<TOUT>::T TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float, float) { return from_f<TO>(__builtin_sqrtf(to_f(x))); }
};
template <int TIN, int TOUT> struct Op<kOpExp, TIN, TOUT> {
  typedef typename DType<TIN>::T TI;
  typedef typename DType<TOUT>::T TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float, float) { return from_f<TO>(expf(to_f(x))); }
};
template <int TIN, int TOUT> struct Op<kOpZero, TIN, TOUT> {
  typedef typename DType<TIN>::T TI;
  typedef typename DType<TOUT>::T TO;
  static constexpr int NIN = 0;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI, TI, TI, float, float) { return TO(0); }
};
// Byte copy: 32-bit words move unchanged.
template <> struct Op<kOpCopy, kU32, kU32> {
  typedef uint32_t TI;
  typedef uint32_t TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float, float) { return x; }
};
// Staged operands: add / mul of binary16 via binary32 are exact then
// rounded once (24 >= 2 * 11 + 2); fma is fused in the operand type.
template <int T> struct Op<kOpAdd, T, T> {
  typedef typename DType<T>::T TI;
  typedef TI TO;
  static constexpr int NIN = 2;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI a, TI b, TI, float, float) { return from_f<TO>(to_f(a) + to_f(b)); }
};
template <int T> struct Op<kOpMul, T, T> {
  typedef typename DType<T>::T TI;
  typedef TI TO;
  static constexpr int NIN = 2;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI a, TI b, TI, float, float) { return from_f<TO>(to_f(a) * to_f(b)); }
};
template <> struct Op<kOpFma, kF32, kF32> {
  typedef float TI;
  typedef float TO;
  static constexpr int NIN = 3;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI a, TI b, TI c, float, float) { return __builtin_fmaf(a, b, c); }
};
template <> struct Op<kOpFma, kF16, kF16> {
  typedef _Float16 TI;
  typedef _Float16 TO;
  static constexpr int NIN = 3;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI a, TI b, TI c, float, float) { return __builtin_fmaf16(a, b, c); }
};
// Store with reduce-add: the staged elements are added into the destination
// with no-return buffer atomics (32-bit integer add, binary32 add, packed
// binary16 pair add), 4 per 16-byte chunk.
// Running sums of a store with reduce-add: u32 and f32 chunks sum in their
// own type; f16 chunks sum in binary32 (8 lanes of a float vector) and are
// rounded once when the group is added to the destination.
struct Acc4 {
  uint32_t w[4];
};
struct Acc8 {
  float v[8];
};
template <int T> struct ReduceOp;
template <class OP, int MODE> struct AccOf { typedef Acc4 T; };
template <int MODE> struct AccOf<ReduceOp<kF16>, MODE> { typedef Acc8 T; };

template <int T> struct ReduceOp {
  typedef typename DType<T>::T TI;
  typedef TI TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float, float) { return x; }
  typedef typename AccOf<ReduceOp<T>, 3>::T Acc;
  static __device__ __forceinline__ Acc zero_acc() { return Acc{}; }
  static __device__ __forceinline__ Acc accumulate(Acc a, u32x4 v) {
    if constexpr (T == kU32) {
      a.w[0] += v.x;
      a.w[1] += v.y;
      a.w[2] += v.z;
      a.w[3] += v.w;
    } else if constexpr (T == kF32) {
      // through memcpy: a bit cast of a vector element (v.y) was compiled
      // as a cast of element 0
      float x[4], s[4];
      __builtin_memcpy(x, &v, 16);
      __builtin_memcpy(s, a.w, 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += x[e];
      __builtin_memcpy(a.w, s, 16);
    } else {
      _Float16 h[8];
      __builtin_memcpy(h, &v, 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) a.v[e] += static_cast<float>(h[e]);
    }
    return a;
  }
  static __device__ __forceinline__ u32x4 finish(Acc a) {
    if constexpr (T == kF16) {
      _Float16 h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(a.v[e]);
      u32x4 w;
      __builtin_memcpy(&w, h, 16);
      return w;
    } else {
      return u32x4{a.w[0], a.w[1], a.w[2], a.w[3]};
    }
  }
  static __device__ __forceinline__ void add(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t w) {
    if constexpr (T == kF32)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(__builtin_bit_cast(float, w), rs, voff, 0, 0);
    else if constexpr (T == kF16)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_v2f16(__builtin_bit_cast(f16x2, w), rs, voff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(static_cast<int>(w), rs, voff, 0, 0);
  }
};

// Sum over the 64 lanes of a wave in a fixed order, with DPP moves: shift-
// and-add within each row of 16 lanes (lane 15 of a row ends with the row's
// sum), then lane 15 of rows 0 and 2 is broadcast into rows 1 and 3, and
// lane 31 into rows 2 and 3.  Lane 63 holds the total, read as a scalar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift(float v) {
  // lanes shifted in from outside a row, and rows outside the mask, read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_shift<0x111, 0xf>(v);  // row_shr:1
  v += dpp_shift<0x112, 0xf>(v);  // row_shr:2
  v += dpp_shift<0x114, 0xf>(v);  // row_shr:4
  v += dpp_shift<0x118, 0xf>(v);  // row_shr:8
  v += dpp_shift<0x142, 0xa>(v);  // row_bcast:15
  v += dpp_shift<0x143, 0xc>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Row reduction: the staged elements are summed (in binary32) per row.
template <int T> struct ReduceRowsOp {
  typedef typename DType<T>::T TI;
  typedef float TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = false;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float, float) { return to_f(x); }
  // sum of one 16-byte chunk, as a fixed pairwise tree
  static __device__ __forceinline__ float chunk(u32x4 v) {
    TI e[16 / sizeof(TI)];
    __builtin_memcpy(e, &v, 16);
    if constexpr (sizeof(TI) == 4) {
      return (to_f(e[0]) + to_f(e[1])) + (to_f(e[2]) + to_f(e[3]));
    } else {
      return ((to_f(e[0]) + to_f(e[1])) + (to_f(e[2]) + to_f(e[3]))) +
             ((to_f(e[4]) + to_f(e[5])) + (to_f(e[6]) + to_f(e[7])));
    }
  }
};

// Streamed x with per-row scalars (binary32): add x + b, mul a * x, fma a * x + b.
template <int OPC> struct RowOp {
  typedef float TI;
  typedef float TO;
  static constexpr int NIN = 1;
  static constexpr bool ROW = true;
  static __device__ __forceinline__ TO f(TI x, TI, TI, float a, float b) {
    if constexpr (OPC == kOpAdd) return x + b;
    if constexpr (OPC == kOpMul) return a * x;
    return __builtin_fmaf(a, x, b);
  }
};

// ---------------------------------------------------------------------------
// Per-lane map of the rounds f < outer: physical chunk (f * waves + wave) *
// 64 + lane of a slot, its logical position through the swizzle, and from the
// image axes its offsets inside the stage.  Computed once per workgroup.

struct LaneMap {
  uint32_t xoff[kMaxOuter];   // input byte offset from the stage origin
  uint32_t ooff[kMaxOuter];   // output byte offset from the stage origin
  uint32_t oobm[kMaxOuter];   // partial slots along which the chunk lies past the edge
  uint32_t lpos[kMaxOuter];   // logical byte offset of the chunk in the image
  uint32_t abo[kMaxOuter];    // LDS offset of the chunk's row scalar (row ops)
};

// Offsets of the staged byte at physical LDS position pb of the image: the
// logical byte lb (through the swizzle), its input and output byte offsets
// from the stage origin, its stage row (row ops) and the partial slots along
// which it lies past the edge.
struct ByteMap {
  uint32_t lb, xo, oo, row, ob, col;  // col: coordinate along the innermost dim (elements)
};

__device__ __forceinline__ ByteMap map_byte(CArgs* A, uint32_t pb, int n_axes, int swz_mask, int es_log2) {
  ByteMap r;
  r.lb = swz(pb, static_cast<uint32_t>(swz_mask));
  const uint32_t sub_byte = r.lb & ((1u << es_log2) - 1u);  // copies of elements wider than the chunk
  uint32_t e = r.lb >> es_log2;
  r.xo = sub_byte;
  r.oo = sub_byte;
  r.row = 0;
  r.col = 0;
  const uint32_t inner = A->ax_inner_mask;
  uint32_t rel[kPartial] = {0, 0, 0, 0};
#pragma nounroll
  for (int k = n_axes - 1; k >= 0; --k) {
    const uint32_t q = mdiv(e, A->ax_mag[k], A->ax_sh[k]);
    const uint32_t idx = e - q * A->ax_count[k];
    e = q;
    r.xo += idx * A->ax_xs[k];
    r.oo += idx * A->ax_os[k];
    r.row += idx * A->ax_rs[k];
    if ((inner >> k) & 1u) r.col += idx * A->ax_step[k];
    const int ps = A->ax_pslot[k];
#pragma unroll
    for (int s2 = 0; s2 < kPartial; ++s2)
      if (ps == s2) rel[s2] += idx * A->ax_step[k];
  }
  r.ob = 0;
#pragma unroll
  for (int s2 = 0; s2 < kPartial; ++s2)
    if (rel[s2] >= A->prem[s2]) r.ob |= 1u << s2;
  return r;
}

template <int VB>
__device__ __forceinline__ void build_map(CArgs* A, int wave, int lane, LaneMap& m) {
  const int outer = A->outer, waves = A->waves, n_axes = A->n_axes;
  const int swz_mask = A->swizzle, es_log2 = A->esize_log2;
#pragma unroll
  for (int g = 0; g < kMaxOuter; ++g) m.xoff[g] = m.ooff[g] = m.oobm[g] = m.lpos[g] = m.abo[g] = 0;
#pragma nounroll
  for (int f = 0; f < outer; ++f) {
    const ByteMap b = map_byte(A, ((f * waves + wave) * 64u + lane) * VB, n_axes, swz_mask, es_log2);
    const uint32_t abo = (b.row >> 5) * 256u + (b.row & 31u) * 4u;
#pragma unroll
    for (int g = 0; g < kMaxOuter; ++g)
      if (g == f) {
        m.xoff[g] = b.xo;
        m.ooff[g] = b.oo;
        m.oobm[g] = b.ob;
        m.lpos[g] = b.lb;
        m.abo[g] = abo;
      }
  }
}

// Consumer pieces of a widening op: every 16-byte round of a wave (1 KiB of
// LDS) is consumed as two halves of 512 B, lane l taking the 8 bytes at
// 8 * l of each half.  Eight input bytes widen to 16 output bytes, so every
// store instruction writes 1 KiB of whole output rows instead of 16-byte
// pieces 32 bytes apart.  Piece 2 * f + h: output offset, partial slots and
// logical image byte.
template <int N>
__device__ __forceinline__ void build_pieces(CArgs* A, int wave, int lane, int outer, uint32_t (&oo)[N],
                                             uint32_t (&ob)[N], uint32_t (&lp)[N]) {
  const int waves = A->waves, n_axes = A->n_axes;
  const int swz_mask = A->swizzle, es_log2 = A->esize_log2;
#pragma unroll
  for (int g = 0; g < N; ++g) oo[g] = ob[g] = lp[g] = 0;
#pragma nounroll
  for (int q = 0; q < 2 * outer; ++q) {
    const uint32_t f = q >> 1, h = q & 1;
    const ByteMap b = map_byte(A, (f * waves + wave) * 1024u + h * 512u + lane * 8u, n_axes, swz_mask, es_log2);
#pragma unroll
    for (int g = 0; g < N; ++g)
      if (g == q) {
        oo[g] = b.oo;
        ob[g] = b.ob;
        lp[g] = b.lb;
      }
  }
}

// Launch values the ring touches every trip, read from the argument block
// once: they then live in registers across the asm statements (whose memory
// clobbers would otherwise force a reload of every argument per trip).
struct Loc {
  const char* in[3];
  char* out;
  uint64_t in_span, out_span, total_rows;
  int64_t lin_x, lin_o, lin_r;
  int lin, load_nt, store_nt;
  int outer, waves, n_in, row_ops, ab_instr;
  uint32_t in_image_bytes, slot_bytes, ab_off, ab_wave_bytes, out_image_off, subs, tile0;
};

__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  return (static_cast<uint64_t>(uni(static_cast<uint32_t>(v >> 32))) << 32) | uni(static_cast<uint32_t>(v));
}
template <typename P> __device__ __forceinline__ P* unip(P* p) {
  return reinterpret_cast<P*>(uni64(reinterpret_cast<uint64_t>(p)));
}

// Every value passes through readfirstlane: the result is a register value
// the compiler cannot re-derive by reloading the argument block inside the
// ring (a reload would also cost an lgkmcnt wait that drains the LDS reads).
__device__ __forceinline__ Loc load_loc(CArgs* A) {
  Loc L;
  for (int k = 0; k < 3; ++k) L.in[k] = unip(A->in[k]);
  L.out = unip(A->out);
  L.in_span = uni64(A->in_span);
  L.out_span = uni64(A->out_span);
  L.total_rows = uni64(A->total_rows);
  L.lin_x = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_x)));
  L.lin_o = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_o)));
  L.lin_r = static_cast<int64_t>(uni64(static_cast<uint64_t>(A->lin_r)));
  L.lin = uni(A->lin);
  L.load_nt = uni(A->load_nt);
  L.store_nt = uni(A->store_nt);
  L.outer = uni(A->outer);
  L.waves = uni(A->waves);
  L.n_in = uni(A->n_in);
  L.row_ops = uni(A->row_ops);
  L.ab_instr = uni(A->ab_instr);
  L.in_image_bytes = uni(A->in_image_bytes);
  L.slot_bytes = uni(A->slot_bytes);
  L.ab_off = uni(A->ab_off);
  L.ab_wave_bytes = uni(A->ab_wave_bytes);
  L.out_image_off = uni(A->out_image_off);
  L.subs = uni(A->subs);
  L.tile0 = uni(A->tile0);
  return L;
}

struct Trip {
  uint64_t xbase, obase, rbase;
  uint32_t last;   // partial slots along which this stage is the cut last one
  bool beyond;     // stage lies entirely past the tensor
};

__device__ __forceinline__ Trip trip_geometry(CArgs* A, const Loc& L, uint32_t wg, uint32_t grid, int j) {
  Trip t{0, 0, 0, 0u, false};
  if (L.lin) {
    // one stage per tile, exact tiling, row-major contiguous grid
    const uint64_t s = static_cast<uint64_t>(L.tile0) + wg + static_cast<uint64_t>(j) * grid;
    t.xbase = s * static_cast<uint64_t>(L.lin_x);
    t.obase = s * static_cast<uint64_t>(L.lin_o);
    t.rbase = s * static_cast<uint64_t>(L.lin_r);
    return t;
  }
  const uint32_t tl = mdiv(static_cast<uint32_t>(j), A->subs_mag, A->subs_sh);
  uint32_t sub = static_cast<uint32_t>(j) - tl * L.subs;
  uint32_t tile = L.tile0 + wg + tl * grid;
#pragma nounroll
  for (int d = A->rank - 1; d >= 0; --d) {
    const uint32_t qt = mdiv(tile, A->tg_mag[d], A->tg_sh[d]);
    const uint32_t tc = tile - qt * A->tgrid[d];
    tile = qt;
    const uint32_t qs = mdiv(sub, A->sub_mag[d], A->sub_sh[d]);
    const uint32_t scs = sub - qs * A->sub[d];
    sub = qs;
    const uint32_t sc = tc * A->sub[d] + scs;
    if (sc >= A->nst[d]) t.beyond = true;
    const int ps = A->pslot_of_dim[d];
    if (ps >= 0 && sc + 1 == A->nst[d]) t.last |= 1u << ps;
    t.xbase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->xstep[d]);
    t.obase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->ostep[d]);
    t.rbase += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->rstep[d]);
  }
  if (t.beyond) t.xbase = t.obase = t.rbase = 0;
  return t;
}

// Per-lane row-scalar sources: lane l < 32 loads a[row], l >= 32 loads b[row]
// for stage rows q * 32 + (l & 31).  row_ptr[0] is the lane's array,
// row_ptr[1 + q] the row's byte offset from the stage's first row, row_bad[q]
// the partial slots along which the row lies past the edge (all bits when
// the stage has no such row).
__device__ __forceinline__ void build_rows(CArgs* A, int lane, uint64_t* row_ptr, uint32_t* row_bad) {
  // both pointers are read as scalars first: a lane-dependent address into
  // the argument block would become a vector load whose wait lands in the ring
  const uint64_t pa = reinterpret_cast<uint64_t>(A->row_a), pb = reinterpret_cast<uint64_t>(A->row_b);
  const uint64_t ua = (static_cast<uint64_t>(uni(static_cast<uint32_t>(pa >> 32))) << 32) | uni(static_cast<uint32_t>(pa));
  const uint64_t ub = (static_cast<uint64_t>(uni(static_cast<uint32_t>(pb >> 32))) << 32) | uni(static_cast<uint32_t>(pb));
  row_ptr[0] = lane < 32 ? ua : ub;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    row_ptr[1 + q] = 0;
    row_bad[q] = ~0u;
    if (!A->row_ops || q >= A->ab_instr) continue;
    uint32_t r = q * 32u + (lane & 31);
    if (r >= static_cast<uint32_t>(A->n_rows)) continue;
    uint64_t off = 0;
    uint32_t bad = 0;
    for (int d = A->rank - 2; d >= 0; --d) {
      const uint32_t sb = A->sbox[d];
      const uint32_t rel = r % sb;
      r /= sb;
      off += static_cast<uint64_t>(rel) * static_cast<uint64_t>(A->rstep[d] / sb);
      const int ps = A->pslot_of_dim[d];
      if (ps >= 0 && rel >= A->prem[ps]) bad |= 1u << ps;
    }
    row_ptr[1 + q] = off * 4u;
    row_bad[q] = bad;
  }
}

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

template <int OB, int CP>
__device__ __forceinline__ void store_chunk_cp(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const uint32_t* w) {
  if constexpr (OB == 32) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rs, voff, 0, CP);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[4], w[5], w[6], w[7]}, rs, voff + 16u, 0, CP);
  } else if constexpr (OB == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rs, voff, 0, CP);
  } else if constexpr (OB == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rs, voff, 0, CP);
  } else if constexpr (OB == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, voff, 0, CP);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[0]), rs, voff, 0, CP);
  }
}

// Stores go out non-temporal (cache policy bit NT) unless disabled: the
// output is written once and never read back by the kernel.
template <int OB>
__device__ __forceinline__ void store_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t voff, const uint32_t* w, bool nt) {
  if (nt)
    store_chunk_cp<OB, 2>(rs, voff, w);
  else
    store_chunk_cp<OB, 0>(rs, voff, w);
}

template <class OP, int VB>
struct ChunkShape {
  static constexpr int EI = sizeof(typename OP::TI);
  static constexpr int EO = sizeof(typename OP::TO);
  static constexpr int NE = VB / EI;            // elements per chunk
  static constexpr int OB = NE * EO;            // output bytes per chunk
  static constexpr int ST = OB == 32 ? 2 : 1;   // stores per chunk
};

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
  __device__ __forceinline__ void wait(int, int, int k) { wait_vmcnt(k); }
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

// ---------------------------------------------------------------------------
// Linear stage grid (one full stage per tile, row-major contiguous), 16-byte
// rounds, OUTER rounds per thread known at compile time.  Same ring control
// and wait counts as the general engine; per trip only the stage base (one
// multiply) changes, and no chunk can be out of bounds.
// * Streaming (STAGE_OUT false): one staged operand.
// * Tile ewise (STAGE_OUT true, "elementwise -> smem"): OP::NIN staged
//   operands, and the result goes through the LDS output image before the
//   store.  A stage is 2^k consecutive tiles (one ring trip), round f
//   belonging to tile f >> tile_rounds_log2 of it.

// Rounds consumed together: the largest power of two dividing `total` (a
// power of two) whose staged operands (ns each) stay within `cap` registers'
// worth of chunks.
constexpr int round_group(int total, int ns, int cap) {
  int g = total;
  while (g > 1 && g * (ns > 0 ? ns : 1) > cap) g /= 2;
  return g;
}

template <class OP, int OUTER, bool SROW, bool STAGE_OUT>
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
  bool load_nt, store_nt;
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

  __device__ __forceinline__ void load(int j, int slot) {
    const uint64_t s = stage(j);
    const uint64_t xb = s * lin_x;
    const uint32_t range = range_from(in_span, xb);
    const uint32_t base = lds0 + slot * slot_bytes + wave * 1024u;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const v4i rs = rsrc_v4(in[k] + xb, range);
#pragma unroll
      for (int f = 0; f < OUTER; ++f) dma_b128(rs, xoff[f], base + k * in_image_bytes + f * waves_kb, load_nt);
    }
    if constexpr (OP::ROW && !SROW) {
      const uint64_t rb = s * lin_r;
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
  __device__ __forceinline__ void wait(int i, int, int k) {
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
    wait_vmcnt(k);
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
        store_chunk<CS::OB>(rs, ooff[f], words, store_nt);
      }
    }
  }
};

template <class OP, int OUTER, bool SROW, bool STAGE_OUT = false>
__global__ __launch_bounds__(1024) void stream_lin_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  CArgs* A = kargs();
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t n_tiles = A->n_tiles;
  const int n = static_cast<int>(wg < n_tiles ? (n_tiles - wg + grid - 1) / grid : 0);
  if (n == 0) return;
  LaneMap m;
  build_map<16>(A, wave, lane, m);
  uint64_t row_ptr[3] = {0, 0, 0};
  uint32_t row_bad[2] = {~0u, ~0u};
  if constexpr (OP::ROW && !SROW) build_rows(A, lane, row_ptr, row_bad);
  uint32_t row_ok[2] = {row_bad[0] == 0u, row_bad[1] == 0u};
  const Loc L = load_loc(A);
  LinPolicy<OP, OUTER, SROW, STAGE_OUT> p;
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
  const int d = LinPolicy<OP, OUTER, SROW, STAGE_OUT>::NL * OUTER + ((OP::ROW && !SROW) ? L.ab_instr : 0);
  run_ring(p, n, uni(A->stages), d, OUTER * CS::ST);
}

// ---------------------------------------------------------------------------
// Row reduction on a linear stage grid whose wave blocks each lie in one row
// and whose rows each lie in one wave (the wave-local case): the linear
// kernel's lean trip (stage base = one multiply) with the wave-local
// reduction of the general kernel.  Stage s holds rows s * lin_r + (the
// packed offsets of its rows); lane k of a wave owns the wave's k-th
// distinct row.

template <class OP, int OUTER>
struct LinRowsPolicy {
  unsigned char* lds;
  const char* in0;
  __amdgpu_buffer_rsrc_t out_rs;  // the whole row array
  uint64_t in_span, lin_x, lin_r;
  uint32_t lds0, slot_bytes, wg, grid, waves_kb;
  int wave, lane;
  bool load_nt, one_row;
  uint32_t xoff[OUTER], row_of[OUTER];
  uint32_t lrow, loff;  // this lane's row of the stage (~0: none) and its packed offset

  __device__ __forceinline__ uint64_t stage(int j) const { return wg + static_cast<uint64_t>(j) * grid; }

  __device__ __forceinline__ void load(int j, int slot) {
    const uint64_t xb = stage(j) * lin_x;
    const v4i rs = rsrc_v4(in0 + xb, range_from(in_span, xb));
    const uint32_t base = lds0 + slot * slot_bytes + wave * 1024u;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) dma_b128(rs, xoff[f], base + f * waves_kb, load_nt);
  }
  __device__ __forceinline__ void wait(int, int, int k) { wait_vmcnt(k); }

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

template <class OP, int OUTER>
__global__ __launch_bounds__(1024) void rows_lin_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  CArgs* A = kargs();
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t n_tiles = A->n_tiles;
  const int n = static_cast<int>(wg < n_tiles ? (n_tiles - wg + grid - 1) / grid : 0);
  if (n == 0) return;
  LaneMap m;
  build_map<16>(A, wave, lane, m);
  const Loc L = load_loc(A);
  LinRowsPolicy<OP, OUTER> p;
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
  run_ring(p, n, uni(A->stages), OUTER, 1);
}

// ---------------------------------------------------------------------------
// General lean kernel: any stage grid (partial and out-of-range stages,
// sub-stages inside a workgroup tile, persistent grids), 16-byte rounds,
// OUTER rounds per thread known at compile time.  Trip geometry lives in a
// table in VGPR lanes: lane l of every wave computes trip (batch * 64 + l)
// with vector arithmetic, and each trip reads its row with v_readlane.  Two
// table sets alternate so that the load cursor (up to S-1 trips ahead) can
// enter the next batch while the consume cursor finishes the current one.

struct TripRow {
  uint32_t xlo, xhi, olo, ohi, rlo, flags;  // flags: bits 0..3 last-stage slots, bit 8 out of range
};

__device__ __forceinline__ TripRow trip_lane(CArgs* A, uint32_t wg, uint32_t grid, uint32_t tile0, uint32_t subs,
                                             uint32_t subs_mag, uint32_t subs_sh, int rank, uint32_t tpt_log2,
                                             uint32_t j) {
  const uint32_t tl = mdiv(j, subs_mag, subs_sh);
  uint32_t sub = j - tl * subs;
  const uint32_t per_wg = A->per_wg;
  uint32_t tile = per_wg ? tile0 + wg * per_wg + tl
                         : tile0 + (((wg + (tl >> tpt_log2) * grid) << tpt_log2) | (tl & ((1u << tpt_log2) - 1u)));
  uint64_t xb = 0, ob = 0, rb = 0;
  uint32_t flags = 0;
  // rolled: the per-dim parameters are read on each refill (once per 64
  // trips) rather than held in scalar registers across the ring
#pragma nounroll
  for (int d = rank - 1; d >= 0; --d) {
    const uint32_t qt = mdiv(tile, A->tg_mag[d], A->tg_sh[d]);
    const uint32_t tc = tile - qt * A->tgrid[d];
    tile = qt;
    const uint32_t qs = mdiv(sub, A->sub_mag[d], A->sub_sh[d]);
    const uint32_t scs = sub - qs * A->sub[d];
    sub = qs;
    const uint32_t sc = tc * A->sub[d] + scs;
    const uint32_t nst = A->nst[d];
    if (sc >= nst) flags |= 0x100u;
    const int ps = A->pslot_of_dim[d];
    if (ps >= 0 && sc + 1 == nst) flags |= 1u << ps;
    xb += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->xstep[d]);
    ob += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->ostep[d]);
    rb += static_cast<uint64_t>(sc) * static_cast<uint64_t>(A->rstep[d]);
  }
  if (tile != 0) flags |= 0x100u;  // past the last tile
  if (flags & 0x100u) xb = ob = rb = 0;
  return TripRow{static_cast<uint32_t>(xb), static_cast<uint32_t>(xb >> 32), static_cast<uint32_t>(ob),
                 static_cast<uint32_t>(ob >> 32), static_cast<uint32_t>(rb), flags};
}

__device__ __forceinline__ uint32_t rdl(uint32_t v, uint32_t lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), static_cast<int>(lane)));
}

template <class OP, int MODE, int OUTER, bool SROW, int ZSET = 0, bool GROUP = false>
struct GenPolicy {
  static constexpr bool STAGE_OUT = (MODE == 1);
  // staged operands: every input of a tile op or of a two-tensor stream op;
  // streams with per-row scalars stage x only
  static constexpr int NS = (MODE == 0 || OP::ROW) ? 1 : OP::NIN;
  // ZSET: the last staged operand is loaded synchronously (registers, wait,
  // LDS store) into its image instead of by a direct-to-LDS load
  static constexpr int NDMA = ZSET ? NS - 1 : NS;
  // widening ops (16 input bytes -> 32 output bytes) consume 8-byte pieces
  // (tile ops up to 4 rounds: beyond, the piece maps no longer fit in registers)
  static constexpr bool SPLIT = (MODE == 2 || (MODE == 1 && OUTER <= 4)) && ChunkShape<OP, 16>::OB == 32;
  static constexpr int NP = SPLIT ? 2 * OUTER : 1;
  uint32_t pooff[NP], poobm[NP], plpos[NP];
  CArgs* A;
  unsigned char* lds;
  const char* in[3];
  char* out;
  uint64_t in_span, out_span, total_rows;
  uint32_t lds0, slot_bytes, in_image_bytes, out_image_off, ab_base, waves_kb, wg, grid, tile0, subs, subs_mag, subs_sh;
  uint32_t tpt_log2, tile_lds;  // tiles per trip (log2) and LDS bytes of one tile's images in a slot
  // row reduction (MODE 4): each round's partial-sum index (row * row_chunks
  // + chunk of the row), and the reduction geometry
  uint32_t pidx[OUTER];
  uint32_t row_chunks, red_rows, part_off, part_bytes, waves;
  uint32_t red_off, red_bad;  // lane k: packed-row offset and cut-edge slots of the wave's k-th row
  // store with reduce-add over batch dims: trips per destination tile, the
  // trips summed so far and the lane's running sums
  uint32_t red_group, rcount;
  typename AccOf<OP, MODE>::T racc[GROUP ? OUTER : 1];
  // wave-local rows: lane k holds the wave's k-th distinct row (in round
  // order; ~0 for none), its packed-row offset and cut-edge slots
  bool red_local;
  bool one_row;      // wave-local: all of the wave's blocks lie in one row
  uint32_t lrow, loff, lbad;
  int wave, lane, rank, ab_instr, swizzle, esize_log2;
  bool load_nt, store_nt;
  uint32_t xoff[OUTER], ooff[OUTER], oobm[OUTER], lpos[OUTER], abo[OUTER];
  // two table sets as separate members: a dynamically indexed array would
  // live in scratch memory, whose loads share the wave's vmcnt with the ring
  TripRow tab0, tab1;
  uint64_t row_ptr[3];   // [0] lane's array, [1 + q] row byte offset in the stage
  uint32_t row_bad[2];   // partial slots along which the lane's row q lies past the edge
  // SROW: this wave's row (relative to the stage) of each round, and the
  // scalars of the trip being consumed, read through the scalar cache
  const float __attribute__((address_space(4)))* ca;
  const float __attribute__((address_space(4)))* cb;
  uint32_t row_of[OUTER];
  float sa[OUTER], sb[OUTER];

  __device__ __forceinline__ void fill(int set, uint32_t j0) {
    const TripRow r =
        trip_lane(A, wg, grid, tile0, subs, subs_mag, subs_sh, rank, tpt_log2, j0 + static_cast<uint32_t>(lane));
    // field-wise selects: a conditional store of the whole row would be
    // merged into one store through a selected address, i.e. into memory
    const bool lo = set == 0;
    tab0 = TripRow{lo ? r.xlo : tab0.xlo, lo ? r.xhi : tab0.xhi, lo ? r.olo : tab0.olo,
                   lo ? r.ohi : tab0.ohi, lo ? r.rlo : tab0.rlo, lo ? r.flags : tab0.flags};
    tab1 = TripRow{lo ? tab1.xlo : r.xlo, lo ? tab1.xhi : r.xhi, lo ? tab1.olo : r.olo,
                   lo ? tab1.ohi : r.ohi, lo ? tab1.rlo : r.rlo, lo ? tab1.flags : r.flags};
  }
  struct T {
    uint64_t xb, ob, rb;
    uint32_t flags;
  };
  __device__ __forceinline__ T row(int j) const {
    const uint32_t l = static_cast<uint32_t>(j) & 63u;
    const bool hi = ((j >> 6) & 1) != 0;
    T t;
    t.xb = (static_cast<uint64_t>(rdl(hi ? tab1.xhi : tab0.xhi, l)) << 32) | rdl(hi ? tab1.xlo : tab0.xlo, l);
    t.ob = (static_cast<uint64_t>(rdl(hi ? tab1.ohi : tab0.ohi, l)) << 32) | rdl(hi ? tab1.olo : tab0.olo, l);
    t.rb = rdl(hi ? tab1.rlo : tab0.rlo, l);
    t.flags = rdl(hi ? tab1.flags : tab0.flags, l);
    return t;
  }

  // Table entry e is the workgroup's e-th tile (tile ops) or stage; ring
  // trip j holds entries j * 2^tpt_log2 ... (a batch boundary of the table
  // always falls on the first entry of a trip).
  __device__ __forceinline__ void load(int j, int slot) {
    const int e0 = j << tpt_log2;
    if (e0 > 0 && (e0 & 63) == 0) fill((e0 >> 6) & 1, static_cast<uint32_t>(e0));
#pragma nounroll
    for (int u = 0; u < (1 << tpt_log2); ++u) load_entry(e0 + u, slot * slot_bytes + u * tile_lds);
  }

  __device__ __forceinline__ void load_entry(int j, uint32_t sl) {
    const T t = row(j);
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    const uint32_t sbase = lds0 + sl + wave * 1024u;
#pragma unroll
    for (int k = 0; k < NDMA; ++k) {
      const v4i rs = rsrc_v4(in[k] + t.xb, range_from(in_span, t.xb));
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const bool ok = !beyond && (oobm[f] & last) == 0;
        dma_b128(rs, ok ? xoff[f] : kOobOffset, sbase + k * in_image_bytes + f * waves_kb, load_nt);
      }
    }
    if constexpr (ZSET) {
      // synchronous staging: the data must reach registers before it can be
      // stored to LDS, so the wave waits for all its outstanding loads here
      const __amdgpu_buffer_rsrc_t rz = rsrc_store(const_cast<char*>(in[NDMA]) + t.xb, range_from(in_span, t.xb));
      u32x4 zv[OUTER];
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const bool ok = !beyond && (oobm[f] & last) == 0;
        zv[f] = __builtin_amdgcn_raw_buffer_load_b128(rz, ok ? xoff[f] : kOobOffset, 0, 0);
      }
      wait_vmcnt(0);
#pragma unroll
      for (int f = 0; f < OUTER; ++f)
        *reinterpret_cast<u32x4*>(__builtin_assume_aligned(
            lds + sl + NDMA * in_image_bytes + f * waves_kb + wave * 1024u + lane * 16u, 16)) = zv[f];
    }
    if constexpr (OP::ROW && !SROW) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q >= ab_instr) continue;
        const bool ok = !beyond && (row_bad[q] & last) == 0;
        uint64_t r = ok ? t.rb + row_ptr[1 + q] / 4u : 0u;
        if (r >= total_rows) r = 0;
        dma_global_b32(reinterpret_cast<const void*>(row_ptr[0] + r * 4u), lds0 + sl + ab_base + q * 256u);
      }
    }
  }

  __device__ __forceinline__ void wait(int i, int, int k) {
    if constexpr (OP::ROW && SROW) {
      // rows of a cut stage may lie past the tensor: their results are
      // never stored, and they read row 0 instead of memory past the arrays
      const T t = row(i);
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        uint64_t r = t.rb + row_of[f];
        if (r >= total_rows) r = 0;
        sa[f] = ca[r];
        sb[f] = cb[r];
      }
    }
    wait_vmcnt(k);
  }

  // Widening ops: 8 input bytes per lane and piece, 16 output bytes.
  __device__ __forceinline__ void consume_pieces(__amdgpu_buffer_rsrc_t rs, uint32_t sl, bool beyond, uint32_t last) {
    typedef typename OP::TI TI;
    typedef typename OP::TO TO;
    constexpr int NE = 8 / sizeof(TI);
    constexpr int GRP = round_group(NP, NS, 32);
    static_assert(NP % GRP == 0, "piece groups must tile the pieces");
#pragma unroll
    for (int g0 = 0; g0 < NP; g0 += GRP) {
      u32x2 v[NS > 0 ? NS : 1][GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = g0 + u, f = q >> 1, h = q & 1;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          v[k][u] = *reinterpret_cast<const u32x2*>(__builtin_assume_aligned(
              lds + sl + k * in_image_bytes + f * waves_kb + wave * 1024u + h * 512u + lane * 8u, 8));
        if constexpr (NS == 0) v[0][u] = u32x2{0, 0};
      }
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int q = g0 + u;
        TI in0[NE], in1[NE], in2[NE];
        __builtin_memcpy(in0, &v[0][u], 8);
        __builtin_memcpy(in1, &v[NS > 1 ? 1 : 0][u], 8);
        __builtin_memcpy(in2, &v[NS > 2 ? 2 : 0][u], 8);
        TO res[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) res[e] = OP::f(in0[e], in1[e], in2[e], 0.f, 0.f);
        uint32_t words[4];
        __builtin_memcpy(words, res, 16);
        if constexpr (STAGE_OUT) {
          const uint32_t lo = (plpos[q] >> esize_log2) * sizeof(TO);
          __builtin_memcpy(lds + out_image_off + swz(lo, swizzle), words, 16);
          asm volatile("" ::: "memory");
          __builtin_memcpy(words, lds + out_image_off + swz(lo, swizzle), 16);
        }
        const bool ok = !beyond && (poobm[q] & last) == 0;
        store_chunk<16>(rs, ok ? pooff[q] : kOobOffset, words, store_nt);
      }
    }
  }

  // Row reduction of one staged trip.  Each lane sums its chunks and puts
  // the partials into LDS at (row, chunk of the row); after a workgroup
  // barrier each wave reduces whole rows: lane-strided sums over the row's
  // chunks, then a DPP sum across the 64 lanes, in a fixed order.  Lane 0
  // stores the row's sum.  Partials alternate between two buffers, so the
  // next trip's writes never meet this trip's reads (every wave passes the
  // next barrier only after finishing them).
  // Rows that a single wave holds entirely (each 1 KiB wave block inside one
  // row): the wave sums each block (chunk sums, then a DPP sum over the 64
  // lanes); lane k accumulates the blocks of the wave's k-th row in round
  // order, and one store instruction writes every row total of the trip.
  // No other wave is involved, so there is no barrier.
  __device__ __forceinline__ void reduce_rows_local(uint32_t sl, const T& t, __amdgpu_buffer_rsrc_t rs) {
    float part[OUTER];
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
      part[f] = OP::chunk(v);
    }
    float acc = 0.f;
    if (one_row) {
      // every block of the wave lies in one row: each lane adds its chunk
      // partials in round order, then one cross-lane sum
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
    const bool ok = (t.flags & 0x100u) == 0 && lrow != ~0u && (lbad & t.flags & 0xFFu) == 0;
    const uint64_t g = t.rb + loff;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), rs,
                                          ok ? static_cast<uint32_t>(g * 4u) : kOobOffset, 0, 0);
  }

  __device__ __forceinline__ void reduce_rows_trip(int i, uint32_t sl, const T& t, __amdgpu_buffer_rsrc_t rs) {
    if (red_local) {
      reduce_rows_local(sl, t, rs);
      return;
    }
    const uint32_t buf = part_off + (static_cast<uint32_t>(i) & 1u) * part_bytes;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
      *reinterpret_cast<float*>(lds + buf + pidx[f] * 4u) = OP::chunk(v);
    }
    // only LDS traffic is waited for: the ring's loads stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    uint32_t k = 0;
#pragma nounroll
    for (uint32_t r = static_cast<uint32_t>(wave); r < red_rows; r += waves, ++k) {
      float acc = 0.f;
      for (uint32_t c = static_cast<uint32_t>(lane); c < row_chunks; c += 64u)
        acc += *reinterpret_cast<const float*>(lds + buf + (r * row_chunks + c) * 4u);
      acc = wave_sum(acc);
      // the row's place in the tensor and the cut edges it lies past (lane k
      // of the wave holds them for the wave's k-th row)
      const uint32_t roff = rdl(red_off, k), rbad = rdl(red_bad, k);
      const bool ok = !beyond && (rbad & last) == 0;
      const uint64_t g = t.rb + roff;
      if (lane == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), rs,
                                              ok ? static_cast<uint32_t>(g * 4u) : kOobOffset, 0, 0);
    }
  }

  __device__ __forceinline__ void consume(int i, int slot) {
    const int e0 = i << tpt_log2;
#pragma nounroll
    for (int u = 0; u < (1 << tpt_log2); ++u) consume_entry(e0 + u, slot * slot_bytes + u * tile_lds);
  }

  __device__ __forceinline__ void consume_entry(int i, uint32_t sl) {
    typedef ChunkShape<OP, 16> CS;
    typedef typename OP::TI TI;
    typedef typename OP::TO TO;
    const T t = row(i);
    const bool beyond = (t.flags & 0x100u) != 0;
    const uint32_t last = t.flags & 0xFFu;
    const __amdgpu_buffer_rsrc_t rs = rsrc_store(out + t.ob, range_from(out_span, t.ob));
    if constexpr (SPLIT) {
      consume_pieces(rs, sl, beyond, last);
      return;
    }
    if constexpr (MODE == 4) {
      reduce_rows_trip(i, sl, t, rs);
      return;
    }
    if constexpr (MODE == 3) {
      if constexpr (GROUP) {
        // sum the group's contributions in registers; the group's last trip
        // adds the sums into the destination (past-the-end chunks were
        // staged as zeros and add nothing)
#pragma unroll
        for (int f = 0; f < OUTER; ++f) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(
              __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
          racc[f] = OP::accumulate(racc[f], v);
        }
        if (++rcount == red_group) {
          rcount = 0;
#pragma unroll
          for (int f = 0; f < OUTER; ++f) {
            const bool ok = !beyond && (oobm[f] & last) == 0;
            const uint32_t o = ok ? ooff[f] : kOobOffset;
            const u32x4 w = OP::finish(racc[f]);
            OP::add(rs, o, w.x);
            OP::add(rs, o + 4u, w.y);
            OP::add(rs, o + 8u, w.z);
            OP::add(rs, o + 12u, w.w);
            racc[f] = OP::zero_acc();
          }
        }
        return;
      }
      // store with reduce-add: four 4-byte atomics per staged chunk
#pragma unroll
      for (int f = 0; f < OUTER; ++f) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(
            __builtin_assume_aligned(lds + sl + f * waves_kb + wave * 1024u + lane * 16u, 16));
        const bool ok = !beyond && (oobm[f] & last) == 0;
        const uint32_t o = ok ? ooff[f] : kOobOffset;
        OP::add(rs, o, v.x);
        OP::add(rs, o + 4u, v.y);
        OP::add(rs, o + 8u, v.z);
        OP::add(rs, o + 12u, v.w);
      }
      return;
    }
    // rounds in groups whose staged operands fit in registers together
    constexpr int GRP = round_group(OUTER, NS, 16);
    static_assert(OUTER % GRP == 0, "round groups must tile the rounds");
#pragma unroll
    for (int g0 = 0; g0 < OUTER; g0 += GRP) {
      u32x4 v[NS > 0 ? NS : 1][GRP];
      float ra[GRP], rb[GRP];
#pragma unroll
      for (int u = 0; u < GRP; ++u) {
        const int f = g0 + u;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          v[k][u] = *reinterpret_cast<const u32x4*>(
              __builtin_assume_aligned(lds + sl + k * in_image_bytes + f * waves_kb + wave * 1024u + lane * 16u, 16));
        if constexpr (NS == 0) v[0][u] = u32x4{0, 0, 0, 0};
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
        __builtin_memcpy(in1, &v[NS > 1 ? 1 : 0][u], 16);
        __builtin_memcpy(in2, &v[NS > 2 ? 2 : 0][u], 16);
        TO res[CS::NE];
#pragma unroll
        for (int e = 0; e < CS::NE; ++e) res[e] = OP::f(in0[e], in1[e], in2[e], ra[u], rb[u]);
        uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        __builtin_memcpy(words, res, CS::OB);
        if constexpr (STAGE_OUT) {
          // the output tile is LDS-resident ("elementwise -> smem") and is copied out from there
          const uint32_t lo = (lpos[f] >> esize_log2) * CS::EO;
          constexpr int P = (CS::OB + 15) / 16;
          constexpr int PB = CS::OB < 16 ? CS::OB : 16;
#pragma unroll
          for (int piece = 0; piece < P; ++piece) {
            const uint32_t lp = lo + piece * 16;
            __builtin_memcpy(lds + out_image_off + swz(lp, swizzle), words + piece * 4, PB);
          }
          asm volatile("" ::: "memory");
#pragma unroll
          for (int piece = 0; piece < P; ++piece) {
            const uint32_t lp = lo + piece * 16;
            __builtin_memcpy(words + piece * 4, lds + out_image_off + swz(lp, swizzle), PB);
          }
        }
        const bool ok = !beyond && (oobm[f] & last) == 0;
        store_chunk<CS::OB>(rs, ok ? ooff[f] : kOobOffset, words, store_nt);
      }
    }
  }
};

template <class OP, int MODE, int OUTER, bool SROW, int ZSET = 0, bool GROUP = false>
__global__ __launch_bounds__(1024) void gen_kernel_t(const EngineArgs) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];
  CArgs* A = kargs();
  const int lane = threadIdx.x & 63;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const uint32_t grid = gridDim.x;
  uint32_t wg = blockIdx.x;
  if (A->xcd_remap) wg = (wg & 7u) * (grid >> 3) + (wg >> 3);
  const uint32_t tpt_log2 = uni(A->tpt_log2);
  const uint32_t groups = (A->n_tiles + (1u << tpt_log2) - 1u) >> tpt_log2;
  const uint32_t per_wg = uni(A->per_wg);
  const uint32_t first = wg * per_wg;
  const uint32_t mine = per_wg ? (first < A->n_tiles ? min(per_wg, A->n_tiles - first) : 0u)
                               : (wg < groups ? (groups - wg + grid - 1) / grid : 0);
  const int n = static_cast<int>(mine * A->subs);  // ring trips
  if (n == 0) return;
  LaneMap m;
  build_map<16>(A, wave, lane, m);
  uint64_t row_ptr[3] = {0, 0, 0};
  uint32_t row_bad[2] = {~0u, ~0u};
  if constexpr (OP::ROW && !SROW) build_rows(A, lane, row_ptr, row_bad);
  const Loc L = load_loc(A);
  GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP> p;
  p.tpt_log2 = tpt_log2;
  p.tile_lds = L.slot_bytes >> tpt_log2;
  p.A = A;
  p.lds = lds;
  for (int k = 0; k < 3; ++k) p.in[k] = L.in[k];
  p.out = L.out;
  p.in_span = L.in_span;
  p.out_span = L.out_span;
  p.total_rows = L.total_rows;
  p.lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  p.slot_bytes = L.slot_bytes;
  p.in_image_bytes = L.in_image_bytes;
  p.out_image_off = L.out_image_off;
  p.ab_base = L.ab_off + wave * L.ab_wave_bytes;
  p.waves_kb = static_cast<uint32_t>(L.waves) * 1024u;
  p.wg = wg;
  p.grid = grid;
  p.tile0 = L.tile0;
  p.subs = L.subs;
  p.subs_mag = uni(A->subs_mag);
  p.subs_sh = uni(A->subs_sh);
  p.wave = wave;
  p.lane = lane;
  p.rank = uni(A->rank);
  p.ab_instr = L.ab_instr;
  p.swizzle = uni(A->swizzle);
  p.esize_log2 = uni(A->esize_log2);
  p.load_nt = L.load_nt != 0;
  p.store_nt = L.store_nt != 0;
#pragma unroll
  for (int q = 0; q < 3; ++q) p.row_ptr[q] = row_ptr[q];
#pragma unroll
  for (int q = 0; q < 2; ++q) p.row_bad[q] = row_bad[q];
  p.ca = (const float __attribute__((address_space(4)))*)(unip(A->row_a));
  p.cb = (const float __attribute__((address_space(4)))*)(unip(A->row_b));
#pragma unroll
  for (int f = 0; f < OUTER; ++f) {
    p.xoff[f] = m.xoff[f];
    p.ooff[f] = m.ooff[f];
    p.oobm[f] = m.oobm[f];
    p.lpos[f] = m.lpos[f];
    p.abo[f] = m.abo[f];
    const uint32_t abo = uni(m.abo[f]);
    p.row_of[f] = (abo >> 8) * 32u + (abo & 255u) / 4u;
    p.sa[f] = p.sb[f] = 0.f;
  }
  if constexpr (GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP>::SPLIT)
    build_pieces(A, wave, lane, OUTER, p.pooff, p.poobm, p.plpos);
  if constexpr (GROUP) {
    p.red_group = uni(A->red_group);
    p.rcount = 0;
#pragma unroll
    for (int f = 0; f < OUTER; ++f) p.racc[f] = OP::zero_acc();
  }
  int red_stores = 0;  // row reduction: rows this wave stores per trip
  if constexpr (MODE == 4) {
    p.row_chunks = uni(A->row_chunks);
    p.red_rows = uni(A->red_rows);
    p.part_off = uni(A->part_off);
    p.part_bytes = uni(A->part_bytes);
    p.waves = static_cast<uint32_t>(L.waves);
    const int n_axes = uni(A->n_axes), swz_mask = uni(A->swizzle), es_log2 = uni(A->esize_log2);
#pragma unroll
    for (int f = 0; f < OUTER; ++f) {
      const ByteMap b = map_byte(A, ((f * L.waves + wave) * 64u + lane) * 16u, n_axes, swz_mask, es_log2);
      p.pidx[f] = b.row * p.row_chunks + ((b.col << es_log2) >> 4);
    }
    red_stores = static_cast<uint32_t>(wave) < p.red_rows
                     ? static_cast<int>((p.red_rows - wave + p.waves - 1) / p.waves) : 0;
    // lane k: the wave's k-th row r = wave + k * waves of a stage (at most
    // 64 per wave): its packed-row offset from the stage's first row and the
    // partial slots along which it lies past the edge of a cut stage
    const uint32_t r = static_cast<uint32_t>(wave) + static_cast<uint32_t>(lane) * p.waves;
    uint32_t rr = r < p.red_rows ? r : 0u, off = 0, bad = 0;
    for (int dd = p.rank - 2; dd >= 0; --dd) {
      const uint32_t sb = A->sbox[dd];
      const uint32_t rel = rr % sb;
      rr /= sb;
      off += rel * A->rowstr[dd];
      const int ps = A->pslot_of_dim[dd];
      if (ps >= 0 && rel >= A->prem[ps]) bad |= 1u << ps;
    }
    p.red_off = off;
    p.red_bad = bad;
    p.red_local = uni(A->red_local) != 0;
    p.one_row = true;
#pragma unroll
    for (int f = 1; f < OUTER; ++f) p.one_row = p.one_row && p.row_of[f] == p.row_of[0];
    p.lrow = ~0u;
    p.loff = p.lbad = 0;
    if (p.red_local) {
      // the wave's distinct block rows in round order; lane k takes the k-th
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
      uint32_t rr2 = p.lrow != ~0u ? p.lrow : 0u, off2 = 0, bad2 = 0;
      for (int dd = p.rank - 2; dd >= 0; --dd) {
        const uint32_t sb = A->sbox[dd];
        const uint32_t rel = rr2 % sb;
        rr2 /= sb;
        off2 += rel * A->rowstr[dd];
        const int ps = A->pslot_of_dim[dd];
        if (ps >= 0 && rel >= A->prem[ps]) bad2 |= 1u << ps;
      }
      p.loff = off2;
      p.lbad = bad2;
      red_stores = 1;  // one store instruction per trip
    }
  }
  p.tab1 = TripRow{0, 0, 0, 0, 0, 0};
  p.fill(0, 0u);
  typedef ChunkShape<OP, 16> CS;
  constexpr int NS = GenPolicy<OP, MODE, OUTER, SROW, ZSET, GROUP>::NS;
  const int d = (NS * OUTER + ((OP::ROW && !SROW) ? L.ab_instr : 0)) << tpt_log2;
  // grouped reduce-add stores only on a group's last trip: counting none
  // per trip only makes the waits stronger
  const int st = MODE == 4 ? red_stores : (MODE == 3 ? (GROUP ? 0 : OUTER * 4) : OUTER * CS::ST);
  run_ring(p, n, uni(A->stages), d, st << tpt_log2);
}

}  // namespace dev

struct KernelEntry {
  KernelKey key;
  const void* fn;
};

#define ACP_K(OPC, TIN, TOUT, VB, MODE, ...) \
  KernelEntry{KernelKey{OPC, TIN, TOUT, VB, MODE, 0, 0}, \
              reinterpret_cast<const void*>(&dev::engine_kernel_t<__VA_ARGS__, VB, (MODE == 1)>)}
#define ACP_L(OPC, TIN, TOUT, OUTER, SR, ...)                         \
  KernelEntry{KernelKey{OPC, TIN, TOUT, 16, 3, OUTER, SR}, \
              reinterpret_cast<const void*>(&dev::stream_lin_kernel_t<__VA_ARGS__, OUTER, (SR != 0)>)}
#define ACP_LIN(OPC, TIN, TOUT, ...) \
  ACP_L(OPC, TIN, TOUT, 1, 0, __VA_ARGS__), ACP_L(OPC, TIN, TOUT, 2, 0, __VA_ARGS__), ACP_L(OPC, TIN, TOUT, 4, 0, __VA_ARGS__), \
      ACP_L(OPC, TIN, TOUT, 8, 0, __VA_ARGS__)
#define ACP_G1(OPC, TIN, TOUT, MODE, OUTER, SR, ...) \
  KernelEntry{KernelKey{OPC, TIN, TOUT, 16, (MODE) + 4, OUTER, SR}, \
              reinterpret_cast<const void*>(&dev::gen_kernel_t<__VA_ARGS__, MODE, OUTER, (SR != 0)>)}
// general lean kernels: mode key 4 (copy), 5 (tile ewise), 6 (stream), 7 (store with reduce-add)
#define ACP_GEN(OPC, TIN, TOUT, MODE, ...) \
  ACP_G1(OPC, TIN, TOUT, MODE, 1, 0, __VA_ARGS__), ACP_G1(OPC, TIN, TOUT, MODE, 2, 0, __VA_ARGS__), \
      ACP_G1(OPC, TIN, TOUT, MODE, 4, 0, __VA_ARGS__), ACP_G1(OPC, TIN, TOUT, MODE, 8, 0, __VA_ARGS__)
#define ACP_GEN_ROW(OPC, ...) \
  ACP_GEN(OPC, kF32, kF32, 2, __VA_ARGS__), ACP_G1(OPC, kF32, kF32, 2, 1, 1, __VA_ARGS__), \
      ACP_G1(OPC, kF32, kF32, 2, 2, 1, __VA_ARGS__), ACP_G1(OPC, kF32, kF32, 2, 4, 1, __VA_ARGS__), \
      ACP_G1(OPC, kF32, kF32, 2, 8, 1, __VA_ARGS__)
// two-tensor stream ops (mode key 6): variant 1 both operands on the ring,
// variant 2 the second one staged synchronously
#define ACP_GB1(OPC, T, OUTER, V, ...)                                                 \
  KernelEntry{KernelKey{OPC, T, T, 16, 6, OUTER, 0, V},                              \
              reinterpret_cast<const void*>(&dev::gen_kernel_t<__VA_ARGS__, 2, OUTER, false, (V == 2)>)}
#define ACP_GEN_BIN(OPC, T, ...)                                                                       \
  ACP_GB1(OPC, T, 1, 1, __VA_ARGS__), ACP_GB1(OPC, T, 2, 1, __VA_ARGS__), ACP_GB1(OPC, T, 4, 1, __VA_ARGS__), \
      ACP_GB1(OPC, T, 8, 1, __VA_ARGS__), ACP_GB1(OPC, T, 1, 2, __VA_ARGS__), ACP_GB1(OPC, T, 2, 2, __VA_ARGS__), \
      ACP_GB1(OPC, T, 4, 2, __VA_ARGS__), ACP_GB1(OPC, T, 8, 2, __VA_ARGS__)
// store with reduce-add summing batch dims in registers (mode key 7, variant 1)
#define ACP_GG1(OPC, T, OUTER, ...)                       \
  KernelEntry{KernelKey{OPC, T, T, 16, 7, OUTER, 0, 1}, \
              reinterpret_cast<const void*>(&dev::gen_kernel_t<__VA_ARGS__, 3, OUTER, false, 0, true>)}
#define ACP_GEN_GROUP(OPC, T, ...) \
  ACP_GG1(OPC, T, 1, __VA_ARGS__), ACP_GG1(OPC, T, 2, __VA_ARGS__), ACP_GG1(OPC, T, 4, __VA_ARGS__), ACP_GG1(OPC, T, 8, __VA_ARGS__)
#define ACP_LIN_ROW(OPC, ...)                                                                              \
  ACP_LIN(OPC, kF32, kF32, __VA_ARGS__), ACP_L(OPC, kF32, kF32, 1, 1, __VA_ARGS__),                          \
      ACP_L(OPC, kF32, kF32, 2, 1, __VA_ARGS__), ACP_L(OPC, kF32, kF32, 4, 1, __VA_ARGS__), \
      ACP_L(OPC, kF32, kF32, 8, 1, __VA_ARGS__)
// two streamed tensors on a linear grid, both on the direct-to-LDS ring (mode key 3, variant 1)
#define ACP_LB1(OPC, T, OUTER, ...)                          \
  KernelEntry{KernelKey{OPC, T, T, 16, 3, OUTER, 0, 1}, \
              reinterpret_cast<const void*>(&dev::stream_lin_kernel_t<__VA_ARGS__, OUTER, false>)}
#define ACP_LIN_BIN(OPC, T, ...) \
  ACP_LB1(OPC, T, 1, __VA_ARGS__), ACP_LB1(OPC, T, 2, __VA_ARGS__), ACP_LB1(OPC, T, 4, __VA_ARGS__), ACP_LB1(OPC, T, 8, __VA_ARGS__)
// tile ewise on a linear tile grid (mode key 9): the linear kernel with the output staged in LDS
#define ACP_LT1(OPC, TIN, TOUT, OUTER, ...)                \
  KernelEntry{KernelKey{OPC, TIN, TOUT, 16, 9, OUTER, 0}, \
              reinterpret_cast<const void*>(&dev::stream_lin_kernel_t<__VA_ARGS__, OUTER, false, true>)}
#define ACP_LIN_TILE(OPC, TIN, TOUT, ...)                                                \
  ACP_LT1(OPC, TIN, TOUT, 1, __VA_ARGS__), ACP_LT1(OPC, TIN, TOUT, 2, __VA_ARGS__),       \
      ACP_LT1(OPC, TIN, TOUT, 4, __VA_ARGS__), ACP_LT1(OPC, TIN, TOUT, 8, __VA_ARGS__)
// row reduction on a linear stage grid, wave-local (mode key 10)
#define ACP_LR1(T, OUTER)                                           \
  KernelEntry{KernelKey{kOpAdd, T, kF32, 16, 10, OUTER, 0},         \
              reinterpret_cast<const void*>(&dev::rows_lin_kernel_t<dev::ReduceRowsOp<T>, OUTER>)}
#define ACP_LIN_ROWS(T) ACP_LR1(T, 1), ACP_LR1(T, 2), ACP_LR1(T, 4), ACP_LR1(T, 8)
#define ACP_BOTH(OPC, TIN, TOUT, MODE, ...) ACP_K(OPC, TIN, TOUT, 16, MODE, __VA_ARGS__), ACP_K(OPC, TIN, TOUT, 4, MODE, __VA_ARGS__)

template <size_t N>
const void* find_entry(const KernelEntry (&table)[N], const KernelKey& k) {
  for (const KernelEntry& e : table)
    if (e.key.op == k.op && e.key.tin == k.tin && e.key.tout == k.tout && e.key.vec_bytes == k.vec_bytes &&
        e.key.mode == k.mode && e.key.outer == k.outer && e.key.srow == k.srow && e.key.variant == k.variant)
      return e.fn;
  return nullptr;
}

}  // namespace acp
