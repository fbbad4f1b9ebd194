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

#include <cstddef>

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

// The argument block (over 1 KiB) is read through the scalar cache, and a
// kernel's set-up reads it in dependent rounds (a field, a branch on it, the
// next field), each of which can miss on a new 64-byte line and wait for
// L2 or HBM.  Reading one word of every line the kernel uses first, in one
// batch behind a single wait, leaves the later reads to hit the scalar
// cache.  At most 15 scalar loads can be outstanding, so a mask of up to 15
// lines costs one round trip.
constexpr int kArgLines = static_cast<int>((sizeof(EngineArgs) + 63) / 64);
constexpr uint32_t arg_lines(size_t lo, size_t hi) {  // lines of bytes [lo, hi)
  uint32_t m = 0;
  for (size_t l = lo / 64; l * 64 < hi; ++l) m |= 1u << l;
  return m;
}
constexpr uint32_t kAllArgLines = arg_lines(0, sizeof(EngineArgs));
// the linear kernels: pointers, stage box, the image axes and everything after
constexpr uint32_t kLinArgLines = arg_lines(0, offsetof(EngineArgs, xstep)) |
                                  arg_lines(offsetof(EngineArgs, sbox), offsetof(EngineArgs, nst)) |
                                  arg_lines(offsetof(EngineArgs, ax_count), sizeof(EngineArgs));
static_assert(__builtin_popcount(kLinArgLines) <= 15, "one batch of scalar loads");

// More than 15 lines take several batches, each a trip to memory.  Then one
// vector load, lane k reading a word of line k, goes out first and brings
// every line into L2 while the first batch is in flight, so the later
// batches hit L2.  The returned word feeds `karg_warm_done`, which the
// kernel places before its first ring load: the wait for the vector load
// falls there, and the ring's vmcnt counts start from zero.
template <uint32_t LINES = kAllArgLines>
__device__ __forceinline__ uint32_t prefetch_kargs() {
  uint32_t warm = 0;
  if constexpr (__builtin_popcount(LINES) > 15) {
    typedef const uint32_t __attribute__((address_space(1))) GWord;
    GWord* g = (GWord*)(__builtin_amdgcn_kernarg_segment_ptr());
    const uint32_t lane = threadIdx.x & 63u;
    if (lane < static_cast<uint32_t>(kArgLines) && ((LINES >> lane) & 1u)) warm = g[lane * 16u];
  }
  typedef const uint32_t __attribute__((address_space(4))) CWord;
  CWord* w = (CWord*)(__builtin_amdgcn_kernarg_segment_ptr());
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kArgLines; ++k)
    if ((LINES >> k) & 1u) x ^= w[k * 16];
  asm volatile("" ::"s"(x));
  return warm;
}

__device__ __forceinline__ void karg_warm_done(uint32_t warm) { asm volatile("" ::"v"(warm) : "memory"); }

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

// Compile-time form of the same wait.
template <int K>
__device__ __forceinline__ void wait_vmcnt_c() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K < 63 ? K : 63) : "memory");
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
//
// A policy provides load(j, slot), pre_wait(i, slot, k) (called just before
// trip i's wait with the count k it allows: the place for scalar loads whose
// latency then hides behind the wait) and consume(i, slot).

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
    const int k = allowed(i, n, s, d, st);
    p.pre_wait(i, cur, k);
    wait_vmcnt(k);
    p.consume(i, cur);
    cur = (cur + 1 == s) ? 0 : cur + 1;
    ld = (ld + 1 == s) ? 0 : ld + 1;
  }
  for (; i < n; ++i) {
    const int k = allowed(i, n, s, d, st);
    p.pre_wait(i, cur, k);
    wait_vmcnt(k);
    p.consume(i, cur);
    cur = (cur + 1 == s) ? 0 : cur + 1;
  }
}

// The ring for per-trip counts D and ST and a slot count S known at compile
// time: every wait is an immediate.  Trip i's allowed count is
// ahead * D + behind * ST (see `allowed`).  In the warm-up (the first S-1
// main-loop trips) ahead is S-1 and behind is i; in the steady state both
// are S-1; in the epilogue ahead is the number of trips left after i (S-2
// down to 0) and behind is S-1 once i >= S-1.  A trip of a very short ring
// (i < S-1 in the epilogue) waits as if no store had been issued since its
// load: a smaller count, hence a stronger wait, and still exact for pre_wait.
template <int D, int ST, int S, class P>
__device__ __forceinline__ void run_ring_s(P& p, int n) {
  static_assert(S >= 1 && S <= 4, "slot count");
  const int nmain = n - (S - 1) > 0 ? n - (S - 1) : 0;
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < n) p.load(j, j);
  int i = 0;
  // warm-up: load trip i + S - 1 into slot i + S - 1 (mod S), consume slot i
  const int warm = nmain < S - 1 ? nmain : S - 1;
  for (; i < warm; ++i) {
    p.load(i + S - 1, (i + S - 1) % S);
    p.pre_wait(i, i, allowed(i, n, S, D, ST));
    if (i == 0) wait_vmcnt_c<(S - 1) * D>();
    else if (i == 1) wait_vmcnt_c<(S - 1) * D + ST>();
    else wait_vmcnt_c<(S - 1) * D + 2 * ST>();
    p.consume(i, i);
  }
  int cur = warm % S, ld = (warm + S - 1) % S;
  for (; i < nmain; ++i) {
    p.load(i + S - 1, ld);
    p.pre_wait(i, cur, (S - 1) * (D + ST));
    wait_vmcnt_c<(S - 1) * (D + ST)>();
    p.consume(i, cur);
    cur = (cur + 1 == S) ? 0 : cur + 1;
    ld = (ld + 1 == S) ? 0 : ld + 1;
  }
  // epilogue: no loads; `left` trips follow trip i
  for (; i < n; ++i) {
    const int left = n - 1 - i;
    p.pre_wait(i, cur, allowed(i, n, S, D, ST));
    if (i >= S - 1) {
      if (left == 0) wait_vmcnt_c<(S - 1) * ST>();
      else if (left == 1) wait_vmcnt_c<D + (S - 1) * ST>();
      else wait_vmcnt_c<2 * D + (S - 1) * ST>();
    } else {
      if (left == 0) wait_vmcnt_c<0>();
      else if (left == 1) wait_vmcnt_c<D>();
      else wait_vmcnt_c<2 * D>();
    }
    p.consume(i, cur);
    cur = (cur + 1 == S) ? 0 : cur + 1;
  }
}

// The same ring for per-trip counts D and ST known at compile time and a
// slot count s (1..4) chosen at launch: one compile-time ring per slot count.
template <int D, int ST, class P>
__device__ __forceinline__ void run_ring_fixed(P& p, int n, int s) {
  if (s == 4) run_ring_s<D, ST, 4>(p, n);
  else if (s == 3) run_ring_s<D, ST, 3>(p, n);
  else if (s == 2) run_ring_s<D, ST, 2>(p, n);
  else run_ring_s<D, ST, 1>(p, n);
}

}  // namespace dev
}  // namespace acp
