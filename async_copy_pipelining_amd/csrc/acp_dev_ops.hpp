// Elementwise and reduction ops of the engine kernels.
#pragma once

#include "acp_dev_base.hpp"

namespace acp {
namespace dev {

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

}  // namespace dev
}  // namespace acp
