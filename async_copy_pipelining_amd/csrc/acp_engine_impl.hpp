// Engine kernels for gfx950 and their registry: each kernel translation
// unit includes this header and lists the instantiations it builds.
#pragma once

#include "acp_dev_engine.hpp"
#include "acp_dev_gen.hpp"
#include "acp_dev_lin.hpp"

namespace acp {

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
