// Engine instantiations: elementwise ops on LDS-resident tiles, general lean
// kernel (16-byte rounds, rounds per thread fixed at compile time).
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_GEN(kOpZero, kF32, kF32, 1, Op<kOpZero, kF32, kF32>),
    ACP_GEN(kOpZero, kF16, kF16, 1, Op<kOpZero, kF16, kF16>),
    ACP_GEN(kOpSqrt, kF32, kF32, 1, Op<kOpSqrt, kF32, kF32>),
    ACP_GEN(kOpSqrt, kF16, kF32, 1, Op<kOpSqrt, kF16, kF32>),
    ACP_GEN(kOpSqrt, kF32, kF16, 1, Op<kOpSqrt, kF32, kF16>),
    ACP_GEN(kOpSqrt, kF16, kF16, 1, Op<kOpSqrt, kF16, kF16>),
    ACP_GEN(kOpExp, kF32, kF32, 1, Op<kOpExp, kF32, kF32>),
    ACP_GEN(kOpExp, kF16, kF32, 1, Op<kOpExp, kF16, kF32>),
    ACP_GEN(kOpExp, kF32, kF16, 1, Op<kOpExp, kF32, kF16>),
    ACP_GEN(kOpExp, kF16, kF16, 1, Op<kOpExp, kF16, kF16>),
    ACP_GEN(kOpAdd, kF32, kF32, 1, Op<kOpAdd, kF32, kF32>),
    ACP_GEN(kOpAdd, kF16, kF16, 1, Op<kOpAdd, kF16, kF16>),
    ACP_GEN(kOpMul, kF32, kF32, 1, Op<kOpMul, kF32, kF32>),
    ACP_GEN(kOpMul, kF16, kF16, 1, Op<kOpMul, kF16, kF16>),
    ACP_GEN(kOpFma, kF32, kF32, 1, Op<kOpFma, kF32, kF32>),
    ACP_GEN(kOpFma, kF16, kF16, 1, Op<kOpFma, kF16, kF16>),
};
}  // namespace
const void* lookup_tile_gen(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
