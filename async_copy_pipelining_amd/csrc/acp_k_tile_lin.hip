// Engine instantiations: elementwise ops on LDS-resident tiles of a linear
// tile grid (the linear kernel with the output staged in LDS; a ring trip
// stages 1, 2 or 4 consecutive tiles as one stage).
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_LIN_TILE(kOpSqrt, kF32, kF32, Op<kOpSqrt, kF32, kF32>),
    ACP_LIN_TILE(kOpSqrt, kF16, kF32, Op<kOpSqrt, kF16, kF32>),
    ACP_LIN_TILE(kOpSqrt, kF32, kF16, Op<kOpSqrt, kF32, kF16>),
    ACP_LIN_TILE(kOpSqrt, kF16, kF16, Op<kOpSqrt, kF16, kF16>),
    ACP_LIN_TILE(kOpExp, kF32, kF32, Op<kOpExp, kF32, kF32>),
    ACP_LIN_TILE(kOpExp, kF16, kF32, Op<kOpExp, kF16, kF32>),
    ACP_LIN_TILE(kOpExp, kF32, kF16, Op<kOpExp, kF32, kF16>),
    ACP_LIN_TILE(kOpExp, kF16, kF16, Op<kOpExp, kF16, kF16>),
    ACP_LIN_TILE(kOpAdd, kF32, kF32, Op<kOpAdd, kF32, kF32>),
    ACP_LIN_TILE(kOpAdd, kF16, kF16, Op<kOpAdd, kF16, kF16>),
    ACP_LIN_TILE(kOpMul, kF32, kF32, Op<kOpMul, kF32, kF32>),
    ACP_LIN_TILE(kOpMul, kF16, kF16, Op<kOpMul, kF16, kF16>),
    ACP_LIN_TILE(kOpFma, kF32, kF32, Op<kOpFma, kF32, kF32>),
    ACP_LIN_TILE(kOpFma, kF16, kF16, Op<kOpFma, kF16, kF16>),
};
}  // namespace
const void* lookup_tile_lin(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
