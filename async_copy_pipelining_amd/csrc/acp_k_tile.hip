// Engine instantiations: elementwise ops on LDS-resident tiles (output staged in LDS).
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_BOTH(kOpZero, kF32, kF32, 1, Op<kOpZero, kF32, kF32>),
    ACP_BOTH(kOpZero, kF16, kF16, 1, Op<kOpZero, kF16, kF16>),
    ACP_BOTH(kOpSqrt, kF32, kF32, 1, Op<kOpSqrt, kF32, kF32>),
    ACP_BOTH(kOpSqrt, kF16, kF32, 1, Op<kOpSqrt, kF16, kF32>),
    ACP_BOTH(kOpSqrt, kF32, kF16, 1, Op<kOpSqrt, kF32, kF16>),
    ACP_BOTH(kOpSqrt, kF16, kF16, 1, Op<kOpSqrt, kF16, kF16>),
    ACP_BOTH(kOpExp, kF32, kF32, 1, Op<kOpExp, kF32, kF32>),
    ACP_BOTH(kOpExp, kF16, kF32, 1, Op<kOpExp, kF16, kF32>),
    ACP_BOTH(kOpExp, kF32, kF16, 1, Op<kOpExp, kF32, kF16>),
    ACP_BOTH(kOpExp, kF16, kF16, 1, Op<kOpExp, kF16, kF16>),
    ACP_BOTH(kOpAdd, kF32, kF32, 1, Op<kOpAdd, kF32, kF32>),
    ACP_BOTH(kOpAdd, kF16, kF16, 1, Op<kOpAdd, kF16, kF16>),
    ACP_BOTH(kOpMul, kF32, kF32, 1, Op<kOpMul, kF32, kF32>),
    ACP_BOTH(kOpMul, kF16, kF16, 1, Op<kOpMul, kF16, kF16>),
    ACP_BOTH(kOpFma, kF32, kF32, 1, Op<kOpFma, kF32, kF32>),
    ACP_BOTH(kOpFma, kF16, kF16, 1, Op<kOpFma, kF16, kF16>),
};
}  // namespace
const void* lookup_tile(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
