// Engine instantiations: streamed ops with float16 staged input.
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_BOTH(kOpZero, kF16, kF16, 2, Op<kOpZero, kF16, kF16>),
    ACP_BOTH(kOpSqrt, kF16, kF32, 2, Op<kOpSqrt, kF16, kF32>),
    ACP_BOTH(kOpSqrt, kF16, kF16, 2, Op<kOpSqrt, kF16, kF16>),
    ACP_BOTH(kOpExp, kF16, kF32, 2, Op<kOpExp, kF16, kF32>),
    ACP_BOTH(kOpExp, kF16, kF16, 2, Op<kOpExp, kF16, kF16>),
    // linear-grid fast path
    ACP_LIN(kOpZero, kF16, kF16, Op<kOpZero, kF16, kF16>),
    ACP_LIN(kOpSqrt, kF16, kF32, Op<kOpSqrt, kF16, kF32>),
    ACP_LIN(kOpSqrt, kF16, kF16, Op<kOpSqrt, kF16, kF16>),
    ACP_LIN(kOpExp, kF16, kF32, Op<kOpExp, kF16, kF32>),
    ACP_LIN(kOpExp, kF16, kF16, Op<kOpExp, kF16, kF16>),
    // general lean kernel
    ACP_GEN(kOpZero, kF16, kF16, 2, Op<kOpZero, kF16, kF16>),
    ACP_GEN(kOpSqrt, kF16, kF32, 2, Op<kOpSqrt, kF16, kF32>),
    ACP_GEN(kOpSqrt, kF16, kF16, 2, Op<kOpSqrt, kF16, kF16>),
    ACP_GEN(kOpExp, kF16, kF32, 2, Op<kOpExp, kF16, kF32>),
    ACP_GEN(kOpExp, kF16, kF16, 2, Op<kOpExp, kF16, kF16>),
    // two streamed tensors
    ACP_GEN_BIN(kOpAdd, kF16, Op<kOpAdd, kF16, kF16>),
    ACP_GEN_BIN(kOpMul, kF16, Op<kOpMul, kF16, kF16>),
    ACP_LIN_BIN(kOpAdd, kF16, Op<kOpAdd, kF16, kF16>),
    ACP_LIN_BIN(kOpMul, kF16, Op<kOpMul, kF16, kF16>),
    // row reduction
    ACP_GEN(kOpAdd, kF16, kF32, 4, ReduceRowsOp<kF16>),
    ACP_LIN_ROWS(kF16),
};
}  // namespace
const void* lookup_stream_f16(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
