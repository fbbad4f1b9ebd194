// Engine instantiations: streamed ops with float32 staged input.
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_BOTH(kOpZero, kF32, kF32, 2, Op<kOpZero, kF32, kF32>),
    ACP_BOTH(kOpSqrt, kF32, kF32, 2, Op<kOpSqrt, kF32, kF32>),
    ACP_BOTH(kOpSqrt, kF32, kF16, 2, Op<kOpSqrt, kF32, kF16>),
    ACP_BOTH(kOpExp, kF32, kF32, 2, Op<kOpExp, kF32, kF32>),
    ACP_BOTH(kOpExp, kF32, kF16, 2, Op<kOpExp, kF32, kF16>),
    ACP_BOTH(kOpAdd, kF32, kF32, 2, RowOp<kOpAdd>),
    ACP_BOTH(kOpMul, kF32, kF32, 2, RowOp<kOpMul>),
    ACP_BOTH(kOpFma, kF32, kF32, 2, RowOp<kOpFma>),
    // linear-grid fast path
    ACP_LIN(kOpZero, kF32, kF32, Op<kOpZero, kF32, kF32>),
    ACP_LIN(kOpSqrt, kF32, kF32, Op<kOpSqrt, kF32, kF32>),
    ACP_LIN(kOpSqrt, kF32, kF16, Op<kOpSqrt, kF32, kF16>),
    ACP_LIN(kOpExp, kF32, kF32, Op<kOpExp, kF32, kF32>),
    ACP_LIN(kOpExp, kF32, kF16, Op<kOpExp, kF32, kF16>),
    ACP_LIN_ROW(kOpAdd, RowOp<kOpAdd>),
    ACP_LIN_ROW(kOpMul, RowOp<kOpMul>),
    ACP_LIN_ROW(kOpFma, RowOp<kOpFma>),
    // general lean kernel
    ACP_GEN(kOpZero, kF32, kF32, 2, Op<kOpZero, kF32, kF32>),
    ACP_GEN(kOpSqrt, kF32, kF32, 2, Op<kOpSqrt, kF32, kF32>),
    ACP_GEN(kOpSqrt, kF32, kF16, 2, Op<kOpSqrt, kF32, kF16>),
    ACP_GEN(kOpExp, kF32, kF32, 2, Op<kOpExp, kF32, kF32>),
    ACP_GEN(kOpExp, kF32, kF16, 2, Op<kOpExp, kF32, kF16>),
    ACP_GEN_ROW(kOpAdd, RowOp<kOpAdd>),
    ACP_GEN_ROW(kOpMul, RowOp<kOpMul>),
    ACP_GEN_ROW(kOpFma, RowOp<kOpFma>),
    // two streamed tensors
    ACP_GEN_BIN(kOpAdd, kF32, Op<kOpAdd, kF32, kF32>),
    ACP_GEN_BIN(kOpMul, kF32, Op<kOpMul, kF32, kF32>),
    ACP_LIN_BIN(kOpAdd, kF32, Op<kOpAdd, kF32, kF32>),
    ACP_LIN_BIN(kOpMul, kF32, Op<kOpMul, kF32, kF32>),
    // row reduction
    ACP_GEN(kOpAdd, kF32, kF32, 4, ReduceRowsOp<kF32>),
    ACP_LIN_ROWS(kF32),
};
}  // namespace
const void* lookup_stream_f32(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
