// Engine instantiations: tile copy (raw bytes moved as 32-bit words; on a
// linear tile grid through the linear kernel) and the store with reduce-add.
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_BOTH(kOpCopy, kU32, kU32, 0, Op<kOpCopy, kU32, kU32>),
    // linear tile grid (one tile per stage, contiguous row-major grid)
    ACP_LIN(kOpCopy, kU32, kU32, Op<kOpCopy, kU32, kU32>),
    // general lean kernel
    ACP_GEN(kOpCopy, kU32, kU32, 0, Op<kOpCopy, kU32, kU32>),
    // store with reduce-add
    ACP_GEN(kOpAdd, kU32, kU32, 3, ReduceOp<kU32>),
    ACP_GEN(kOpAdd, kF32, kF32, 3, ReduceOp<kF32>),
    ACP_GEN(kOpAdd, kF16, kF16, 3, ReduceOp<kF16>),
    ACP_GEN_GROUP(kOpAdd, kU32, ReduceOp<kU32>),
    ACP_GEN_GROUP(kOpAdd, kF32, ReduceOp<kF32>),
    ACP_GEN_GROUP(kOpAdd, kF16, ReduceOp<kF16>),
};
}  // namespace
const void* lookup_copy(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
