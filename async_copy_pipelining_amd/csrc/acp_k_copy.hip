// Engine instantiations: tile copy (raw bytes moved as 32-bit words).
#include "acp_engine_impl.hpp"

namespace acp {
using namespace dev;
namespace {
const KernelEntry kTable[] = {
    ACP_BOTH(kOpCopy, kU32, kU32, 0, Op<kOpCopy, kU32, kU32>),
    // general lean kernel
    ACP_GEN(kOpCopy, kU32, kU32, 0, Op<kOpCopy, kU32, kU32>),
};
}  // namespace
const void* lookup_copy(const KernelKey& k) { return find_entry(kTable, k); }
}  // namespace acp
