// Instantiations of the persistent GEMM for bf16 operands (every major combination), activation-backward epilogue, dense batched.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_BF16, true, 0>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
