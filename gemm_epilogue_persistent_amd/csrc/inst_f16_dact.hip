// Instantiations of the persistent GEMM for f16 operands (every major combination), activation-backward epilogue, dense batched.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_F16, true, 0>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
