// Instantiations of the persistent GEMM for fp8 operands (K-major, e4m3 or e5m2 in either operand), activation-backward epilogue, varlen-M.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_FP8, true, 1>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
