// Instantiations of the persistent GEMM for fp8 operands (K-major, e4m3 or e5m2 in either operand), forward epilogue, dense batched.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_FP8, false, 0>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
