// Instantiations of the persistent GEMM for f16 operands (every major combination), forward epilogue, varlen-K.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_F16, false, 2>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
