// Instantiations of the persistent GEMM for fp8 operands (K-major; e4m3 / e5m2 mixes), activation-backward epilogue.
#include "launch.hpp"

namespace gep {
template hipError_t launch_family<OP_FP8, true>(const KernelKey&, const KParams&, hipStream_t);
}  // namespace gep
