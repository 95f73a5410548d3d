// Instantiations of the persistent GEMM for bf16 operands (every major combination).
#include "launch.hpp"

namespace gep {

template <int BM, bool VL>
static hipError_t by_major(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (k.a_kmajor && k.b_kmajor) return launch_one<BM, OP_BF16, 0, 0, true, true, VL>(p, s);
  if (k.a_kmajor && !k.b_kmajor) return launch_one<BM, OP_BF16, 0, 0, true, false, VL>(p, s);
  if (!k.a_kmajor && k.b_kmajor) return launch_one<BM, OP_BF16, 0, 0, false, true, VL>(p, s);
  return launch_one<BM, OP_BF16, 0, 0, false, false, VL>(p, s);
}

hipError_t launch_bf16(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (k.op != OP_BF16) return hipErrorInvalidValue;
  if (k.tile == 0) return k.varlen ? by_major<256, true>(k, p, s) : by_major<256, false>(k, p, s);
  return k.varlen ? by_major<128, true>(k, p, s) : by_major<128, false>(k, p, s);
}

}  // namespace gep
