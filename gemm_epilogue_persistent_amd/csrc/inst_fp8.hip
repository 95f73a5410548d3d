// Instantiations of the persistent GEMM for fp8 operands (K-major only; e4m3/e5m2 mixes).
#include "launch.hpp"

namespace gep {

template <int BM, bool VL>
static hipError_t by_format(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (!k.a_kmajor || !k.b_kmajor) return hipErrorInvalidValue;
  if (k.fmt_a == 0 && k.fmt_b == 0) return launch_one<BM, OP_FP8, 0, 0, true, true, VL>(p, s);
  if (k.fmt_a == 0 && k.fmt_b == 1) return launch_one<BM, OP_FP8, 0, 1, true, true, VL>(p, s);
  if (k.fmt_a == 1 && k.fmt_b == 0) return launch_one<BM, OP_FP8, 1, 0, true, true, VL>(p, s);
  return launch_one<BM, OP_FP8, 1, 1, true, true, VL>(p, s);
}

hipError_t launch_fp8(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (k.op != OP_FP8) return hipErrorInvalidValue;
  if (k.tile == 0) return k.varlen ? by_format<256, true>(k, p, s) : by_format<256, false>(k, p, s);
  return k.varlen ? by_format<128, true>(k, p, s) : by_format<128, false>(k, p, s);
}

}  // namespace gep
