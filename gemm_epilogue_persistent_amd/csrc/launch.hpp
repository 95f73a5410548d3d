// Kernel entry points and the launcher table shared by the instantiation units.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace gep {


// Workgroups per CU the kernel is built for: 256x256 tiles keep 256 accumulators per lane
// over a CU's waves (one workgroup per CU); 128x128 tiles fit two per CU.
template <int BM>
constexpr int wg_per_cu() { return BM == 256 ? 1 : 2; }
// Waves per workgroup. 16-bit K-major x K-major 256x256 kernels (dense and varlen-M) run 8
// waves (two per SIMD, 128x64 accumulators each) with global -> LDS transfers: measured +2%
// on the 8192^3 GEMM, +4% on the 4096^3 GEMM with C and GELU, +0.5-2.5% on varlen-M (its
// epilogue halves; the store drain moves into the next tile's first wait). Every other kernel
// runs 4: transfers slowed the M/N-major one by ~30%.
template <int BM, int OP, bool AK, bool BK, bool VL>
constexpr int waves() { return (BM == 256 && OP != OP_FP8 && AK && BK) ? 8 : 4; }

// DA: the activation-backward epilogue (its own instantiations, so that the forward kernels
// carry none of its code or registers).
template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL, bool DA>
__global__ __launch_bounds__((waves<BM, OP, AK, BK, VL>() * 64), (wg_per_cu<BM>())) void gemm_persistent_kernel(
    const KParams p) {
  GemmKernel<BM, BM, OP, FA, FB, AK, BK, VL, waves<BM, OP, AK, BK, VL>(), DA>::run(p);
}

template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL, bool DA>
hipError_t launch_one(const KParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_persistent_kernel<BM, OP, FA, FB, AK, BK, VL, DA>), dim3(p.P),
                     dim3(waves<BM, OP, AK, BK, VL>() * 64), 0, s, p);
  return hipGetLastError();
}

// Every kernel of one op family with one epilogue kind (a unit instantiates one pair);
// returns hipErrorInvalidValue for a key the family does not hold.
template <int OP, bool DA>
hipError_t launch_family(const KernelKey& k, const KParams& p, hipStream_t s);

template <int BM, int OP, bool VL, bool DA>
hipError_t by_layout(const KernelKey& k, const KParams& p, hipStream_t s) {
  if constexpr (OP == OP_FP8) {
    // K-major only; e4m3 / e5m2 in either operand
    if (!k.a_kmajor || !k.b_kmajor) return hipErrorInvalidValue;
    if (k.fmt_a == 0 && k.fmt_b == 0) return launch_one<BM, OP, 0, 0, true, true, VL, DA>(p, s);
    if (k.fmt_a == 0 && k.fmt_b == 1) return launch_one<BM, OP, 0, 1, true, true, VL, DA>(p, s);
    if (k.fmt_a == 1 && k.fmt_b == 0) return launch_one<BM, OP, 1, 0, true, true, VL, DA>(p, s);
    return launch_one<BM, OP, 1, 1, true, true, VL, DA>(p, s);
  } else {
    if (k.a_kmajor && k.b_kmajor) return launch_one<BM, OP, 0, 0, true, true, VL, DA>(p, s);
    if (k.a_kmajor && !k.b_kmajor) return launch_one<BM, OP, 0, 0, true, false, VL, DA>(p, s);
    if (!k.a_kmajor && k.b_kmajor) return launch_one<BM, OP, 0, 0, false, true, VL, DA>(p, s);
    return launch_one<BM, OP, 0, 0, false, false, VL, DA>(p, s);
  }
}

template <int OP, bool DA>
hipError_t launch_family(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (k.op != OP || (k.dact != 0) != DA) return hipErrorInvalidValue;
  if (k.tile == 0) return k.varlen ? by_layout<256, OP, true, DA>(k, p, s) : by_layout<256, OP, false, DA>(k, p, s);
  return k.varlen ? by_layout<128, OP, true, DA>(k, p, s) : by_layout<128, OP, false, DA>(k, p, s);
}

#define GEP_DECLARE_FAMILY(OP, DA) \
  extern template hipError_t launch_family<OP, DA>(const KernelKey&, const KParams&, hipStream_t);
GEP_DECLARE_FAMILY(OP_F16, false)
GEP_DECLARE_FAMILY(OP_F16, true)
GEP_DECLARE_FAMILY(OP_BF16, false)
GEP_DECLARE_FAMILY(OP_BF16, true)
GEP_DECLARE_FAMILY(OP_FP8, false)
GEP_DECLARE_FAMILY(OP_FP8, true)
#undef GEP_DECLARE_FAMILY

}  // namespace gep
