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

template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL>
__global__ __launch_bounds__((waves<BM, OP, AK, BK, VL>() * 64), (wg_per_cu<BM>())) void gemm_persistent_kernel(
    const KParams p) {
  GemmKernel<BM, BM, OP, FA, FB, AK, BK, VL, waves<BM, OP, AK, BK, VL>()>::run(p);
}

template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL>
hipError_t launch_one(const KParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_persistent_kernel<BM, OP, FA, FB, AK, BK, VL>), dim3(p.P),
                     dim3(waves<BM, OP, AK, BK, VL>() * 64), 0, s, p);
  return hipGetLastError();
}

// One unit per op family; each returns hipErrorInvalidValue for a key it does not hold.
hipError_t launch_f16(const KernelKey& k, const KParams& p, hipStream_t s);
hipError_t launch_bf16(const KernelKey& k, const KParams& p, hipStream_t s);
hipError_t launch_fp8(const KernelKey& k, const KParams& p, hipStream_t s);

}  // namespace gep
