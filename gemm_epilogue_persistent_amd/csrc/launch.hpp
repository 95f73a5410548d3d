// Kernel entry points and the launcher table shared by the instantiation units.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace gep {


// Workgroups per CU the kernel is built for: 256x256 tiles keep 256 accumulators per lane
// over a CU's waves (one workgroup per CU); 128x128 tiles fit two per CU.
template <int BM>
constexpr int wg_per_cu() { return BM == 256 ? 1 : 2; }
// Waves per workgroup. The kernel also runs with 8 waves (two per SIMD, 128x64 accumulators
// each); measured on the 8192^3 bf16, varlen-M and batched M/N-major workloads, 4 waves
// were as fast or faster (8 waves lost ~30% on varlen-M), so every kernel uses 4.
template <int BM, int OP>
constexpr int waves() { return 4; }

template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL>
__global__ __launch_bounds__((waves<BM, OP>() * 64), (wg_per_cu<BM>())) void gemm_persistent_kernel(const KParams p) {
  GemmKernel<BM, BM, OP, FA, FB, AK, BK, VL, waves<BM, OP>()>::run(p);
}

template <int BM, int OP, int FA, int FB, bool AK, bool BK, bool VL>
hipError_t launch_one(const KParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_persistent_kernel<BM, OP, FA, FB, AK, BK, VL>), dim3(p.P), dim3(waves<BM, OP>() * 64), 0,
                     s, p);
  return hipGetLastError();
}

// One unit per op family; each returns hipErrorInvalidValue for a key it does not hold.
hipError_t launch_f16(const KernelKey& k, const KParams& p, hipStream_t s);
hipError_t launch_bf16(const KernelKey& k, const KParams& p, hipStream_t s);
hipError_t launch_fp8(const KernelKey& k, const KParams& p, hipStream_t s);

}  // namespace gep
