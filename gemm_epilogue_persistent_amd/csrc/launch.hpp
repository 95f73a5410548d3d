// Kernel entry points and the launcher table shared by the instantiation units.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm_kernel.hpp"

namespace gep {


// Workgroups per CU the kernel is built for: 256x256 tiles keep 256 accumulators per lane
// over a CU's waves (one workgroup per CU); 128x128 tiles fit two per CU.
template <int BM>
constexpr int wg_per_cu() { return BM == 256 ? 1 : 2; }
// Waves per workgroup. K-major x K-major 256x256 kernels (16-bit: dense, varlen-M, gathered
// rows, dact; fp8: all) run 8 waves (two per SIMD, 128x64 accumulators each, 16x16 MFMA
// blocks) with global -> LDS transfers; on 32x32 blocks 8 waves had measured +2% on the 8192^3
// GEMM, +4% on the 4096^3 GEMM with C and GELU, +0.5-2.5% on varlen-M against 4 (the epilogue
// halves; the store drain moves into the next tile's first wait); fp8 on 16x16x128 blocks
// +3.7% on 8192^3 against 4 waves on 32x32x64 (on 32x32x64, 8 waves had been 4% slower). Every
// other kernel runs 4. With 8 waves and transfers the M/N-major kernels ran at half speed
// (batched 2048x2048x4096x16 550 vs 1125 TFLOP/s, varlen-K 544 vs 1108): their transposed
// fragment reads (two ds_read_b64_tr_b16 per fragment) grow to 1.5x as many per CU with
// 128x64 wave tiles and bound the loop.
template <int BM, int OP, bool AK, bool BK>
constexpr int waves() { return (BM == 256 && AK && BK) ? 8 : 4; }

// VM: 0 dense batched, 1 varlen-M, 2 varlen-K. DA: the activation-backward epilogue (its own
// instantiations, so that the forward kernels carry none of its code or registers). GA: A read
// through a_idx: its rows (varlen-M, K-major A) or its k-rows (varlen-K, M-major A).
template <int BM, int OP, int FA, int FB, bool AK, bool BK, int VM, bool DA, bool GA>
__global__ __launch_bounds__((waves<BM, OP, AK, BK>() * 64), (wg_per_cu<BM>())) void gemm_persistent_kernel(
    const KParams p) {
  GemmKernel<BM, BM, OP, FA, FB, AK, BK, VM, waves<BM, OP, AK, BK>(), DA, GA>::run(p);
}

template <int BM, int OP, int FA, int FB, bool AK, bool BK, int VM, bool DA, bool GA>
hipError_t launch_one(const KParams& p, hipStream_t s) {
  hipLaunchKernelGGL((gemm_persistent_kernel<BM, OP, FA, FB, AK, BK, VM, DA, GA>), dim3(p.P),
                     dim3(waves<BM, OP, AK, BK>() * 64), 0, s, p);
  return hipGetLastError();
}

// Every kernel of one op family, epilogue kind and varlen mode (a unit instantiates one);
// returns hipErrorInvalidValue for a key the family does not hold.
template <int OP, bool DA, int VM>
hipError_t launch_family(const KernelKey& k, const KParams& p, hipStream_t s);

template <int BM, int OP, int VM, bool DA>
hipError_t by_layout(const KernelKey& k, const KParams& p, hipStream_t s) {
  if constexpr (OP == OP_FP8) {
    // K-major only; e4m3 / e5m2 in either operand
    if (!k.a_kmajor || !k.b_kmajor || k.gather) return hipErrorInvalidValue;
    if (k.fmt_a == 0 && k.fmt_b == 0) return launch_one<BM, OP, 0, 0, true, true, VM, DA, false>(p, s);
    if (k.fmt_a == 0 && k.fmt_b == 1) return launch_one<BM, OP, 0, 1, true, true, VM, DA, false>(p, s);
    if (k.fmt_a == 1 && k.fmt_b == 0) return launch_one<BM, OP, 1, 0, true, true, VM, DA, false>(p, s);
    return launch_one<BM, OP, 1, 1, true, true, VM, DA, false>(p, s);
  } else {
    if (k.gather) {
      if constexpr (VM == 1 && !DA) {  // gathered rows of a K-major A
        if (!k.a_kmajor) return hipErrorInvalidValue;
        if (k.b_kmajor) return launch_one<BM, OP, 0, 0, true, true, VM, DA, true>(p, s);
        return launch_one<BM, OP, 0, 0, true, false, VM, DA, true>(p, s);
      }
      if constexpr (VM == 2 && !DA) {  // gathered k-rows of an M-major A
        if (k.a_kmajor) return hipErrorInvalidValue;
        if (k.b_kmajor) return launch_one<BM, OP, 0, 0, false, true, VM, DA, true>(p, s);
        return launch_one<BM, OP, 0, 0, false, false, VM, DA, true>(p, s);
      }
      return hipErrorInvalidValue;
    }
    if (k.a_kmajor && k.b_kmajor) return launch_one<BM, OP, 0, 0, true, true, VM, DA, false>(p, s);
    if (k.a_kmajor && !k.b_kmajor) return launch_one<BM, OP, 0, 0, true, false, VM, DA, false>(p, s);
    if (!k.a_kmajor && k.b_kmajor) return launch_one<BM, OP, 0, 0, false, true, VM, DA, false>(p, s);
    return launch_one<BM, OP, 0, 0, false, false, VM, DA, false>(p, s);
  }
}

template <int OP, bool DA, int VM>
hipError_t launch_family(const KernelKey& k, const KParams& p, hipStream_t s) {
  if (k.op != OP || (k.dact != 0) != DA || k.varlen != VM) return hipErrorInvalidValue;
  if (k.tile == 0) return by_layout<256, OP, VM, DA>(k, p, s);
  return by_layout<128, OP, VM, DA>(k, p, s);
}

#define GEP_DECLARE_FAMILY(OP, DA, VM) \
  extern template hipError_t launch_family<OP, DA, VM>(const KernelKey&, const KParams&, hipStream_t);
#define GEP_DECLARE_OP(OP)           \
  GEP_DECLARE_FAMILY(OP, false, 0)   \
  GEP_DECLARE_FAMILY(OP, false, 1)   \
  GEP_DECLARE_FAMILY(OP, false, 2)   \
  GEP_DECLARE_FAMILY(OP, true, 0)    \
  GEP_DECLARE_FAMILY(OP, true, 1)
GEP_DECLARE_OP(OP_F16)
GEP_DECLARE_OP(OP_BF16)
GEP_DECLARE_OP(OP_FP8)
#undef GEP_DECLARE_OP
#undef GEP_DECLARE_FAMILY

}  // namespace gep
