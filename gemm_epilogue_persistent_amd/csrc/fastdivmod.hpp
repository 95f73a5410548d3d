// Integer division by a runtime-invariant divisor via a multiply-high and a shift
// (quack-kernels 0.1.10 -> 0.2.0 diff, page 6, quack/fast_math.py, FastDivmod).
//
// For 1 <= d < 2^31: p = 31 + ceil(log2 d), multiplier = ceil(2^p / d) (fits in 32 bits),
// shift = p - 32. Then for 0 <= n < 2^31, n / d == umulhi(n, multiplier) >> shift, because
// multiplier * d - 2^p = e lies in [0, d) and n * e < 2^31 * 2^ceil(log2 d) = 2^p, so the
// error term n * e / (d * 2^p) stays below 1/d and never carries the quotient over.
// d == 1 is handled apart (p = 31 would need a negative shift).
// On gfx950 the multiply-high is v_mul_hi_u32 (__umulhi).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define GEP_HD __host__ __device__
#else
#define GEP_HD
#endif

struct FastDiv {
  uint32_t divisor;
  uint32_t multiplier;
  uint32_t shift;
};

GEP_HD static inline uint32_t gep_ceil_log2(uint32_t d) {
  // 31 - count-leading-zeros, plus one unless d is a power of two
  return (uint32_t)(31 - __builtin_clz(d)) + ((d & (d - 1)) != 0 ? 1u : 0u);
}

GEP_HD static inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.divisor = d;
  uint32_t p = 31u + gep_ceil_log2(d);
  f.multiplier = (uint32_t)((((uint64_t)1 << p) + d - 1) / d);
  f.shift = p - 32u;  // wraps for d == 1, where it is not used
  return f;
}

GEP_HD static inline uint32_t fd_div(const FastDiv& f, uint32_t n) {
  if (f.divisor == 1) return n;
#if defined(__HIP_DEVICE_COMPILE__)
  return __umulhi(n, f.multiplier) >> f.shift;
#else
  return (uint32_t)(((uint64_t)n * f.multiplier) >> 32) >> f.shift;
#endif
}

GEP_HD static inline void fd_divmod(const FastDiv& f, uint32_t n, uint32_t& q, uint32_t& r) {
  q = fd_div(f, n);
  r = n - q * f.divisor;
}
