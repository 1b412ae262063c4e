// Division by a divisor fixed at launch, as one multiply-high and a shift (the
// round-up method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): for 1 <= d < 2^31 and 0 <= c < 2^31, with
// sh = ceil(log2 d) and m = ceil(2^(31+sh) / d) (which fits 32 bits),
// c / d = floor(c * m / 2^(31+sh)); d = 1 is taken apart.
// Exact: m*d = 2^(31+sh) + e with 0 <= e < d, so c*m / 2^(31+sh) = c/d + c*e / (d*2^(31+sh))
// and the second term is below 1/d whenever c*d < 2^(31+sh), i.e. for every c < 2^31.
// Host-and-device header with no dependencies (also compiled by the host tests).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SOL_ATTN_HD __host__ __device__
#else
#define SOL_ATTN_HD
#endif

namespace sol_attn {

struct FastDiv {
  uint32_t d = 1, m = 0;
  int s = 0;   // right shift after the multiply-high (sh - 1)

  FastDiv() = default;
  explicit FastDiv(uint32_t divisor) : d(divisor) {
    if (d <= 1) return;
    int sh = 0;
    while ((1ull << sh) < d) ++sh;
    m = (uint32_t)(((1ull << (31 + sh)) + d - 1) / d);
    s = sh - 1;
  }
  SOL_ATTN_HD uint32_t div(uint32_t c) const {
    if (d == 1) return c;
#if defined(__HIP_DEVICE_COMPILE__)
    return __umulhi(c, m) >> s;
#else
    return (uint32_t)(((uint64_t)c * m) >> 32) >> s;
#endif
  }
};

}  // namespace sol_attn
