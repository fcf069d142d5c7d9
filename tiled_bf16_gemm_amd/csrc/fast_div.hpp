// Division of 32-bit unsigned integers by a divisor fixed at launch, as a multiply-high and
// shifts (Granlund and Montgomery, "Division by invariant integers using multiplication", 1994,
// section 4): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d equals
// (t + ((n - t) >> 1)) >> (l - 1) for t = mulhi(n, m) and every n below 2^32; d = 1 is magic 0.
// Host and device code; plain C++ when not compiled by hipcc.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TBG_HD __host__ __device__
#else
#define TBG_HD
#endif

namespace tbg {

struct FastDiv {
  uint32_t magic, shift;
};

TBG_HD inline FastDiv make_fast_div(uint32_t d) {
  if (d <= 1) return FastDiv{0, 0};
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  return FastDiv{(uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1), l - 1};
}

TBG_HD inline uint32_t fast_div(uint32_t n, FastDiv d) {
  if (d.magic == 0) return n;
  const uint32_t t = (uint32_t)(((uint64_t)n * d.magic) >> 32);
  return (t + ((n - t) >> 1)) >> d.shift;
}

}  // namespace tbg
