// Division by a divisor known at launch time, as a multiply and shifts
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the unsigned case with N = 32): for d >= 1 let
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1; then for every
// 32-bit n, t = mulhi(m, n) and floor(n / d) = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0).
// An integer divide on the vector ALU is a long dependent chain; this is five
// instructions.
#pragma once
#include <cstdint>

namespace mla {

struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

#if defined(__HIPCC__)
__host__ __device__
#endif
inline uint32_t fastdiv(uint32_t n, const FastDiv &f) {
  const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

}  // namespace mla
