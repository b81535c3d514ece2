// Host side of the rotation for row lengths that are not powers of two: the choice of
// the Paley factor m for a length n, the square mask of GF(q), and the kernel arguments
// that depend on n only. Pure C++ (no HIP call), shared by the entry points and the host
// emulator of the kernel body.
//
// Rule: n = m * p with p a power of two and m the smallest of 4 o, 8 o, 16 o, ... (o the
// odd part of n; m <= 256 and m dividing n) that has a Paley construction over a prime
// field: Paley I when q = m - 1 is a prime with q = 3 (mod 4), else Paley II when
// q = m / 2 - 1 is a prime with q = 1 (mod 4). A power of two has m = 1.
#pragma once

#include <math.h>
#include <stdint.h>

#include "kron_engine.h"

namespace rbq {

inline bool kron_is_prime(uint32_t v) {
  if (v < 2) return false;
  for (uint32_t d = 2; d * d <= v; ++d)
    if (v % d == 0) return false;
  return true;
}

struct KronFactor {
  uint32_t m;      // 0: no factor; 1: power of two
  uint32_t q;
  uint32_t paley;  // 1 or 2
};

inline KronFactor kron_factor(int64_t n) {
  if (n < 1) return {0, 0, 0};
  if ((n & (n - 1)) == 0) return {1, 0, 0};
  int64_t o = n;
  while ((o & 1) == 0) o >>= 1;
  for (int64_t m = 4 * o; m <= 256 && n % m == 0; m *= 2) {
    const uint32_t mm = (uint32_t)m;
    if (kron_is_prime(mm - 1) && (mm - 1) % 4 == 3) return {mm, mm - 1, 1};
    if (kron_is_prime(mm / 2 - 1) && (mm / 2 - 1) % 4 == 1) return {mm, mm / 2 - 1, 2};
  }
  return {0, 0, 0};
}

// bit d of qr is set iff d = x^2 mod q for some x in [1, q)
inline void kron_square_mask(uint32_t q, uint32_t (&qr)[8]) {
  for (uint32_t& w : qr) w = 0;
  for (uint32_t x = 1; x < q; ++x) {
    const uint32_t d = (x * x) % q;
    qr[d >> 5] |= 1u << (d & 31);
  }
}

// Fills the size-dependent kernel arguments. Returns the LDS words the launch needs, or 0
// when n has no factor or the kernel cannot take it (m > 160, p < 16, p > 2048,
// n > 32768, LDS).
inline uint32_t kron_setup(int64_t n, KronArgs& a) {
  const KronFactor f = kron_factor(n);
  if (f.m < 2 || f.m > kKronMaxM || n > (int64_t)kKronMaxN) return 0;
  const int64_t p = n / f.m;
  if (p < (int64_t)kKronMinP || p > (int64_t)kKronMaxP) return 0;
  uint32_t pl = 0;
  while ((int64_t{1} << pl) < p) ++pl;
  a.m = f.m;
  a.q = f.q;
  a.paley = f.paley;
  a.p_log = pl;
  kron_square_mask(f.q, a.qr);
  a.sqrtn = sqrtf((float)n);
  a.inv_sqrtn = 1.0f / a.sqrtn;
  const uint32_t words = kron_lds_words(f.m, pl, &a.rs, &a.hs, &a.tab0, &a.red0);
  return words <= 40960u ? words : 0u;
}

}  // namespace rbq
