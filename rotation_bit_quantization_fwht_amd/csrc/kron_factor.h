// Host side of the rotation for row lengths that are not powers of two: the choice of
// the Paley factor m for a length n, the square mask of GF(q), and the kernel arguments
// that depend on n only. Pure C++ (no HIP call), shared by the entry points and the host
// emulator of the kernel body.
//
// Rule: n = m * p with p a power of two and m the smallest of 4 o, 8 o, 16 o, ... (o the
// odd part of n; m <= 256 and m dividing n) that has a construction: Paley I when
// q = m - 1 is a prime with q = 3 (mod 4), else Paley II when q = m / 2 - 1 is a prime
// with q = 1 (mod 4), or the Goethals-Seidel matrix of order 172 = 4 * 43 (four circulant
// blocks of order 43, see gs_first_rows). A power of two has m = 1.
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
  uint32_t q;      // the field order (Paley) or the circulant order (Goethals-Seidel)
  uint32_t paley;  // 1 or 2: Paley I / II; 3: Goethals-Seidel
};

// Goethals-Seidel factor of order 172: A, B, C, D circulant +-1 matrices of order 43 with
// A A^T + B B^T + C C^T + D D^T = 172 I (periodic autocorrelations adding up to zero at
// every nonzero shift), in the array
//   [[ A, BR, CR, DR], [-BR, A, D^T R, -C^T R], [-CR, -D^T R, A, B^T R], [-DR, C^T R, -B^T R, A]]
// (R the back-diagonal permutation; Goethals and Seidel, 1967). The first rows are
// constant on the cosets of the order-7 subgroup of (Z/43)^*: the sequence of code v has
// entry +1 at 0 when bit 0 of v is set and +1 on the j-th coset (cosets ordered by their
// smallest element) when bit j is set. The four rows are the lexicographically first
// quadruple of codes i <= j <= k <= l that meets the autocorrelation condition, found by
// exhaustive search once per process.
constexpr uint32_t kGsOrder = 172, kGsP = 43, kGsSub = 7;

struct GsRows {
  uint64_t bits[4];  // bit t of row X: entry t of X's first row is +1
};

inline GsRows gs_first_rows() {
  static const GsRows rows = [] {
    constexpr uint32_t P = kGsP, NCOS = (kGsP - 1) / kGsSub, NCODE = 1u << (NCOS + 1);
    uint32_t g = 2;
    for (;; ++g) {  // smallest primitive root
      uint32_t v = 1, order = 0;
      do { v = v * g % P; ++order; } while (v != 1);
      if (order == P - 1) break;
    }
    uint32_t h = 1;  // generator of the subgroup of order kGsSub: g^((P - 1) / kGsSub)
    for (uint32_t e = 0; e < (P - 1) / kGsSub; ++e) h = h * g % P;
    int coset[P];
    for (uint32_t t = 0; t < P; ++t) coset[t] = -1;
    int ncos = 0;
    for (uint32_t t = 1; t < P; ++t) {
      if (coset[t] >= 0) continue;
      ++ncos;
      uint32_t u = t;
      for (uint32_t e = 0; e < kGsSub; ++e) { coset[u] = ncos; u = u * h % P; }
    }
    static int8_t seq[NCODE][P];
    static int16_t paf[NCODE][P - 1];
    for (uint32_t v = 0; v < NCODE; ++v) {
      seq[v][0] = (v & 1u) ? 1 : -1;
      for (uint32_t t = 1; t < P; ++t) seq[v][t] = ((v >> coset[t]) & 1u) ? 1 : -1;
      for (uint32_t sft = 1; sft < P; ++sft) {
        int acc = 0;
        for (uint32_t t = 0; t < P; ++t) acc += seq[v][t] * seq[v][(t + sft) % P];
        paf[v][sft - 1] = (int16_t)acc;
      }
    }
    GsRows r{{0, 0, 0, 0}};
    for (uint32_t i = 0; i < NCODE; ++i)
      for (uint32_t j = i; j < NCODE; ++j)
        for (uint32_t k = j; k < NCODE; ++k)
          for (uint32_t l = k; l < NCODE; ++l) {
            bool ok = true;
            for (uint32_t sft = 0; sft < P - 1 && ok; ++sft)
              ok = paf[i][sft] + paf[j][sft] + paf[k][sft] + paf[l][sft] == 0;
            if (!ok) continue;
            const uint32_t codes[4] = {i, j, k, l};
            for (int x = 0; x < 4; ++x)
              for (uint32_t t = 0; t < P; ++t)
                if (seq[codes[x]][t] > 0) r.bits[x] |= uint64_t{1} << t;
            return r;
          }
    return r;  // not reached: a quadruple exists
  }();
  return rows;
}

inline KronFactor kron_factor(int64_t n) {
  if (n < 1) return {0, 0, 0};
  if ((n & (n - 1)) == 0) return {1, 0, 0};
  int64_t o = n;
  while ((o & 1) == 0) o >>= 1;
  for (int64_t m = 4 * o; m <= 256 && n % m == 0; m *= 2) {
    const uint32_t mm = (uint32_t)m;
    if (kron_is_prime(mm - 1) && (mm - 1) % 4 == 3) return {mm, mm - 1, 1};
    if (kron_is_prime(mm / 2 - 1) && (mm / 2 - 1) % 4 == 1) return {mm, mm / 2 - 1, 2};
    if (mm == kGsOrder) return {mm, kGsP, 3};
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
// when n has no factor or the kernel cannot take it (m > 256, p < 16, p > 2048,
// n > 32768, more LDS than a workgroup has).
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
  if (f.paley == 3) {
    const GsRows g = gs_first_rows();
    for (int x = 0; x < 4; ++x) {
      a.qr[2 * x] = (uint32_t)g.bits[x];
      a.qr[2 * x + 1] = (uint32_t)(g.bits[x] >> 32);
    }
  } else {
    kron_square_mask(f.q, a.qr);
  }
  a.sqrtn = sqrtf((float)n);
  a.inv_sqrtn = 1.0f / a.sqrtn;
  const uint32_t words = kron_lds_words(f.m, pl, &a.rs, &a.hs, &a.tab0, &a.red0);
  return words <= 40960u ? words : 0u;
}

}  // namespace rbq
