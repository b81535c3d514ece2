// Shared helpers for the rbq kernels: portable (host + device) small types, a
// compile-time loop, exact number-format conversions and fast integer division.
//
// Everything here is plain C++ so the kernel bodies can also be executed on the host
// by the layout emulator used in the CPU test-suite; the HIP build marks the
// functions __host__ __device__.
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define RBQ_HD __host__ __device__ __forceinline__
#else
#define RBQ_HD inline
#endif

namespace rbq {

struct alignas(16) u32x4 { uint32_t x, y, z, w; };
struct alignas(8) u32x2 { uint32_t x, y; };
struct alignas(16) f32x4 { float x, y, z, w; };

// Compile-time for loop: calls f(IC<i>{}) for i in [B, E) (a fold over an index pack).
template <int I> struct IC { static constexpr int value = I; };
template <int... I> struct ISeq {};
template <int N, int... I> struct MakeSeq : MakeSeq<N - 1, N - 1, I...> {};
template <int... I> struct MakeSeq<0, I...> { using type = ISeq<I...>; };
template <int B, class F, int... I>
RBQ_HD void static_for_impl(F& f, ISeq<I...>) {
  (f(IC<B + I>{}), ...);
}
template <int B, int E, class F>
RBQ_HD void static_for(F&& f) {
  if constexpr (B < E) static_for_impl<B>(f, typename MakeSeq<E - B>::type{});
}

RBQ_HD uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
RBQ_HD float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

// bfloat16 bits -> float (exact).
RBQ_HD float bf16_to_f32(uint32_t h16) { return bits_f32(h16 << 16); }

// The conversions below round to nearest even (finite inputs); device code uses the
// gfx950 conversion instructions, which do the same, and host code (the emulator) the
// integer forms written out here.

// float -> bfloat16 bits, round to nearest even (finite inputs).
RBQ_HD uint32_t f32_to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
#else
  uint32_t u = f32_bits(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
#endif
}

// two floats -> bfloat16 bits of lo (bits 0..15) and hi (bits 16..31), one
// v_cvt_pk_bf16_f32 on the device
RBQ_HD uint32_t f32x2_to_bf16x2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, b2_t));
#else
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
#endif
}

// binary16 bits -> float (exact, handles subnormals).
RBQ_HD float f16_to_f32(uint32_t h) {
#if defined(__HIP_DEVICE_COMPILE__)
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
#else
  uint32_t sign = (h & 0x8000u) << 16;
  uint32_t exp = (h >> 10) & 0x1Fu;
  uint32_t man = h & 0x3FFu;
  if (exp == 0) {
    // subnormal or zero: man * 2^-24, exact in float
    float v = (float)man * 5.9604644775390625e-08f;
    return bits_f32(f32_bits(v) | sign);
  }
  if (exp == 31) return bits_f32(sign | 0x7F800000u | (man << 13));
  return bits_f32(sign | ((exp + 112u) << 23) | (man << 13));
#endif
}

// float -> binary16 bits, IEEE round to nearest even, including subnormal results and
// overflow to infinity. Written from the binary16/binary32 formats: the result keeps
// 11 significant bits (fewer for subnormals); the discarded bits decide the rounding.
RBQ_HD uint32_t f32_to_f16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (_Float16)f);
#else
  uint32_t u = f32_bits(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return sign | 0x7C00u | (a > 0x7F800000u ? 0x200u : 0u);
  int32_t e = (int32_t)(a >> 23) - 127;  // unbiased exponent
  if (e > 15) return sign | 0x7C00u;     // overflow (rounding may also overflow below)
  uint32_t m = (a & 0x7FFFFFu) | 0x800000u;  // 24-bit significand (a != 0 here unless e<-126)
  if (e < -25) return sign;              // below half the smallest subnormal: +-0
  // number of significand bits to drop: 13 for normals, more for subnormals
  int32_t drop = (e >= -14) ? 13 : 13 + (-14 - e);
  if (a < 0x00800000u) return sign;      // float subnormal: far below fp16 range
  uint32_t keep = m >> drop;
  uint32_t rem = m & ((1u << drop) - 1u);
  uint32_t half = 1u << (drop - 1);
  if (rem > half || (rem == half && (keep & 1u))) keep += 1u;
  if (e >= -14) {
    // normal: keep has 11 bits (1.xxx); a carry to 12 bits bumps the exponent
    uint32_t exp16 = (uint32_t)(e + 15);
    if (keep >> 11) { keep >>= 1; exp16 += 1; }
    if (exp16 >= 31) return sign | 0x7C00u;
    return sign | (exp16 << 10) | (keep & 0x3FFu);
  }
  // subnormal: keep is the 10-bit fraction; a carry into bit 10 yields the smallest normal
  return sign | keep;
#endif
}

// Funnel shift: low 32 bits of ({hi, lo} >> s), 0 <= s < 32 (one v_alignbit_b32).
RBQ_HD uint32_t alignbit(uint32_t hi, uint32_t lo, uint32_t s) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_alignbit(hi, lo, s);
#else
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> s);
#endif
}

// Unsigned division by a runtime constant d >= 1 for numerators n < 2^31, by a
// multiply-high and a shift (round-up reciprocal method): with l = ceil(log2 d) and
// mul = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, mul) + n) >> l.
struct FastDiv {
  uint32_t d, mul, shr;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0, 0};
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.shr = l;
  f.mul = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  return f;
}

RBQ_HD uint32_t mulhi_u32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

RBQ_HD uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)mulhi_u32(n, f.mul) + n) >> f.shr);
}

}  // namespace rbq
