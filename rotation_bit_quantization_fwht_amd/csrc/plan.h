// Data-layout plans for the fused fast Walsh-Hadamard transform + INT4 quantizer.
//
// The transform on n = 2^k points is a product of k radix-2 butterflies, one per bit of
// the element index (natural Sylvester order: the butterfly on bit b pairs elements i
// and i | 2^b with bit b clear and maps (a, c) to (a + c, a - c)). Butterflies on
// different bits commute, so they can be applied in any order and grouped freely: H_n is
// the Kronecker product of one H_2 per bit, and any subset of bits forms a smaller
// Hadamard factor.
//
// A workgroup holds 2^(e + 6 + w) values: 2^e registers per lane, 64 lanes per wave and
// 2^w waves. A "phase" is a bijection between the bits of a value's slot (register,
// lane, wave) and the bits of its "element-space" index, which is the element index
// inside a row (bits 0..k-1) followed by the row index inside the workgroup
// (bits k..k+r-1). In a phase, the butterflies on every element bit held in register
// bits are register arithmetic. Between phases the values are exchanged through LDS (a
// "transpose") so that the remaining element bits become register bits.
//
// Two plan families:
//  * vector plans (any input dtype): phase 0 is the global-load layout, register bits
//    0..c0-1 = element bits 0..c0-1 (16-byte loads across consecutive lanes);
//  * matrix plans (16-bit inputs, k >= 7): each wave loads 512 consecutive elements per
//    instruction, lane l holding elements 32 (l mod 16) + 8 (l / 16) + [0, 8); one
//    16x16x32 MFMA pair multiplies every 32-element group by the 32-point Hadamard
//    factor (element bits 0..4, exact: the inputs are exact in 16 bits and the weights
//    are +-1), leaving output bits 0..2 in registers and bits 3..4 in lanes 16..63.
// The last phase has register bits 0..2 = element bits 0..2, so 8 codes of one lane
// pack into one dword. A transpose may be split into 2^sr sub-rounds over element bits
// that sit in the same register bits in both phases, which bounds the LDS footprint,
// and uses its own padding (one pad word every 2^a and every 2^b words) chosen so the
// lanes of each LDS instruction fall in distinct banks.
#pragma once

#include "common.h"

namespace rbq {

constexpr int kMaxPhases = 3;

struct Plan {
  int k;    // log2 of the row length
  int e;    // log2 registers per lane
  int w;    // log2 waves per workgroup
  int r;    // log2 rows per workgroup
  int nph;  // number of phases
  bool mfma;          // phase 0 produced by the 32-point matrix-core factor
  uint32_t pre_done;  // element bits already transformed when phase 0 starts
  int8_t reg[kMaxPhases][8];
  int8_t lane[kMaxPhases][6];
  int8_t wave[kMaxPhases][4];
  int sr[kMaxPhases - 1];    // sub-round bits of transpose t (phase t -> t+1)
  int8_t pad[kMaxPhases - 1][2];  // LDS padding shifts of transpose t (0 = none)
};

constexpr Plan blank_plan(int k) {
  Plan p{};
  for (int a = 0; a < kMaxPhases; ++a) {
    for (int i = 0; i < 8; ++i) p.reg[a][i] = -1;
    for (int i = 0; i < 6; ++i) p.lane[a][i] = -1;
    for (int i = 0; i < 4; ++i) p.wave[a][i] = -1;
  }
  for (int t = 0; t + 1 < kMaxPhases; ++t) { p.pad[t][0] = 5; p.pad[t][1] = 10; }
  p.k = k;
  return p;
}

template <int N>
constexpr void set8(int8_t (&dst)[N], const int8_t* src, int n) {
  for (int i = 0; i < n; ++i) dst[i] = src[i];
}

// ----------------------------------------------------------------- vector plans

constexpr Plan make_vector_plan(int k) {
  Plan p = blank_plan(k);
  auto R = [k](int j) { return (int8_t)(k + j); };  // row bit j
  if (k <= 6) {
    // whole rows in registers: 2^(6-k) rows per lane, 64 lanes, 4 waves
    p.e = 6; p.w = 2; p.r = 14 - k; p.nph = 1;
    for (int i = 0; i < k; ++i) p.reg[0][i] = (int8_t)i;
    for (int j = 0; j < 6 - k; ++j) p.reg[0][k + j] = R(j);
    for (int j = 0; j < 6; ++j) p.lane[0][j] = R(6 - k + j);
    p.wave[0][0] = R(12 - k); p.wave[0][1] = R(13 - k);
  } else if (k == 7) {
    // 128 points: each lane loads 16 consecutive elements of 4 rows; 8 lanes per row
    p.e = 6; p.w = 2; p.r = 7; p.nph = 2;
    const int8_t r0[6] = {0, 1, 2, 3, R(3), R(4)};
    const int8_t l0[6] = {4, 5, 6, R(0), R(1), R(2)};
    const int8_t r1[6] = {0, 1, 2, 4, 5, 6};
    const int8_t l1[6] = {3, R(0), R(1), R(2), R(3), R(4)};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6); set8(p.lane[1], l1, 6);
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(5); p.wave[a][1] = R(6); }
    p.sr[0] = 2;
  } else if (k == 8) {
    p.e = 6; p.w = 2; p.r = 6; p.nph = 2;
    const int8_t r0[6] = {0, 1, 2, 3, 4, R(3)};
    const int8_t l0[6] = {5, 6, 7, R(0), R(1), R(2)};
    const int8_t r1[6] = {0, 1, 2, 5, 6, 7};
    const int8_t l1[6] = {3, 4, R(0), R(1), R(2), R(3)};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6); set8(p.lane[1], l1, 6);
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(4); p.wave[a][1] = R(5); }
    p.sr[0] = 2;
  } else if (k <= 12) {
    // one wave holds 4096 elements = 2^(12-k) rows; 4 independent waves per workgroup
    p.e = 6; p.w = 2; p.r = 14 - k; p.nph = 3;
    const int nrw = 12 - k;
    int i = 0;
    p.reg[0][i++] = 0; p.reg[0][i++] = 1; p.reg[0][i++] = 2;
    for (int b = 9; b < k; ++b) p.reg[0][i++] = (int8_t)b;
    for (int j = 0; j < nrw; ++j) p.reg[0][i++] = R(j);
    for (int j = 0; j < 6; ++j) p.lane[0][j] = (int8_t)(3 + j);
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7};
    const int8_t r2[6] = {0, 1, 2, 3, 4, 8};
    set8(p.reg[1], r1, 6); set8(p.reg[2], r2, 6);
    int l1 = 0, l2 = 0;
    p.lane[1][l1++] = 1; p.lane[1][l1++] = 2; p.lane[1][l1++] = 8;
    p.lane[2][l2++] = 5; p.lane[2][l2++] = 6; p.lane[2][l2++] = 7;
    for (int b = 9; b < k; ++b) { p.lane[1][l1++] = (int8_t)b; p.lane[2][l2++] = (int8_t)b; }
    for (int j = 0; j < nrw; ++j) { p.lane[1][l1++] = R(j); p.lane[2][l2++] = R(j); }
    for (int a = 0; a < 3; ++a) { p.wave[a][0] = R(nrw); p.wave[a][1] = R(nrw + 1); }
    p.sr[0] = 1; p.sr[1] = 1;
  } else if (k == 13) {
    p.e = 6; p.w = 1; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 10, 11, 12}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7}, l1[6] = {1, 2, 8, 10, 11, 12};
    const int8_t r2[6] = {0, 1, 2, 3, 8, 9}, l2[6] = {4, 5, 6, 7, 10, 11};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6);
    set8(p.lane[1], l1, 6); set8(p.reg[2], r2, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 9; p.wave[1][0] = 9; p.wave[2][0] = 12;
    p.sr[0] = 1; p.sr[1] = 1;
  } else if (k == 14) {
    p.e = 6; p.w = 2; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 11, 12, 13}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7}, l1[6] = {1, 2, 8, 11, 12, 13};
    const int8_t r2[6] = {0, 1, 2, 8, 9, 10}, l2[6] = {3, 4, 5, 6, 7, 11};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6);
    set8(p.lane[1], l1, 6); set8(p.reg[2], r2, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 9; p.wave[0][1] = 10; p.wave[1][0] = 9; p.wave[1][1] = 10;
    p.wave[2][0] = 12; p.wave[2][1] = 13;
    p.sr[0] = 1; p.sr[1] = 1;
  } else {  // k == 15
    p.e = 7; p.w = 2; p.r = 0; p.nph = 3;
    const int8_t r0[7] = {0, 1, 2, 11, 12, 13, 14}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[7] = {0, 3, 4, 5, 6, 7, 8}, l1[6] = {1, 2, 11, 12, 13, 14};
    const int8_t r2[7] = {0, 1, 2, 3, 4, 9, 10}, l2[6] = {5, 6, 7, 8, 11, 12};
    set8(p.reg[0], r0, 7); set8(p.reg[1], r1, 7); set8(p.reg[2], r2, 7);
    set8(p.lane[0], l0, 6); set8(p.lane[1], l1, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 9; p.wave[0][1] = 10; p.wave[1][0] = 9; p.wave[1][1] = 10;
    p.wave[2][0] = 13; p.wave[2][1] = 14;
    p.sr[0] = 1; p.sr[1] = 1;
  }
  return p;
}

// ----------------------------------------------------------------- matrix plans (k >= 7)

constexpr Plan make_matrix_plan(int k) {
  Plan p = blank_plan(k);
  p.mfma = true;
  p.pre_done = 0x1Fu;  // element bits 0..4 are transformed by the 32-point factor
  auto R = [k](int j) { return (int8_t)(k + j); };
  if (k == 7) {
    // 4 rows per 512-element load block; 16 rows per wave; 64 rows per workgroup. Half the
    // registers of the larger plans (32 values per lane), so twice the waves fit per SIMD:
    // at 128 points a row is too short for one workgroup's arithmetic to hide its loads.
    p.e = 5; p.w = 2; p.r = 6; p.nph = 2;
    const int8_t r0[5] = {0, 1, 2, R(2), R(3)}, l0[6] = {5, 6, R(0), R(1), 3, 4};
    const int8_t r1[5] = {0, 1, 2, 5, 6}, l1[6] = {3, 4, R(0), R(1), R(2), R(3)};
    set8(p.reg[0], r0, 5); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 5); set8(p.lane[1], l1, 6);
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(4); p.wave[a][1] = R(5); }
    p.sr[0] = 2; p.pad[0][0] = 2; p.pad[0][1] = 3;
  } else if (k == 8) {
    p.e = 6; p.w = 2; p.r = 6; p.nph = 2;
    const int8_t r0[6] = {0, 1, 2, R(1), R(2), R(3)}, l0[6] = {5, 6, 7, R(0), 3, 4};
    const int8_t r1[6] = {0, 1, 2, 5, 6, 7}, l1[6] = {3, 4, R(0), R(1), R(3), R(2)};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6); set8(p.lane[1], l1, 6);
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(4); p.wave[a][1] = R(5); }
    p.sr[0] = 2; p.pad[0][0] = 3; p.pad[0][1] = 9;
  } else if (k <= 12) {
    p.e = 6; p.w = 2; p.r = 14 - k; p.nph = 3;
    const int nrw = 12 - k;
    int i = 0;
    p.reg[0][i++] = 0; p.reg[0][i++] = 1; p.reg[0][i++] = 2;
    for (int b = 9; b < k; ++b) p.reg[0][i++] = (int8_t)b;
    for (int j = 0; j < nrw; ++j) p.reg[0][i++] = R(j);
    const int8_t l0[6] = {5, 6, 7, 8, 3, 4};
    const int8_t r1[6] = {0, 1, 5, 6, 7, 8};
    const int8_t r2[6] = {0, 1, 2, 3, 4, 5};
    set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6); set8(p.reg[2], r2, 6);
    int l1 = 0, l2 = 0;
    p.lane[1][l1++] = 2; p.lane[1][l1++] = 3; p.lane[1][l1++] = 4;
    p.lane[2][l2++] = 6; p.lane[2][l2++] = 7; p.lane[2][l2++] = 8;
    for (int b = 9; b < k; ++b) { p.lane[1][l1++] = (int8_t)b; p.lane[2][l2++] = (int8_t)b; }
    for (int j = 0; j < nrw; ++j) { p.lane[1][l1++] = R(j); p.lane[2][l2++] = R(j); }
    for (int a = 0; a < 3; ++a) { p.wave[a][0] = R(nrw); p.wave[a][1] = R(nrw + 1); }
    p.sr[0] = 2; p.sr[1] = 2;
  } else if (k == 13) {
    p.e = 6; p.w = 1; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 9, 10, 11}, l0[6] = {5, 6, 7, 8, 3, 4};
    const int8_t r1[6] = {0, 5, 6, 7, 8, 12}, l1[6] = {1, 2, 3, 10, 11, 4};
    const int8_t r2[6] = {0, 1, 2, 3, 4, 5}, l2[6] = {6, 7, 8, 10, 11, 12};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6);
    set8(p.lane[1], l1, 6); set8(p.reg[2], r2, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 12; p.wave[1][0] = 9; p.wave[2][0] = 9;
    p.sr[0] = 1; p.sr[1] = 1;
    p.pad[0][0] = 6; p.pad[0][1] = 0; p.pad[1][0] = 3; p.pad[1][1] = 6;
  } else if (k == 14) {
    p.e = 6; p.w = 2; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 9, 10, 11}, l0[6] = {5, 6, 7, 8, 3, 4};
    const int8_t r1[6] = {0, 5, 6, 7, 8, 12}, l1[6] = {1, 2, 3, 4, 13, 11};
    const int8_t r2[6] = {0, 1, 2, 3, 4, 13}, l2[6] = {5, 6, 7, 8, 12, 11};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6);
    set8(p.lane[1], l1, 6); set8(p.reg[2], r2, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 12; p.wave[0][1] = 13;
    p.wave[1][0] = 9; p.wave[1][1] = 10; p.wave[2][0] = 9; p.wave[2][1] = 10;
    p.sr[0] = 1; p.sr[1] = 1;
    p.pad[0][0] = 6; p.pad[0][1] = 8; p.pad[1][0] = 5; p.pad[1][1] = 8;
  } else {  // k == 15: 8 waves
    p.e = 6; p.w = 3; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 9, 10, 11}, l0[6] = {5, 6, 7, 8, 3, 4};
    const int8_t r1[6] = {0, 5, 6, 7, 8, 12}, l1[6] = {1, 2, 3, 4, 13, 14};
    const int8_t r2[6] = {0, 1, 2, 3, 13, 14}, l2[6] = {4, 5, 6, 7, 8, 12};
    set8(p.reg[0], r0, 6); set8(p.lane[0], l0, 6); set8(p.reg[1], r1, 6);
    set8(p.lane[1], l1, 6); set8(p.reg[2], r2, 6); set8(p.lane[2], l2, 6);
    p.wave[0][0] = 12; p.wave[0][1] = 13; p.wave[0][2] = 14;
    for (int a = 1; a < 3; ++a) { p.wave[a][0] = 9; p.wave[a][1] = 10; p.wave[a][2] = 11; }
    p.sr[0] = 1; p.sr[1] = 1;
    p.pad[0][0] = 6; p.pad[0][1] = 8; p.pad[1][0] = 5; p.pad[1][1] = 8;
  }
  return p;
}

constexpr Plan make_plan(int k, bool mfma) { return mfma ? make_matrix_plan(k) : make_vector_plan(k); }

template <int K, bool MF = false> struct PlanOf { static constexpr Plan value = make_plan(K, MF); };

// ---------------------------------------------------------------- derived quantities

// element-space index contributed by register index `reg` in phase `ph`
constexpr uint32_t reg_part(const Plan& p, int ph, uint32_t reg) {
  uint32_t idx = 0;
  for (int i = 0; i < p.e; ++i)
    if ((reg >> i) & 1u) idx |= 1u << p.reg[ph][i];
  return idx;
}

// bitmask of register positions whose element bit gets its butterfly in phase ph
constexpr uint32_t stage_mask(const Plan& p, int ph) {
  uint32_t done = p.pre_done;
  for (int a = 0; a < ph; ++a)
    for (int i = 0; i < p.e; ++i)
      if (p.reg[a][i] < p.k) done |= 1u << p.reg[a][i];
  uint32_t m = 0;
  for (int i = 0; i < p.e; ++i) {
    int b = p.reg[ph][i];
    if (b < p.k && !((done >> b) & 1u)) m |= 1u << i;
  }
  return m;
}

constexpr uint32_t reg_row_mask(const Plan& p, int ph) {
  uint32_t m = 0;
  for (int i = 0; i < p.e; ++i) if (p.reg[ph][i] >= p.k) m |= 1u << i;
  return m;
}
constexpr uint32_t lane_elem_mask(const Plan& p, int ph) {
  uint32_t m = 0;
  for (int i = 0; i < 6; ++i) if (p.lane[ph][i] < p.k) m |= 1u << i;
  return m;
}
constexpr uint32_t wave_elem_mask(const Plan& p, int ph) {
  uint32_t m = 0;
  for (int i = 0; i < p.w; ++i) if (p.wave[ph][i] < p.k) m |= 1u << i;
  return m;
}

// number of leading register bits that are element bits 0, 1, 2, ... (run length log2)
constexpr int run_log(const Plan& p, int ph) {
  int c = 0;
  while (c < p.e && p.reg[ph][c] == c && c < p.k) ++c;
  return c;
}

// element-space mask removed by the sub-rounds of transpose t
constexpr uint32_t sub_mask(const Plan& p, int t) {
  uint32_t m = 0;
  for (int i = 0; i < p.sr[t]; ++i) m |= 1u << p.reg[t][i];
  return m;
}

// squeeze out the bits of `remove` from idx (parallel bit extract of ~remove)
constexpr uint32_t compress(uint32_t idx, uint32_t remove) {
  uint32_t out = 0;
  int o = 0;
  for (int b = 0; b < 32; ++b) {
    if ((remove >> b) & 1u) continue;
    if ((idx >> b) & 1u) out |= 1u << o;
    ++o;
  }
  return out;
}

// LDS word address of a compressed index in transpose t: the padding adds one word every
// 2^a and every 2^b words; the map is additive over disjoint bit sets, so register
// offsets stay compile-time immediates.
RBQ_HD constexpr uint32_t lds_pad(const Plan& p, int t, uint32_t i) {
  uint32_t a = (uint32_t)p.pad[t][0], b = (uint32_t)p.pad[t][1];
  return i + (a ? (i >> a) : 0u) + (b ? (i >> b) : 0u);
}

constexpr bool transpose_is_wave_local(const Plan& p, int t) {
  for (int i = 0; i < p.w; ++i)
    if (p.wave[t][i] != p.wave[t + 1][i]) return false;
  return true;
}

constexpr uint32_t lds_words(const Plan& p) {
  uint32_t words = 0;
  for (int t = 0; t + 1 < p.nph; ++t) {
    uint32_t n = 1u << (p.k + p.r - p.sr[t]);
    uint32_t w = lds_pad(p, t, n - 1) + 1;
    if (w > words) words = w;
  }
  return words;
}

// structural checks, evaluated at compile time for every plan
constexpr bool plan_ok(const Plan& p) {
  if (p.e + 6 + p.w != p.k + p.r) return false;
  uint32_t covered = p.pre_done;
  for (int a = 0; a < p.nph; ++a) {
    uint32_t seen = 0;
    for (int i = 0; i < p.e; ++i) { int b = p.reg[a][i]; if (b < 0 || (seen >> b) & 1u) return false; seen |= 1u << b; }
    for (int i = 0; i < 6; ++i) { int b = p.lane[a][i]; if (b < 0 || (seen >> b) & 1u) return false; seen |= 1u << b; }
    for (int i = 0; i < p.w; ++i) { int b = p.wave[a][i]; if (b < 0 || (seen >> b) & 1u) return false; seen |= 1u << b; }
    if (seen != (1u << (p.k + p.r)) - 1u) return false;
    for (int i = 0; i < p.e; ++i) if (p.reg[a][i] < p.k) covered |= 1u << p.reg[a][i];
  }
  if (covered != (1u << p.k) - 1u) return false;
  // the store layout packs 8 consecutive codes per dword (or a whole tiny row)
  int c = run_log(p, p.nph - 1);
  if (c < 3 && c < p.k) return false;
  if (run_log(p, 0) < 3 && run_log(p, 0) < p.k) return false;
  for (int t = 0; t + 1 < p.nph; ++t)
    for (int i = 0; i < p.sr[t]; ++i)
      if (p.reg[t][i] != p.reg[t + 1][i] || p.reg[t][i] >= p.k) return false;
  // rows never spread over waves together with element bits (one reduction level)
  for (int a = 0; a < p.nph; ++a)
    if (wave_elem_mask(p, a) != 0 && p.r != 0) return false;
  if (p.mfma) {
    // matrix load layout: lanes 0..15 index 32-element groups, lanes 16..63 carry
    // element bits 3 and 4, registers 0..2 are element bits 0..2
    if (p.lane[0][4] != 3 || p.lane[0][5] != 4) return false;
    for (int i = 0; i < 3; ++i) if (p.reg[0][i] != i) return false;
    if (p.k < 7) return false;
  }
  return true;
}

constexpr bool all_plans_ok() {
  for (int k = 1; k <= 15; ++k) if (!plan_ok(make_vector_plan(k))) return false;
  for (int k = 7; k <= 15; ++k) if (!plan_ok(make_matrix_plan(k))) return false;
  return true;
}
static_assert(all_plans_ok(), "invalid FWHT layout plan");

// ---------------------------------------------------------------- 32-point factor weights

// Operand A of the 16x16x32 MFMA pair, per lane: lane l holds row i = l mod 16 and the
// 8 weights for k = 8 (l / 16) + v, v = 0..7, of A_m[i][k] = H_32[o][k] with output row
// o = (i mod 4) + 4 m + 8 (i / 4), so that the accumulator of lane l, register j of MFMA
// m holds output element j + 4 m + 8 (l / 16): bits 0..2 in registers, 3..4 in lanes.
// H_32[o][k] = (-1)^popcount(o AND k) (the Sylvester closed form). Entries are +-1 in
// the 16-bit input format, two per dword (v even in the low half).
struct HadamardA {
  uint32_t w[2][2][64][4];  // [format: 0 bf16, 1 fp16][m][lane][dword]
};

constexpr int parity_c(uint32_t x) { int p = 0; while (x) { p ^= (int)(x & 1u); x >>= 1; } return p; }

constexpr HadamardA make_hadamard_a() {
  HadamardA t{};
  const uint32_t pos[2] = {0x3F80u, 0x3C00u}, neg[2] = {0xBF80u, 0xBC00u};
  for (int f = 0; f < 2; ++f)
    for (int m = 0; m < 2; ++m)
      for (int l = 0; l < 64; ++l)
        for (int d = 0; d < 4; ++d) {
          const uint32_t i = (uint32_t)(l % 16);
          const uint32_t o = (i % 4u) + 4u * (uint32_t)m + 8u * (i / 4u);
          uint32_t word = 0;
          for (int h = 0; h < 2; ++h) {
            const uint32_t kk = 8u * (uint32_t)(l / 16) + (uint32_t)(2 * d + h);
            const uint32_t v = parity_c(o & kk) ? neg[f] : pos[f];
            word |= v << (16 * h);
          }
          t.w[f][m][l][d] = word;
        }
  return t;
}

}  // namespace rbq
