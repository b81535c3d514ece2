// Data-layout plans for the fused fast Walsh-Hadamard transform + INT4 quantizer.
//
// The transform on n = 2^k points is a product of k radix-2 butterflies, one per bit of
// the element index (natural Sylvester order: the butterfly on bit b pairs elements i
// and i | 2^b with bit b clear and maps (a, c) to (a + c, a - c)). The butterflies on
// different bits commute, so they can be applied in any order.
//
// A workgroup holds 2^(e + 6 + w) values: 2^e registers per lane, 64 lanes per wave and
// 2^w waves. A "phase" is a bijection between the bits of a value's slot (register,
// lane, wave) and the bits of its "element-space" index, which is the element index
// inside a row (bits 0..k-1) followed by the row index inside the workgroup
// (bits k..k+r-1). In a phase, the butterflies on every element bit held in register
// bits are pure register arithmetic. Between phases the values are exchanged through
// LDS (a "transpose") so that the remaining element bits become register bits.
//
// Phase 0 is the global-load layout: register bits 0..c0-1 are element bits 0..c0-1
// (contiguous runs of 2^c0 elements, c0 >= 3 except for tiny rows), lane bits follow,
// so loads are 16-byte vectors across consecutive lanes. The last phase again has
// register bits 0..2 = element bits 0..2, so 8 codes of one lane pack into one dword.
// A transpose may be split into 2^sr sub-rounds over element bits that are the same
// register bits in both phases; this bounds the LDS footprint.
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
  int8_t reg[kMaxPhases][8];
  int8_t lane[kMaxPhases][6];
  int8_t wave[kMaxPhases][4];
  int sr[kMaxPhases - 1];  // sub-round bits of transpose t (phase t -> t+1)
};

constexpr int8_t EL(int b) { return (int8_t)b; }

constexpr Plan make_plan(int k) {
  Plan p{};
  for (int a = 0; a < kMaxPhases; ++a) {
    for (int i = 0; i < 8; ++i) p.reg[a][i] = -1;
    for (int i = 0; i < 6; ++i) p.lane[a][i] = -1;
    for (int i = 0; i < 4; ++i) p.wave[a][i] = -1;
  }
  p.k = k;
  auto R = [k](int j) { return (int8_t)(k + j); };  // row bit j
  if (k <= 6) {
    // whole rows in registers: 2^(6-k) rows per lane, 64 lanes, 4 waves
    p.e = 6; p.w = 2; p.r = 14 - k; p.nph = 1;
    for (int i = 0; i < k; ++i) p.reg[0][i] = EL(i);
    for (int j = 0; j < 6 - k; ++j) p.reg[0][k + j] = R(j);
    for (int j = 0; j < 6; ++j) p.lane[0][j] = R(6 - k + j);
    p.wave[0][0] = R(12 - k); p.wave[0][1] = R(13 - k);
  } else if (k == 7) {
    // head_dim 128: each lane loads 16 consecutive elements of 4 rows; 8 lanes per row
    p.e = 6; p.w = 2; p.r = 7; p.nph = 2;
    const int8_t r0[6] = {0, 1, 2, 3, R(3), R(4)};
    const int8_t l0[6] = {4, 5, 6, R(0), R(1), R(2)};
    const int8_t r1[6] = {0, 1, 2, 4, 5, 6};
    const int8_t l1[6] = {3, R(0), R(1), R(2), R(3), R(4)};
    for (int i = 0; i < 6; ++i) { p.reg[0][i] = r0[i]; p.lane[0][i] = l0[i]; p.reg[1][i] = r1[i]; p.lane[1][i] = l1[i]; }
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(5); p.wave[a][1] = R(6); }
    p.sr[0] = 2;
  } else if (k == 8) {
    p.e = 6; p.w = 2; p.r = 6; p.nph = 2;
    const int8_t r0[6] = {0, 1, 2, 3, 4, R(3)};
    const int8_t l0[6] = {5, 6, 7, R(0), R(1), R(2)};
    const int8_t r1[6] = {0, 1, 2, 5, 6, 7};
    const int8_t l1[6] = {3, 4, R(0), R(1), R(2), R(3)};
    for (int i = 0; i < 6; ++i) { p.reg[0][i] = r0[i]; p.lane[0][i] = l0[i]; p.reg[1][i] = r1[i]; p.lane[1][i] = l1[i]; }
    for (int a = 0; a < 2; ++a) { p.wave[a][0] = R(4); p.wave[a][1] = R(5); }
    p.sr[0] = 2;
  } else if (k <= 12) {
    // one wave holds 4096 elements = 2^(12-k) rows; 4 independent waves per workgroup
    p.e = 6; p.w = 2; p.r = 14 - k; p.nph = 3;
    const int nrw = 12 - k;
    int i = 0;
    p.reg[0][i++] = 0; p.reg[0][i++] = 1; p.reg[0][i++] = 2;
    for (int b = 9; b < k; ++b) p.reg[0][i++] = EL(b);
    for (int j = 0; j < nrw; ++j) p.reg[0][i++] = R(j);
    for (int j = 0; j < 6; ++j) p.lane[0][j] = EL(3 + j);
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7};
    const int8_t r2[6] = {0, 1, 2, 3, 4, 8};
    for (int j = 0; j < 6; ++j) { p.reg[1][j] = r1[j]; p.reg[2][j] = r2[j]; }
    int l1 = 0, l2 = 0;
    p.lane[1][l1++] = 1; p.lane[1][l1++] = 2; p.lane[1][l1++] = 8;
    p.lane[2][l2++] = 5; p.lane[2][l2++] = 6; p.lane[2][l2++] = 7;
    for (int b = 9; b < k; ++b) { p.lane[1][l1++] = EL(b); p.lane[2][l2++] = EL(b); }
    for (int j = 0; j < nrw; ++j) { p.lane[1][l1++] = R(j); p.lane[2][l2++] = R(j); }
    for (int a = 0; a < 3; ++a) { p.wave[a][0] = R(nrw); p.wave[a][1] = R(nrw + 1); }
    p.sr[0] = 1; p.sr[1] = 1;
  } else if (k == 13) {
    p.e = 6; p.w = 1; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 10, 11, 12}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7}, l1[6] = {1, 2, 8, 10, 11, 12};
    const int8_t r2[6] = {0, 1, 2, 3, 8, 9}, l2[6] = {4, 5, 6, 7, 10, 11};
    for (int i = 0; i < 6; ++i) {
      p.reg[0][i] = r0[i]; p.lane[0][i] = l0[i]; p.reg[1][i] = r1[i];
      p.lane[1][i] = l1[i]; p.reg[2][i] = r2[i]; p.lane[2][i] = l2[i];
    }
    p.wave[0][0] = 9; p.wave[1][0] = 9; p.wave[2][0] = 12;
    p.sr[0] = 1; p.sr[1] = 1;
  } else if (k == 14) {
    p.e = 6; p.w = 2; p.r = 0; p.nph = 3;
    const int8_t r0[6] = {0, 1, 2, 11, 12, 13}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[6] = {0, 3, 4, 5, 6, 7}, l1[6] = {1, 2, 8, 11, 12, 13};
    const int8_t r2[6] = {0, 1, 2, 8, 9, 10}, l2[6] = {3, 4, 5, 6, 7, 11};
    for (int i = 0; i < 6; ++i) {
      p.reg[0][i] = r0[i]; p.lane[0][i] = l0[i]; p.reg[1][i] = r1[i];
      p.lane[1][i] = l1[i]; p.reg[2][i] = r2[i]; p.lane[2][i] = l2[i];
    }
    p.wave[0][0] = 9; p.wave[0][1] = 10; p.wave[1][0] = 9; p.wave[1][1] = 10;
    p.wave[2][0] = 12; p.wave[2][1] = 13;
    p.sr[0] = 1; p.sr[1] = 1;
  } else {  // k == 15
    p.e = 7; p.w = 2; p.r = 0; p.nph = 3;
    const int8_t r0[7] = {0, 1, 2, 11, 12, 13, 14}, l0[6] = {3, 4, 5, 6, 7, 8};
    const int8_t r1[7] = {0, 3, 4, 5, 6, 7, 8}, l1[6] = {1, 2, 11, 12, 13, 14};
    const int8_t r2[7] = {0, 1, 2, 3, 4, 9, 10}, l2[6] = {5, 6, 7, 8, 11, 12};
    for (int i = 0; i < 7; ++i) { p.reg[0][i] = r0[i]; p.reg[1][i] = r1[i]; p.reg[2][i] = r2[i]; }
    for (int i = 0; i < 6; ++i) { p.lane[0][i] = l0[i]; p.lane[1][i] = l1[i]; p.lane[2][i] = l2[i]; }
    p.wave[0][0] = 9; p.wave[0][1] = 10; p.wave[1][0] = 9; p.wave[1][1] = 10;
    p.wave[2][0] = 13; p.wave[2][1] = 14;
    p.sr[0] = 1; p.sr[1] = 1;
  }
  return p;
}

template <int K> struct PlanOf { static constexpr Plan value = make_plan(K); };

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
  uint32_t done = 0;
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

// masks of register / lane / wave positions holding element (not row) bits
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

// LDS word address of a compressed index: one pad word every 32 words plus one every
// 1024 (the map is additive over disjoint bit sets, so register offsets stay
// compile-time immediates).
RBQ_HD constexpr uint32_t lds_pad(uint32_t i) { return i + (i >> 5) + (i >> 10); }

constexpr bool transpose_is_wave_local(const Plan& p, int t) {
  for (int i = 0; i < p.w; ++i)
    if (p.wave[t][i] != p.wave[t + 1][i]) return false;
  return true;
}

constexpr uint32_t lds_words(const Plan& p) {
  uint32_t words = 0;
  for (int t = 0; t + 1 < p.nph; ++t) {
    uint32_t n = 1u << (p.k + p.r - p.sr[t]);
    uint32_t w = lds_pad(n - 1) + 1;
    if (w > words) words = w;
  }
  return words;
}

// structural checks, evaluated at compile time for every plan
constexpr bool plan_ok(const Plan& p) {
  if (p.e + 6 + p.w != p.k + p.r) return false;
  uint32_t covered = 0;
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
  return true;
}

static_assert(plan_ok(make_plan(1)) && plan_ok(make_plan(2)) && plan_ok(make_plan(3)) &&
              plan_ok(make_plan(4)) && plan_ok(make_plan(5)) && plan_ok(make_plan(6)) &&
              plan_ok(make_plan(7)) && plan_ok(make_plan(8)) && plan_ok(make_plan(9)) &&
              plan_ok(make_plan(10)) && plan_ok(make_plan(11)) && plan_ok(make_plan(12)) &&
              plan_ok(make_plan(13)) && plan_ok(make_plan(14)) && plan_ok(make_plan(15)),
              "invalid FWHT layout plan");

}  // namespace rbq
