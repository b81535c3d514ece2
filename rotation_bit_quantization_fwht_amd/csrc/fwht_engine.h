// Workgroup body of the fused Walsh-Hadamard rotation + INT4 quantizer.
//
// One workgroup owns 2^r rows of length n = 2^k (see plan.h for the data layouts):
//   load (global -> registers) and the first transform factor: for 16-bit inputs with
//   k >= 7 a pair of 16x16x32 MFMAs multiplies every 32-element group by H_32 (the 32
//   products of 16-bit inputs and +-1 weights are exact; their fp32 sum is rounded like any
//   butterfly sum); otherwise widen to fp32, fusing the
//   first butterfly into the widening of 16-bit pairs with a 2-term dot product
//   -> register butterflies -> LDS transpose -> register butterflies [-> transpose ->
//   butterflies] -> per-row absmax (registers, lane shuffles, LDS across waves)
//   -> scale, round half to even, clamp, nibble packing -> coalesced stores.
//
// Math (restated from the pages): y = H_n x / sqrt(n) with the Sylvester H_n
// ("Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices");
// s = max(max|y| / 7, 1e-8) rounded to the scale dtype; q = RNE(clamp(y / s, -8, 7))
// ("SpinQuant Guide: Learned Rotations for 4-Bit LLMs", step-size equation and
// quantizer listing), or with OPT_INT8 the same equation at b = 8: s = max|y| / 127,
// q in [-128, 127], one code per byte. The 1/sqrt(n) is folded into the per-row multiplier: the kernel
// keeps u = H_n x and uses q = RNE(u * (1 / (s * sqrt(n)))).
//
// The body is written against a small context object (lane/wave ids, LDS, barriers,
// lane shuffles, global loads/stores, the MFMA pair) so the same code runs in the HIP
// kernel and in the host-side emulator used by the CPU tests.
#pragma once

#include "common.h"
#include "plan.h"

namespace rbq {

enum InKind : int { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2 };

enum : uint32_t {
  MODE_QUANT = 1u,  // write codes + scales
  MODE_ROT32 = 2u,  // write the rotated row as float
  MODE_ROT16 = 4u   // write the rotated row in the input's 16-bit format
};
// OPT_INT8: 8-bit codes (scale max/127, grid [-128, 127], one per byte) instead of INT4
enum : uint32_t { OPT_PACKED = 1u, OPT_SCALE_F16 = 2u, OPT_INT8 = 4u };

struct TensorArgs {
  const void* x;
  int64_t row_stride;      // 2-D addressing: elements between consecutive rows
  int64_t sb, sh, ss;      // 4-D addressing: element strides of (batch, head, seq)
  FastDiv div_s, div_h;    // 4-D: row -> (b, h, s)
  uint32_t seq, heads;
  void* codes;             // uint8 [rows, n/2] (packed) or int8 [rows, n]
  void* scales;            // [rows] fp16 or fp32
  float* rot32;            // [rows, n] float
  uint16_t* rot16;         // [rows, n] bf16/fp16 bits
  const void* signs;       // optional [n] +-1 in the input dtype: rows are multiplied by
                           // this diagonal before the transform (randomized Hadamard)
  const float* rope_cos;   // optional fp32 [positions, n/2]: RoPE before the transform,
  const float* rope_sin;   // pairing element i with i + n/2 at position rope_pos0 + s
  uint32_t rope_pos0;
  uint32_t mode;
  int64_t rows;            // rows of this tensor
  uint32_t hs;             // RoPE, matrix plans: 1 = blocks in head-group order (hs_coords)
  uint32_t nsb, nhh;       // head-group order: token blocks per head, head groups per batch
  FastDiv div_nsb, div_nhh;
  uint32_t out_cap;        // 0: codes and scales rows follow the input rows; else the rows
                           // of (batch, head) pair bh go to bh * out_cap + s (a cache of
                           // capacity out_cap per head, its base pointers at the first
                           // position written)
};

struct KArgs {
  TensorArgs t[2];
  uint32_t blocks0;   // row blocks of tensor 0 (blocks past it belong to tensor 1)
  uint32_t nblocks;   // row blocks in total; workgroups loop over them with a stride
  uint32_t opts;
  // cache kernels only: blocks from blocks1 on quantize rows of tv as they are (no
  // rotation), n / 8 lanes per row, into tv's per-head cache (see as_is_rows)
  TensorArgs tv;
  uint32_t blocks1;
};

// one block of rows: its tensor and first row
struct Block {
  const TensorArgs* t;
  int64_t row0;
};

// plan of a kernel instantiation: matrix plans for 16-bit rotated inputs with k >= 7
constexpr bool use_matrix_plan(int k, int in, bool rot) { return rot && in != IN_F32 && k >= 7; }

#define RBQ_PLAN PlanOf<K, MF>::value

// the per-lane register file of one workgroup slot: 2^e values
template <int K, bool MF>
using Regs = float[1 << PlanOf<K, MF>::value.e];

RBQ_HD uint32_t min_u32(uint32_t a, uint32_t b) { return a < b ? a : b; }

constexpr int popcount_c(uint32_t x) { int c = 0; while (x) { c += x & 1u; x >>= 1; } return c; }

// gather the bits of x selected by mask into the low bits
constexpr uint32_t pext_c(uint32_t x, uint32_t mask) {
  uint32_t out = 0; int o = 0;
  for (int b = 0; b < 32; ++b) if ((mask >> b) & 1u) { if ((x >> b) & 1u) out |= 1u << o; ++o; }
  return out;
}
// scatter the low bits of x to the positions selected by mask
constexpr uint32_t pdep_c(uint32_t x, uint32_t mask) {
  uint32_t out = 0; int o = 0;
  for (int b = 0; b < 32; ++b) if ((mask >> b) & 1u) { if ((x >> o) & 1u) out |= 1u << b; ++o; }
  return out;
}

constexpr float sqrt_pow2(int k) {
  float p = (float)(1u << (k / 2));
  return (k & 1) ? 1.41421356237309504880f * p : p;
}

// element-space index contributed by the lane and wave ids in phase PH, with the bits
// of RM squeezed out (every bit's destination is a compile-time constant)
// compressed destination bit of slot bit i (lane bits 0..5, then wave bits 6..)
constexpr int slot_dest(const Plan& p, int ph, int i, uint32_t rm) {
  const int b = i < 6 ? p.lane[ph][i] : p.wave[ph][i - 6];
  int pos = 0;
  while ((compress(1u << b, rm) >> pos) != 1u) ++pos;
  return pos;
}
// length of the run of slot bits starting at i whose destinations are consecutive (0 if
// bit i continues a run started earlier)
constexpr int slot_run(const Plan& p, int ph, int i, uint32_t rm) {
  const int end = i < 6 ? 6 : 6 + p.w;
  if (i != 0 && i != 6 && slot_dest(p, ph, i - 1, rm) + 1 == slot_dest(p, ph, i, rm)) return 0;
  int len = 1;
  while (i + len < end && slot_dest(p, ph, i + len, rm) == slot_dest(p, ph, i, rm) + len) ++len;
  return len;
}

template <int K, bool MF, int PH, uint32_t RM = 0u>
RBQ_HD uint32_t lane_part(uint32_t lane, uint32_t wave) {
  uint32_t idx = 0;
  static_for<0, 6 + RBQ_PLAN.w>([&](auto I) {
    constexpr int len = slot_run(RBQ_PLAN, PH, I.value, RM);
    if constexpr (len > 0) {
      constexpr int dst = slot_dest(RBQ_PLAN, PH, I.value, RM);
      const uint32_t src = (I.value < 6) ? (lane >> I.value) : (wave >> (I.value - 6));
      idx |= (src & ((1u << len) - 1u)) << dst;
    }
  });
  return idx;
}

// the LDS padding of transpose T for a runtime index (shift amounts are constants)
template <int K, bool MF, int T>
RBQ_HD uint32_t lds_pad_rt(uint32_t i) {
  constexpr int PA = RBQ_PLAN.pad[T][0];
  constexpr int PB = RBQ_PLAN.pad[T][1];
  uint32_t r = i;
  if constexpr (PA > 0) r += i >> PA;
  if constexpr (PB > 0) r += i >> PB;
  return r;
}

template <bool FOURD>
RBQ_HD int64_t row_offset(const TensorArgs& t, int64_t row) {
  if constexpr (FOURD) {
    uint32_t r = (uint32_t)row;
    uint32_t bh = fastdiv(r, t.div_s);
    uint32_t s = r - bh * t.seq;
    uint32_t b = fastdiv(bh, t.div_h);
    uint32_t h = bh - b * t.heads;
    return (int64_t)b * t.sb + (int64_t)h * t.sh + (int64_t)s * t.ss;
  } else {
    return row * t.row_stride;
  }
}

// Head-group order (RoPE kernels of the matrix plans, when t.hs is set). Each block of 2^r
// rows covers HG heads x 2^r / HG consecutive tokens of one batch, the blocks running over
// the tokens, then the head groups, then the batch. The rows of one lane's loads (the row
// bits its register index selects) are then HG heads at one token, which share their RoPE
// angles, and each head's rows in the block are consecutive tokens, read as one contiguous
// run. (A block of 64 rows over 32 heads at 2 tokens, 512 bytes per head, read ~1.6x
// slower on the R3 workload; 4 heads x 16 tokens about as fast as the natural order.)
// Without t.hs rows keep their natural (batch, head, token) order.
struct Bhs {
  uint32_t b, h, s;
};

// the row bits of a block that a lane's register index selects in phase 0
template <int K, bool MF>
constexpr uint32_t hs_jbits() {
  return reg_part(RBQ_PLAN, 0, ((1u << RBQ_PLAN.e) - 1u) & ~7u) >> K;
}

// (batch, head, token) of block row r in head-group order
template <int K, bool MF>
RBQ_HD Bhs hs_coords(const TensorArgs& t, uint32_t r) {
  constexpr uint32_t JB = hs_jbits<K, MF>();
  constexpr int RB = RBQ_PLAN.r;
  constexpr int HB = popcount_c(JB);
  const uint32_t blk = r >> RB, rw = r & ((1u << RB) - 1u);
  const uint32_t q = fastdiv(blk, t.div_nsb);  // batch * head groups + head group
  const uint32_t b = fastdiv(q, t.div_nhh);
  uint32_t hl = 0u, sl = 0u;
  static_for<0, RB>([&](auto I) {
    constexpr uint32_t below = (1u << I.value) - 1u;
    const uint32_t bit = (rw >> I.value) & 1u;
    if constexpr ((JB >> I.value) & 1u) hl |= bit << popcount_c(JB & below);
    else sl |= bit << popcount_c(~JB & below);
  });
  return Bhs{b, ((q - b * t.nhh) << HB) | hl, ((blk - q * t.nsb) << (RB - HB)) | sl};
}

// the natural (batch, head, token) tensor row that block row r stands for
template <int K, bool MF, bool RMAP>
RBQ_HD int64_t tensor_row(const TensorArgs& t, int64_t r) {
  if constexpr (RMAP && MF) {
    if (t.hs) {
      const Bhs x = hs_coords<K, MF>(t, (uint32_t)r);
      return ((int64_t)x.b * t.heads + x.h) * t.seq + x.s;
    }
  }
  return r;
}

// element offset of row (b, h, s): 4-D strides, or the natural rows of a 2-D tensor
template <bool FOURD>
RBQ_HD int64_t bhs_offset(const TensorArgs& t, const Bhs& x) {
  if constexpr (FOURD) return (int64_t)x.b * t.sb + (int64_t)x.h * t.sh + (int64_t)x.s * t.ss;
  else return ((int64_t)x.b * t.heads + x.h) * t.seq * t.row_stride + (int64_t)x.s * t.row_stride;
}

// host: head-group order for a RoPE launch at row length 2^k, when the heads and tokens
// divide into whole blocks (so every block is full); else the natural order
template <int K, bool MF>
inline void set_rope_order(TensorArgs& t) {
  t.hs = 0u;
  if constexpr (MF) {
    constexpr uint32_t HG = 1u << popcount_c(hs_jbits<K, MF>());
    constexpr uint32_t SG = (1u << RBQ_PLAN.r) / HG;
    if (t.heads > 0u && t.seq > 0u && t.heads % HG == 0u && t.seq % SG == 0u) {
      t.hs = 1u;
      t.nsb = t.seq / SG;
      t.nhh = t.heads / HG;
      t.div_nsb = make_fastdiv(t.nsb);
      t.div_nhh = make_fastdiv(t.nhh);
    }
  }
}

// host: the order of a RoPE launch at row length 2^k (the matrix plans serve k = 7, 8)
inline void set_rope_order_rt(TensorArgs& t, int k) {
  if (k == 7) set_rope_order<7, true>(t);
  else if (k == 8) set_rope_order<8, true>(t);
  else t.hs = 0u;
}

// output row (codes, scales) of input row r: r itself, or with CACHE and t.out_cap != 0 row
// s of (batch, head) pair bh = r / seq in a cache of t.out_cap rows per pair
template <bool CACHE>
RBQ_HD int64_t out_row(const TensorArgs& t, int64_t r) {
  if constexpr (CACHE) {
    if (t.out_cap != 0u)
      return r + (int64_t)fastdiv((uint32_t)r, t.div_s) * (int64_t)(t.out_cap - t.seq);
  }
  return r;
}

// RoPE on one row held whole in this lane's registers (rows of at most 64 elements): w holds
// the row's 16-bit values two per word, element i in half i % 2 of word i / 2; element i
// pairs with i + n/2. Same arithmetic as apply_rope below: x cos -+ p sin in fp32 as a
// rounded product p sin and a fused multiply-add, rounded back to the 16-bit format.
template <int K, int IN, class Ctx>
RBQ_HD void apply_rope_in_lane(Ctx& c, const TensorArgs& t, uint32_t srow, uint32_t (&w)[1 << (K - 1)]) {
  constexpr uint32_t H = 1u << (K - 1);  // pairs, and the words of one half
  const float* cp = t.rope_cos + (int64_t)(t.rope_pos0 + srow) * H;
  const float* sp = t.rope_sin + (int64_t)(t.rope_pos0 + srow) * H;
  static_for<0, (int)(H / 8)>([&](auto G) {  // eight pairs at a time: four words of each half
    constexpr int g = G.value;
    const f32x4 c0 = c.template load<f32x4>(cp + 8 * g), c1 = c.template load<f32x4>(cp + 8 * g + 4);
    const f32x4 s0 = c.template load<f32x4>(sp + 8 * g), s1 = c.template load<f32x4>(sp + 8 * g + 4);
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    static_for<0, 4>([&](auto D) {
      constexpr int lo = 4 * g + D.value, hi = lo + (int)(H / 2);
      float rl[2], rh[2];
      static_for<0, 2>([&](auto HALF) {
        constexpr int j = 2 * D.value + HALF.value;
        const uint32_t ab = (w[lo] >> (16 * HALF.value)) & 0xFFFFu;
        const uint32_t bb = (w[hi] >> (16 * HALF.value)) & 0xFFFFu;
        const float a = (IN == IN_F16) ? f16_to_f32(ab) : bits_f32(ab << 16);
        const float b = (IN == IN_F16) ? f16_to_f32(bb) : bits_f32(bb << 16);
        // x cos -+ p sin as one product and one fused multiply-add
        rl[HALF.value] = fmaf(a, cs[j], b * -sn[j]);
        rh[HALF.value] = fmaf(b, cs[j], a * sn[j]);
      });
      if constexpr (IN == IN_F16) {
        w[lo] = f32_to_f16(rl[0]) | (f32_to_f16(rl[1]) << 16);
        w[hi] = f32_to_f16(rh[0]) | (f32_to_f16(rh[1]) << 16);
      } else {
        w[lo] = f32x2_to_bf16x2(rl[0], rl[1]);
        w[hi] = f32x2_to_bf16x2(rh[0], rh[1]);
      }
    });
  });
}

// ------------------------------------------------------------------ load (phase 0)

// address of element `el` of row `row0 + rw` (rw < 2^r): a uniform 64-bit block base plus
// a 32-bit lane offset for 2-D tensors (the host checks 2^r * stride * esize < 2^31);
// 4-D tensors decompose each row into (batch, head, token)
template <int K, bool MF, int ESZ, bool FOURD>
RBQ_HD const char* in_addr(const TensorArgs& t, int64_t row0, uint32_t rw, uint32_t el) {
  if constexpr (FOURD) {
    return (const char*)t.x + (row_offset<true>(t, row0 + rw) + (int64_t)el) * ESZ;
  } else {
    const char* base = (const char*)t.x + row0 * t.row_stride * ESZ;
    if constexpr (RBQ_PLAN.r == 0) return base + el * (uint32_t)ESZ;
    else return base + (rw * (uint32_t)t.row_stride + el) * (uint32_t)ESZ;
  }
}

// SIGNS: t.signs is set (see matrix_issue)
template <int K, bool MF, int IN, bool ROT, bool FOURD, bool ROPE, bool SIGNS, class Ctx>
RBQ_HD void load_phase0(Ctx& c, const TensorArgs& t, int64_t rows, int64_t row0,
                        Regs<K, MF>& v) {
  constexpr int C0 = run_log(RBQ_PLAN, 0);
  constexpr int L = 1 << C0;
  constexpr int NRUN = (1 << RBQ_PLAN.e) / L;
  constexpr int ESZ = (IN == IN_F32) ? 4 : 2;
  constexpr int BYTES = L * ESZ;
  const uint32_t lp = lane_part<K, MF, 0>(c.lane, c.wave);
  const uint32_t last = (uint32_t)(rows - 1 - row0);  // last valid row of the block
  static_for<0, NRUN>([&](auto J) {
    constexpr uint32_t rb = (uint32_t)J.value << C0;
    constexpr uint32_t rp = reg_part(RBQ_PLAN, 0, rb);
    const uint32_t idx = lp | rp;
    // rows past the end (last block only) re-read the last row: their results are never
    // stored, and rows do not mix, so no branch is needed
    const uint32_t rw = (RBQ_PLAN.r == 0) ? 0u : min_u32(idx >> K, last);
    const uint32_t el = idx & ((1u << K) - 1u);
    uint32_t w[BYTES / 4];
    {
      const char* src = in_addr<K, MF, ESZ, FOURD>(t, row0, rw, el);
      if constexpr (BYTES >= 16) {
        static_for<0, BYTES / 16>([&](auto Q) {
          u32x4 q4 = c.template load<u32x4>(src + 16 * Q.value);
          w[4 * Q.value + 0] = q4.x; w[4 * Q.value + 1] = q4.y;
          w[4 * Q.value + 2] = q4.z; w[4 * Q.value + 3] = q4.w;
        });
      } else if constexpr (BYTES == 8) {
        u32x2 q2 = c.template load<u32x2>(src);
        w[0] = q2.x; w[1] = q2.y;
      } else {
        w[0] = c.template load<uint32_t>(src);
      }
    }
    if constexpr (SIGNS) {
      // multiply by the +-1 diagonal: flip each value's sign bit where the sign is negative
      constexpr uint32_t SIGN = (IN == IN_F32) ? 0x80000000u : 0x80008000u;
      const char* sp = (const char*)t.signs + el * (uint32_t)ESZ;
      uint32_t sw[BYTES / 4];
      if constexpr (BYTES >= 16) {
        static_for<0, BYTES / 16>([&](auto Q) {
          const u32x4 q4 = c.template load<u32x4>(sp + 16 * Q.value);
          sw[4 * Q.value + 0] = q4.x; sw[4 * Q.value + 1] = q4.y;
          sw[4 * Q.value + 2] = q4.z; sw[4 * Q.value + 3] = q4.w;
        });
      } else if constexpr (BYTES == 8) {
        const u32x2 q2 = c.template load<u32x2>(sp);
        sw[0] = q2.x; sw[1] = q2.y;
      } else {
        sw[0] = c.template load<uint32_t>(sp);
      }
      static_for<0, BYTES / 4>([&](auto I) { w[I.value] ^= sw[I.value] & SIGN; });
    }
    if constexpr (ROPE) {
      static_assert(IN != IN_F32 && C0 == K && NRUN == 1, "RoPE in the load needs a whole 16-bit row per lane");
      const uint32_t row = (uint32_t)(row0 + rw);
      apply_rope_in_lane<K, IN>(c, t, row - fastdiv(row, t.div_s) * t.seq, w);
    }
    if constexpr (IN == IN_F32) {
      static_for<0, L>([&](auto I) { v[rb + I.value] = bits_f32(w[I.value]); });
    } else {
      static_for<0, L / 2>([&](auto I) {
        float a, b;
        if constexpr (ROT) c.template widen_butterfly<IN>(w[I.value], a, b);
        else c.template widen<IN>(w[I.value], a, b);
        v[rb + 2 * I.value] = a;
        v[rb + 2 * I.value + 1] = b;
      });
    }
  });
}

// matrix plans: every load instruction brings 512 consecutive elements per wave, one
// 16-byte vector per lane, which is operand B of the MFMA pair. The loads are issued
// one block ahead (see fwht_quant_persistent), so they are split from the MFMAs.
template <int K, bool MF>
constexpr int kMatrixLoads = (1 << PlanOf<K, MF>::value.e) / 8;

// lane bit of phase 0 that holds element bit K - 1 (the RoPE partner i +- n/2 sits in the
// lane that differs in this bit); -1 if it is not a lane bit
template <int K, bool MF>
constexpr int rope_partner_lane_bit() {
  for (int i = 0; i < 6; ++i)
    if (RBQ_PLAN.lane[0][i] == K - 1) return i;
  return -1;
}

// the RoPE angles of elements el .. el + 7 (mod n/2) at token srow of a row: cos, and sin
// negated below n/2 (x' = x cos - p sin there, x cos + p sin above)
template <int K, class Ctx>
RBQ_HD void rope_tables(Ctx& c, const TensorArgs& t, uint32_t srow, uint32_t el, float (&cs)[8], float (&sn)[8]) {
  constexpr uint32_t H = 1u << (K - 1);
  const float* cp = t.rope_cos + (int64_t)(t.rope_pos0 + srow) * H + (el & (H - 1));
  const float* sp = t.rope_sin + (int64_t)(t.rope_pos0 + srow) * H + (el & (H - 1));
  const f32x4 c0 = c.template load<f32x4>(cp), c1 = c.template load<f32x4>(cp + 4);
  const f32x4 s0 = c.template load<f32x4>(sp), s1 = c.template load<f32x4>(sp + 4);
  cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w; cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
  sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w; sn[4] = s1.x; sn[5] = s1.y; sn[6] = s1.z; sn[7] = s1.w;
  const uint32_t neg = (el & H) ? 0u : 0x80000000u;
  static_for<0, 8>([&](auto I) { sn[I.value] = bits_f32(f32_bits(sn[I.value]) ^ neg); });
}

// RoPE on the 8 16-bit values of one lane (8 consecutive elements of a row, angles cs and sn
// from rope_tables): x' = x cos - p sin below n/2 and x cos + p sin above, p the partner
// i +- n/2, computed in fp32 as a rounded product p sn and a fused multiply-add, and
// rounded back to the 16-bit format.
template <int K, bool MF, int IN, class Ctx>
RBQ_HD void apply_rope(Ctx& c, const float (&cs)[8], const float (&sn)[8], u32x4& q4) {
  constexpr int PB = rope_partner_lane_bit<K, MF>();
  static_assert(PB >= 0, "RoPE needs the half-split partner in another lane");
  uint32_t w[4] = {q4.x, q4.y, q4.z, q4.w};
  uint32_t p[4];
  static_for<0, 4>([&](auto D) {
    p[D.value] = f32_bits(c.template shfl_xor_c<1 << PB>(bits_f32(w[D.value])));
  });
  static_for<0, 4>([&](auto D) {
    float r[2];
    static_for<0, 2>([&](auto HALF) {
      constexpr int j = 2 * D.value + HALF.value;
      const uint32_t xb = (w[D.value] >> (16 * HALF.value)) & 0xFFFFu;
      const uint32_t pb = (p[D.value] >> (16 * HALF.value)) & 0xFFFFu;
      const float x = (IN == IN_F16) ? f16_to_f32(xb) : bits_f32(xb << 16);
      const float pv = (IN == IN_F16) ? f16_to_f32(pb) : bits_f32(pb << 16);
      r[HALF.value] = fmaf(x, cs[j], pv * sn[j]);
    });
    w[D.value] = (IN == IN_F16) ? (f32_to_f16(r[0]) | (f32_to_f16(r[1]) << 16)) : f32x2_to_bf16x2(r[0], r[1]);
  });
  q4 = u32x4{w[0], w[1], w[2], w[3]};
}

// SIGNS: t.signs is set (the randomized transform; only 2-D rows without RoPE take it). It
// is a template parameter so that the sign loads of a block are issued with its other
// loads, with no branch between them: with a runtime branch per load, each flip waits for
// its loads before the next load is issued.
template <int K, bool MF, bool FOURD, int IN, bool ROPE, bool SIGNS, class Ctx>
RBQ_HD void matrix_issue(Ctx& c, const TensorArgs& t, int64_t rows, int64_t row0,
                         uint32_t (&raw)[kMatrixLoads<K, MF>][4]) {
  const uint32_t lp = lane_part<K, MF, 0>(c.lane, c.wave);
  const uint32_t last = (uint32_t)(rows - 1 - row0);  // last valid row of the block
  if constexpr (ROPE) {
    // A lane's loads are one column of several rows (its register index selects the row
    // bits hs_jbits). In head-group order those rows are consecutive heads at one token:
    // one fetch of the angles serves them all, and their addresses are one head stride
    // apart. In the natural order each row has its own token and angles. Every load of the
    // block is issued before RoPE uses any. (No RoPE entry point takes signs.)
    constexpr int NJ = kMatrixLoads<K, MF>;
    const uint32_t el = lp & ((1u << K) - 1u);  // the register index selects rows only
    u32x4 q4[NJ];
    float cs[8], sn[8];
    if (t.hs) {
      // every block is full in this order (the host checks that heads and tokens divide)
      const Bhs x = hs_coords<K, MF>(t, (uint32_t)(row0 + (lp >> K)));
      const int64_t head_step = FOURD ? t.sh : (int64_t)t.seq * t.row_stride;
      const char* src = (const char*)t.x + (bhs_offset<FOURD>(t, x) + (int64_t)el) * 2;
      static_for<0, NJ>([&](auto J) {
        q4[J.value] = c.template load<u32x4>(src + (int64_t)J.value * head_step * 2);
      });
      rope_tables<K>(c, t, x.s, el, cs, sn);
      static_for<0, NJ>([&](auto J) { apply_rope<K, MF, IN>(c, cs, sn, q4[J.value]); });
    } else {
      uint32_t srow[NJ];
      static_for<0, NJ>([&](auto J) {
        constexpr uint32_t rp = reg_part(RBQ_PLAN, 0, (uint32_t)J.value << 3);
        // rows past the end re-read the last row (their results are never stored)
        const uint32_t rw = (RBQ_PLAN.r == 0) ? 0u : min_u32((lp | rp) >> K, last);
        const uint32_t row = (uint32_t)(row0 + rw);
        srow[J.value] = row - fastdiv(row, t.div_s) * t.seq;
        q4[J.value] = c.template load<u32x4>(in_addr<K, MF, 2, FOURD>(t, row0, rw, el));
      });
      static_for<0, NJ>([&](auto J) {
        rope_tables<K>(c, t, srow[J.value], el, cs, sn);
        apply_rope<K, MF, IN>(c, cs, sn, q4[J.value]);
      });
    }
    static_for<0, NJ>([&](auto J) {
      raw[J.value][0] = q4[J.value].x; raw[J.value][1] = q4[J.value].y;
      raw[J.value][2] = q4[J.value].z; raw[J.value][3] = q4[J.value].w;
    });
    return;
  }
  static_for<0, kMatrixLoads<K, MF>>([&](auto J) {
    constexpr uint32_t rp = reg_part(RBQ_PLAN, 0, (uint32_t)J.value << 3);
    const uint32_t idx = lp | rp;
    // rows past the end re-read the last row (their results are never stored)
    const uint32_t rw = (RBQ_PLAN.r == 0) ? 0u : min_u32(idx >> K, last);
    const uint32_t el = idx & ((1u << K) - 1u);
    // randomized Hadamard: flip the 16-bit sign bits where the diagonal is -1. The sign
    // load goes first, so the two variants differ from their first instruction on and no
    // common load is moved above the branch that selects them.
    u32x4 s4{0u, 0u, 0u, 0u};
    if constexpr (SIGNS) s4 = c.template load<u32x4>((const char*)t.signs + el * 2u);
    u32x4 q4 = c.template load<u32x4>(in_addr<K, MF, 2, FOURD>(t, row0, rw, el));
    if constexpr (SIGNS) {
      q4.x ^= s4.x & 0x80008000u; q4.y ^= s4.y & 0x80008000u;
      q4.z ^= s4.z & 0x80008000u; q4.w ^= s4.w & 0x80008000u;
    }
    raw[J.value][0] = q4.x; raw[J.value][1] = q4.y; raw[J.value][2] = q4.z; raw[J.value][3] = q4.w;
  });
}

template <int K, bool MF, int IN, class Ctx>
RBQ_HD void matrix_apply(Ctx& c, const uint32_t (&raw)[kMatrixLoads<K, MF>][4], Regs<K, MF>& v) {
  static_for<0, kMatrixLoads<K, MF>>([&](auto J) {
    constexpr uint32_t rb = (uint32_t)J.value << 3;
    float d0[4], d1[4];
    c.template hadamard32<IN>(raw[J.value], 0, d0);
    c.template hadamard32<IN>(raw[J.value], 1, d1);
    static_for<0, 4>([&](auto R) {
      v[rb + R.value] = d0[R.value];
      v[rb + 4 + R.value] = d1[R.value];
    });
  });
}

// ------------------------------------------------------------------ register butterflies

template <int K, bool MF, int PH, bool SKIP_R0>
RBQ_HD void stages(Regs<K, MF>& v) {
  constexpr uint32_t M = stage_mask(RBQ_PLAN, PH) & (SKIP_R0 ? ~1u : ~0u);
  static_for<0, RBQ_PLAN.e>([&](auto J) {
    if constexpr ((M >> J.value) & 1u) {
      constexpr int S = 1 << J.value;
      static_for<0, (1 << RBQ_PLAN.e)>([&](auto R) {
        if constexpr ((R.value & S) == 0) {
          const float a = v[R.value];
          const float b = v[R.value + S];
          v[R.value] = a + b;
          v[R.value + S] = a - b;
        }
      });
    }
  });
}

// ------------------------------------------------------------------ LDS transpose

template <int K, bool MF, int T, class Ctx>
RBQ_HD void transpose(Ctx& c, Regs<K, MF>& v) {
  constexpr int SR = RBQ_PLAN.sr[T];
  constexpr uint32_t RM = sub_mask(RBQ_PLAN, T);
  constexpr bool WL = transpose_is_wave_local(RBQ_PLAN, T);
  constexpr uint32_t SMASK = (1u << SR) - 1u;
  const uint32_t wbase = lds_pad_rt<K, MF, T>(lane_part<K, MF, T, RM>(c.lane, c.wave));
  const uint32_t rbase = lds_pad_rt<K, MF, T>(lane_part<K, MF, T + 1, RM>(c.lane, c.wave));
  if constexpr (!WL) c.barrier();
  static_for<0, (1 << SR)>([&](auto S) {
    static_for<0, (1 << RBQ_PLAN.e)>([&](auto R) {
      if constexpr ((R.value & SMASK) == (uint32_t)S.value) {
        constexpr uint32_t off = lds_pad(RBQ_PLAN, T, compress(reg_part(RBQ_PLAN, T, R.value), RM));
        c.lds_store(wbase + off, v[R.value]);
      }
    });
    if constexpr (WL) c.wave_sync(); else c.barrier();
    static_for<0, (1 << RBQ_PLAN.e)>([&](auto R) {
      if constexpr ((R.value & SMASK) == (uint32_t)S.value) {
        constexpr uint32_t off = lds_pad(RBQ_PLAN, T, compress(reg_part(RBQ_PLAN, T + 1, R.value), RM));
        v[R.value] = c.lds_load(rbase + off);
      }
    });
    if constexpr (WL) c.wave_sync(); else c.barrier();
  });
}

// ------------------------------------------------------------------ quantize + pack

// Rounding by the float adder: for |t| < 2^22, fma(u, mul, 1.5 * 2^23) equals
// 1.5 * 2^23 + RNE(u * mul) (single rounding of the exact product, half to even), so the
// low mantissa bits hold RNE(u * mul) as a two's complement integer; clamping the float
// to [1.5 * 2^23 - 8, 1.5 * 2^23 + 7] clamps the code to [-8, 7].
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23, bit pattern 0x4B400000

// Round u / d half to even exactly, given mk ~= 1/d (d > 0, or mk == 0 for a zero
// scale). The product u * mk can sit on the other side of a half-integer than the exact
// quotient; the sign of u - b*d at the nearest boundary b, computed exactly by a fused
// multiply-add, settles it. Used where exact ties are frequent: quantizing the input as
// is, and rows of length 4, 16 or 64, whose transform is usually exact in float and
// whose sqrt(n) is a power of two (for odd log2 n the quotient is irrational).
RBQ_HD float round_quotient_exact(float u, float mk, float d) {
  const float t = u * mk;
  const float q0 = rintf(t);
  if (mk == 0.0f) return 0.0f;
  const float dl = t - q0;
  const float b = q0 + (dl >= 0.0f ? 0.5f : -0.5f);
  const float e = fmaf(-b, d, u);  // sign(u/d - b), exact
  const bool odd = (((int)q0) & 1) != 0;
  if (dl >= 0.0f) {
    if (e > 0.0f || (e == 0.0f && odd)) return q0 + 1.0f;
  } else {
    if (e < 0.0f || (e == 0.0f && odd)) return q0 - 1.0f;
  }
  return q0;
}

// FAST: only packed codes and scales are written (no unpacked codes, no rotated rows), so
// the kernel carries no registers for the other outputs
template <int K, bool MF, int PH, bool ROT, int IN, bool FAST, bool CACHE, bool RMAP, class Ctx>
RBQ_HD void finish(Ctx& c, const TensorArgs& t, const KArgs& a, int64_t row0,
                   Regs<K, MF>& v) {
  constexpr int E = 1 << RBQ_PLAN.e;
  constexpr uint32_t RRM = reg_row_mask(RBQ_PLAN, PH);
  constexpr int NRR = popcount_c(RRM);
  constexpr int NC = 1 << NRR;
  constexpr uint32_t LEM = lane_elem_mask(RBQ_PLAN, PH);
  constexpr uint32_t WEM = wave_elem_mask(RBQ_PLAN, PH);
  constexpr int N = 1 << K;
  constexpr float SQRTN = ROT ? sqrt_pow2(K) : 1.0f;
  // INT4: qmax 7, grid [-8, 7]; INT8: qmax 127, grid [-128, 127] (a uniform choice)
  const bool int8 = (a.opts & OPT_INT8) != 0;
  const float qmax = int8 ? 127.0f : 7.0f;
  const float QMAX_SQRTN = qmax * SQRTN;
  constexpr float INV_SQRTN = ROT ? 1.0f / sqrt_pow2(K) : 1.0f;
  // exact rounding decisions where the quotient is exact often enough to tie
  constexpr bool EXACT = !ROT || (K <= 6 && (K % 2) == 0);
  constexpr bool ONE_ROW = RBQ_PLAN.r == 0;  // the grid never runs past the last row

  // ---- per-row absmax of |u|
  float m[NC];
  static_for<0, NC>([&](auto C) { m[C.value] = 0.0f; });
  static_for<0, E>([&](auto R) {
    constexpr int ci = (int)pext_c(R.value, RRM);
    m[ci] = fmaxf(m[ci], fabsf(v[R.value]));
  });
  static_for<0, 6>([&](auto B) {
    if constexpr ((LEM >> B.value) & 1u) {
      static_for<0, NC>([&](auto C) {
        m[C.value] = fmaxf(m[C.value], c.template shfl_xor_c<1 << B.value>(m[C.value]));
      });
    }
  });
  if constexpr (WEM != 0) {
    static_assert(NC == 1, "cross-wave reduction assumes one row per workgroup");
    constexpr uint32_t RED = lds_words(RBQ_PLAN);
    if (c.lane == 0) c.lds_store(RED + c.wave, m[0]);
    c.barrier();
    float mm = 0.0f;
    static_for<0, (1 << RBQ_PLAN.w)>([&](auto W) { mm = fmaxf(mm, c.lds_load(RED + W.value)); });
    m[0] = mm;
  }

  // ---- per-row scale and multiplier
  const uint32_t mode = t.mode;
  const bool scale_f16 = (a.opts & OPT_SCALE_F16) != 0;
  const uint32_t lp = lane_part<K, MF, PH>(c.lane, c.wave);
  const bool leader = ((c.lane & LEM) == 0) && ((c.wave & WEM) == 0);
  float mul[NC];
  float divv[NC];
  int64_t orows[NC];  // output rows (CACHE or RMAP): tensor row, then cache row
  bool any_clamp = false;
  static_for<0, NC>([&](auto C) {
    const float mu = m[C.value];
    float s = mu / QMAX_SQRTN;
    s = fmaxf(s, 1e-8f);
    float s_st;
    uint32_t h16 = 0;
    if (scale_f16) { h16 = f32_to_f16(s); s_st = f16_to_f32(h16); }
    else s_st = s;
    const float mk = (s_st == 0.0f) ? 0.0f : 1.0f / (s_st * SQRTN);
    mul[C.value] = mk;
    divv[C.value] = s_st * SQRTN;
    // subnormal fp16 scales can sit far below max/qmax: then codes need the clamp
    any_clamp = any_clamp || ((mu * mk) > qmax + 0.25f);
    if constexpr (CACHE || RMAP) {
      constexpr uint32_t rp = reg_part(RBQ_PLAN, PH, pdep_c((uint32_t)C.value, RRM));
      const uint32_t rw = ONE_ROW ? 0u : ((lp | rp) >> K);
      orows[C.value] = out_row<CACHE>(t, tensor_row<K, MF, RMAP>(t, row0 + rw));
    }
    if (FAST || (mode & MODE_QUANT)) {
      constexpr uint32_t rp = reg_part(RBQ_PLAN, PH, pdep_c((uint32_t)C.value, RRM));
      const uint32_t rw = ONE_ROW ? 0u : ((lp | rp) >> K);
      if (leader && (ONE_ROW || row0 + rw < t.rows)) {
        const int64_t orow = (CACHE || RMAP) ? orows[C.value] : row0 + rw;
        if (scale_f16) c.template store<uint16_t>((uint16_t*)t.scales + orow, (uint16_t)h16);
        else c.template store<float>((float*)t.scales + orow, s_st);
      }
    }
  });

  // ---- one contiguous run of L elements at a time
  constexpr int CF = run_log(RBQ_PLAN, PH);
  constexpr int L = 1 << CF;
  constexpr int NRUN = E / L;

  auto codes_pass = [&](auto PACKEDC, auto CL) {
    constexpr bool PACKED = decltype(PACKEDC)::value != 0;
    constexpr bool CLAMP = decltype(CL)::value != 0;
    constexpr int FB = PACKED ? 4 : 8;            // bits per code field
    constexpr int PER = PACKED ? 8 : 4;            // codes per dword
    constexpr int G = (L >= PER) ? PER : L;        // codes per output word
    constexpr int NW = (L >= PER) ? L / PER : 1;   // output words per run
    static_for<0, NRUN>([&](auto J) {
      constexpr uint32_t rb = (uint32_t)J.value << CF;
      constexpr uint32_t rp = reg_part(RBQ_PLAN, PH, rb);
      constexpr int ci = (int)pext_c(rb, RRM);
      const uint32_t idx = lp | rp;
      const uint32_t rw = ONE_ROW ? 0u : (idx >> K);
      const uint32_t el = idx & (uint32_t)(N - 1);
      if (!ONE_ROW && row0 + rw >= t.rows) return;
      const float mk = mul[ci];
      uint32_t out[NW];
      static_for<0, NW>([&](auto D) {
        uint32_t acc = 0u;
        static_for<0, G>([&](auto I) {
          const float u = v[rb + G * D.value + I.value];
          float q;
          if constexpr (EXACT) q = round_quotient_exact(u, mk, divv[ci]) + kMagic;
          else q = fmaf(u, mk, kMagic);
          if constexpr (CLAMP) q = fminf(fmaxf(q, kMagic - qmax - 1.0f), kMagic + qmax);
          // insert the low FB bits of the field at the top, shifting earlier ones down
          acc = alignbit(f32_bits(q), acc, FB);
        });
        out[D.value] = (G * FB < 32) ? (acc >> (32 - G * FB)) : acc;
      });
      constexpr int RUN_BYTES = PACKED ? L / 2 : L;
      constexpr uint32_t ROWB = PACKED ? N / 2 : N;
      uint8_t* dst;
      if constexpr (CACHE || RMAP)
        dst = (uint8_t*)t.codes + orows[ci] * (int64_t)ROWB + (PACKED ? el / 2 : el);
      else dst = (uint8_t*)t.codes + row0 * (int64_t)ROWB + (rw * ROWB + (PACKED ? el / 2 : el));
      if constexpr (RUN_BYTES >= 16) {
        static_for<0, RUN_BYTES / 16>([&](auto Q) {
          c.template store<u32x4>(dst + 16 * Q.value, u32x4{out[4 * Q.value], out[4 * Q.value + 1], out[4 * Q.value + 2], out[4 * Q.value + 3]});
        });
      } else if constexpr (RUN_BYTES == 8) {
        c.template store<u32x2>(dst, u32x2{out[0], out[1]});
      } else if constexpr (RUN_BYTES == 4) {
        c.template store<uint32_t>(dst, out[0]);
      } else if constexpr (RUN_BYTES == 2) {
        c.template store<uint16_t>(dst, (uint16_t)out[0]);
      } else {
        c.template store<uint8_t>(dst, (uint8_t)out[0]);
      }
    });
  };

  if constexpr (FAST) {
    if (any_clamp) codes_pass(IC<1>{}, IC<1>{}); else codes_pass(IC<1>{}, IC<0>{});
    return;
  }
  if (mode & MODE_QUANT) {
    const bool packed = (a.opts & OPT_PACKED) != 0;
    if (packed) {
      if (any_clamp) codes_pass(IC<1>{}, IC<1>{}); else codes_pass(IC<1>{}, IC<0>{});
    } else {
      if (any_clamp) codes_pass(IC<0>{}, IC<1>{}); else codes_pass(IC<0>{}, IC<0>{});
    }
  }
  if (mode & MODE_ROT32) {
    static_for<0, NRUN>([&](auto J) {
      constexpr uint32_t rb = (uint32_t)J.value << CF;
      constexpr uint32_t rp = reg_part(RBQ_PLAN, PH, rb);
      const uint32_t idx = lp | rp;
      const uint32_t rw = ONE_ROW ? 0u : (idx >> K);
      const uint32_t el = idx & (uint32_t)(N - 1);
      if (!ONE_ROW && row0 + rw >= t.rows) return;
      float* dst;
      if constexpr (RMAP) dst = t.rot32 + tensor_row<K, MF, RMAP>(t, row0 + rw) * (int64_t)N + el;
      else dst = t.rot32 + row0 * (int64_t)N + (rw * (uint32_t)N + el);
      if constexpr (L >= 4) {
        static_for<0, L / 4>([&](auto Q) {
          constexpr int o = 4 * Q.value;
          c.template store<f32x4>(dst + o, f32x4{v[rb + o] * INV_SQRTN, v[rb + o + 1] * INV_SQRTN, v[rb + o + 2] * INV_SQRTN, v[rb + o + 3] * INV_SQRTN});
        });
      } else {
        static_for<0, L>([&](auto I) { c.template store<float>(dst + I.value, v[rb + I.value] * INV_SQRTN); });
      }
    });
  }
  if (mode & MODE_ROT16) {
    static_for<0, NRUN>([&](auto J) {
      constexpr uint32_t rb = (uint32_t)J.value << CF;
      constexpr uint32_t rp = reg_part(RBQ_PLAN, PH, rb);
      const uint32_t idx = lp | rp;
      const uint32_t rw = ONE_ROW ? 0u : (idx >> K);
      const uint32_t el = idx & (uint32_t)(N - 1);
      if (!ONE_ROW && row0 + rw >= t.rows) return;
      uint16_t* dst;
      if constexpr (RMAP) dst = t.rot16 + tensor_row<K, MF, RMAP>(t, row0 + rw) * (int64_t)N + el;
      else dst = t.rot16 + row0 * (int64_t)N + (rw * (uint32_t)N + el);
      constexpr int NW = (L >= 2) ? L / 2 : 1;
      uint32_t out[NW];
      static_for<0, NW>([&](auto D) {
        const float y0 = v[rb + 2 * D.value] * INV_SQRTN;
        const float y1 = v[rb + 2 * D.value + 1] * INV_SQRTN;
        if constexpr (IN == IN_F16) out[D.value] = f32_to_f16(y0) | (f32_to_f16(y1) << 16);
        else out[D.value] = f32x2_to_bf16x2(y0, y1);
      });
      if constexpr (L >= 8) {
        static_for<0, L / 8>([&](auto Q) {
          c.template store<u32x4>((char*)dst + 16 * Q.value, u32x4{out[4 * Q.value], out[4 * Q.value + 1], out[4 * Q.value + 2], out[4 * Q.value + 3]});
        });
      } else if constexpr (L == 4) {
        c.template store<u32x2>(dst, u32x2{out[0], out[1]});
      } else {
        c.template store<uint32_t>(dst, out[0]);
      }
    });
  }
}

// ------------------------------------------------------------------ the workgroup loop

template <int K, bool MF>
RBQ_HD Block block_of(const KArgs& a, uint32_t blk) {
  const bool second = blk >= a.blocks0;
  Block b;
  b.t = second ? &a.t[1] : &a.t[0];
  b.row0 = (int64_t)(second ? blk - a.blocks0 : blk) << RBQ_PLAN.r;
  return b;
}

// Rows of a 4-D [B, H, S, n] 16-bit tensor quantized as they are (no rotation) into its
// per-head cache: kv_cache_append_int4's values, in the launch that rotates its keys (and
// query). n / 8 lanes take a row, 8 values (one 16-byte load) each; the row's absmax by
// shuffles across them; then the scale and codes of finish() for an unrotated row: max / 7
// floored at 1e-8, stored as fp16 (RNE) or fp32, codes u / scale rounded half to even by
// round_quotient_exact and clamped to [-8, 7] (a no-op unless a subnormal fp16 scale sits
// below max / 7), packed low nibble first. Block vblk covers nthreads / (n / 8) rows.
template <int K, int IN, class Ctx>
RBQ_HD void as_is_rows(Ctx& c, const TensorArgs& t, const KArgs& a, uint32_t vblk, uint32_t nthreads) {
  static_assert(K >= 6 && K <= 8 && IN != IN_F32, "16-bit rows of 64, 128 or 256 values");
  constexpr uint32_t LPR = (1u << K) / 8;  // lanes per row
  const uint32_t tid = c.wave * 64u + c.lane;
  const int64_t row = (int64_t)vblk * (nthreads / LPR) + tid / LPR;
  const uint32_t el = (tid % LPR) * 8u;
  const bool live = row < t.rows;
  const int64_t r = live ? row : t.rows - 1;  // every lane takes part in the shuffles
  const u32x4 q4 = c.template load<u32x4>((const char*)t.x + (row_offset<true>(t, r) + (int64_t)el) * 2);
  const uint32_t w[4] = {q4.x, q4.y, q4.z, q4.w};
  float v[8];
  static_for<0, 4>([&](auto D) { c.template widen<IN>(w[D.value], v[2 * D.value], v[2 * D.value + 1]); });
  float mu = 0.0f;
  static_for<0, 8>([&](auto I) { mu = fmaxf(mu, fabsf(v[I.value])); });
  static_for<0, K - 3>([&](auto B) { mu = fmaxf(mu, c.template shfl_xor_c<1 << B.value>(mu)); });
  const bool scale_f16 = (a.opts & OPT_SCALE_F16) != 0;
  float s = fmaxf(mu / 7.0f, 1e-8f);
  uint32_t h16 = 0;
  if (scale_f16) { h16 = f32_to_f16(s); s = f16_to_f32(h16); }
  const float mk = (s == 0.0f) ? 0.0f : 1.0f / s;
  uint32_t acc = 0u;
  static_for<0, 8>([&](auto I) {
    float q = round_quotient_exact(v[I.value], mk, s) + kMagic;
    q = fminf(fmaxf(q, kMagic - 8.0f), kMagic + 7.0f);
    acc = alignbit(f32_bits(q), acc, 4);
  });
  if (live) {
    const int64_t orow = out_row<true>(t, r);
    c.template store<uint32_t>((uint8_t*)t.codes + orow * (int64_t)(1u << (K - 1)) + el / 2, acc);
    if (tid % LPR == 0) {
      if (scale_f16) c.template store<uint16_t>((uint16_t*)t.scales + orow, (uint16_t)h16);
      else c.template store<float>((float*)t.scales + orow, s);
    }
  }
}

// the transform after phase 0, the reduction, the scale and the stores of one block
template <int K, bool MF, int IN, bool ROT, bool FAST, bool CACHE, bool RMAP, class Ctx>
RBQ_HD void rest_of_block(Ctx& c, const KArgs& a, const Block& b, Regs<K, MF>& v) {
  if constexpr (ROT) {
    if constexpr (RBQ_PLAN.nph >= 2) {
      transpose<K, MF, 0>(c, v);
      stages<K, MF, 1, false>(v);
    }
    if constexpr (RBQ_PLAN.nph >= 3) {
      transpose<K, MF, 1>(c, v);
      stages<K, MF, 2, false>(v);
    }
    finish<K, MF, RBQ_PLAN.nph - 1, true, IN, FAST, CACHE, RMAP>(c, *b.t, a, b.row0, v);
  } else {
    finish<K, MF, 0, false, IN, FAST, CACHE, RMAP>(c, *b.t, a, b.row0, v);
  }
}

#ifndef RBQ_PREFETCH
#define RBQ_PREFETCH 0
#endif

// Workgroup `first` processes blocks first, first + step, ... < a.nblocks (with ROPE in
// head-group order when t.hs is set, see hs_coords). With
// RBQ_PREFETCH and matrix plans the next block's loads are issued as soon as the MFMAs
// have consumed the current block's, so they are in flight while the current block is
// transformed.
template <int K, int IN, bool ROT, bool FOURD, bool FAST, bool ROPE, bool CACHE, class Ctx>
RBQ_HD void fwht_quant_persistent(Ctx& c, const KArgs& a, uint32_t first, uint32_t step) {
  constexpr bool MF = use_matrix_plan(K, IN, ROT);
  const uint32_t nb = a.nblocks;
  static_assert(!(CACHE && RBQ_PREFETCH), "cache launches use the one-block-at-a-time loop");
  constexpr uint32_t NT = 64u << RBQ_PLAN.w;
  if constexpr (MF && !RBQ_PREFETCH) {
    for (uint32_t blk = first; blk < nb; blk += step) {
      c.refresh_ids();
      if constexpr (CACHE) {
        if (blk >= a.blocks1) { as_is_rows<K, IN>(c, a.tv, a, blk - a.blocks1, NT); continue; }
      }
      const Block b = block_of<K, MF>(a, blk);
      uint32_t raw[kMatrixLoads<K, MF>][4];
      Regs<K, MF> v;
      // the branch holds the MFMAs too, so no load is still in flight where the two paths
      // meet (a join with loads in flight makes the first use wait for all of them)
      if (!ROPE && !FOURD && b.t->signs) {
        matrix_issue<K, MF, FOURD, IN, ROPE, true>(c, *b.t, b.t->rows, b.row0, raw);
        matrix_apply<K, MF, IN>(c, raw, v);
      } else {
        matrix_issue<K, MF, FOURD, IN, ROPE, false>(c, *b.t, b.t->rows, b.row0, raw);
        matrix_apply<K, MF, IN>(c, raw, v);
      }
      stages<K, MF, 0, false>(v);
      rest_of_block<K, MF, IN, ROT, FAST, CACHE, ROPE>(c, a, b, v);
    }
  } else if constexpr (MF) {
    uint32_t raw[kMatrixLoads<K, MF>][4];
    if (first < nb) {
      const Block b = block_of<K, MF>(a, first);
      if (!ROPE && !FOURD && b.t->signs) matrix_issue<K, MF, FOURD, IN, ROPE, true>(c, *b.t, b.t->rows, b.row0, raw);
      else matrix_issue<K, MF, FOURD, IN, ROPE, false>(c, *b.t, b.t->rows, b.row0, raw);
    }
    for (uint32_t blk = first; blk < nb; blk += step) {
      c.refresh_ids();
      const Block b = block_of<K, MF>(a, blk);
      Regs<K, MF> v;
      matrix_apply<K, MF, IN>(c, raw, v);
      const uint32_t nxt = blk + step;
      if (nxt < nb) {
        const Block bn = block_of<K, MF>(a, nxt);
        if (!ROPE && !FOURD && bn.t->signs) matrix_issue<K, MF, FOURD, IN, ROPE, true>(c, *bn.t, bn.t->rows, bn.row0, raw);
        else matrix_issue<K, MF, FOURD, IN, ROPE, false>(c, *bn.t, bn.t->rows, bn.row0, raw);
      }
      stages<K, MF, 0, false>(v);
      rest_of_block<K, MF, IN, ROT, FAST, CACHE, ROPE>(c, a, b, v);
    }
  } else {
    for (uint32_t blk = first; blk < nb; blk += step) {
      c.refresh_ids();
      if constexpr (CACHE) {
        if (blk >= a.blocks1) { as_is_rows<K, IN>(c, a.tv, a, blk - a.blocks1, NT); continue; }
      }
      const Block b = block_of<K, MF>(a, blk);
      Regs<K, MF> v;
      if (!ROPE && !FOURD && b.t->signs) load_phase0<K, MF, IN, ROT, FOURD, ROPE, true>(c, *b.t, b.t->rows, b.row0, v);
      else load_phase0<K, MF, IN, ROT, FOURD, ROPE, false>(c, *b.t, b.t->rows, b.row0, v);
      if constexpr (ROT) stages<K, MF, 0, IN != IN_F32>(v);
      rest_of_block<K, MF, IN, ROT, FAST, CACHE, ROPE>(c, a, b, v);
    }
  }
}

#undef RBQ_PLAN

}  // namespace rbq
